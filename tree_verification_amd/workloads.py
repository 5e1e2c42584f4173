"""Seeded synthetic inputs for the token-tree attention + verification path.

This module only draws random data and lays it out; it computes none of the
method's arithmetic (no softmax, no attention, no acceptance test).  Both the
HIP path and the CPU oracle consume the same arrays produced here.

Layouts (all arrays are NumPy, C-contiguous):

  q            [B][Nmax][Hq][D]            float32 holding bf16-exact values when dtype == "bf16"
  k_cache      [num_blocks][Hkv][bs][D]    token-major key blocks
  v_cache      [num_blocks][Hkv][bs][D]    token-major value blocks
  block_table  [B][max_blocks]  int32     -1 past the blocks a request owns
  prefix_len   [B] int32, n_nodes [B] int32
  parent       [B][Nmax] int32            parent[b][0] = -1, 0 <= parent[i] < i, -1 as padding
  tokens       [B][Nmax] int32            token of each tree node (the root's is the last emitted token)
  target_logits, draft_logits [B][Nmax][V] float32 (zero rows past n_nodes)
  u_accept, u_sample          [B][Nmax]    float32 uniforms in [0, 1)

Trees are drawn by random attachment (each new node picks a uniformly random
eligible parent, subject to optional width/depth caps), then renumbered to
depth-first preorder as the SpecInfer guide lays nodes out ("Depth-First
Flattening and KV Cache Reuse").  A child's token is an independent draw from
the draft distribution of its parent (Gumbel-max on the parent's draft-logit
row), so the i.i.d.-proposal precondition of rejection sampling holds.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# Named workloads.  Sizes follow the five synthetic configurations this path is
# measured on: a tiny fp32 case, a Llama-3-8B-shaped layer, a ragged paged
# batch, a batch of chains (linear speculative decoding) and a 70B-shaped share.
CONFIGS = {
    "tiny": dict(batch=1, n_q_heads=1, n_kv_heads=1, head_dim=64, dtype="f32",
                 prefix=(128, 128), n_nodes=8, tree="capped", width=3, depth=3,
                 vocab=1000, target_sd=2.0, draft_noise_sd=0.5, block_size=16, paged=False),
    "llama8b": dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
                    prefix=(2048, 2048), n_nodes=64, tree="capped", width=4, depth=8,
                    vocab=128256, target_sd=3.0, draft_noise_sd=1.0, block_size=16, paged=False),
    "ragged": dict(batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
                   prefix=(512, 8192), n_nodes=32, tree="recursive", width=None, depth=None,
                   vocab=128256, target_sd=3.0, draft_noise_sd=1.0, block_size=16, paged=True),
    "chain": dict(batch=64, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
                  prefix=(4096, 4096), n_nodes=(3, 8), tree="chain", width=1, depth=None,
                  vocab=128256, target_sd=3.0, draft_noise_sd=1.0, block_size=16, paged=False),
    "llama70b_share": dict(batch=4, n_q_heads=64, n_kv_heads=8, head_dim=128, dtype="bf16",
                           prefix=(32768, 32768), n_nodes=128, tree="capped", width=8, depth=10,
                           vocab=128256, target_sd=3.0, draft_noise_sd=1.0, block_size=16, paged=False),
}

CONFIG_ORDER = ["tiny", "llama8b", "ragged", "chain", "llama70b_share"]


def seed_for(name: str, extra: int = 0) -> int:
    """Seed = 1000 + position of the config in CONFIG_ORDER (+100 per extra parity seed)."""
    return 1000 + CONFIG_ORDER.index(name) + 100 * extra


# --------------------------------------------------------------------------
# bf16 helpers (data preparation only)
# --------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bit patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# trees
# --------------------------------------------------------------------------

def dfs_renumber(parent: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Renumber a tree (parent[i] < i) to depth-first preorder.

    Children are visited in creation (ascending index) order.  Returns
    (new_parent, order) where order[new_id] = old_id.
    """
    n = len(parent)
    kids = [[] for _ in range(n)]
    for i in range(1, n):
        kids[parent[i]].append(i)
    order = []
    stack = [0]
    while stack:
        u = stack.pop()
        order.append(u)
        stack.extend(reversed(kids[u]))
    new_id = np.empty(n, dtype=np.int64)
    new_id[np.asarray(order)] = np.arange(n)
    new_parent = np.full(n, -1, dtype=np.int32)
    for old in range(1, n):
        new_parent[new_id[old]] = new_id[parent[old]]
    return new_parent, np.asarray(order)


def random_tree(rng: np.random.Generator, n: int, kind: str, width=None, depth=None) -> np.ndarray:
    """Parent array of an n-node tree in DFS preorder.

    kind = "capped": random attachment to a node with depth < depth cap and
    fewer than `width` children; "recursive": uniform random recursive tree
    (no caps); "chain": parent[i] = i - 1; "star": every node hangs off the root.
    """
    if kind == "chain":
        p = np.arange(-1, n - 1, dtype=np.int32)
        return p
    if kind == "star":
        p = np.zeros(n, dtype=np.int32)
        p[0] = -1
        return p
    parent = np.full(n, -1, dtype=np.int32)
    dep = np.zeros(n, dtype=np.int64)
    nkid = np.zeros(n, dtype=np.int64)
    for i in range(1, n):
        if kind == "recursive":
            cand = np.arange(i)
        elif kind == "capped":
            ok = np.ones(i, dtype=bool)
            if depth is not None:
                ok &= dep[:i] < depth
            if width is not None:
                ok &= nkid[:i] < width
            cand = np.nonzero(ok)[0]
            if len(cand) == 0:
                raise ValueError("tree caps leave no eligible parent")
        else:
            raise ValueError(kind)
        pu = int(cand[rng.integers(len(cand))])
        parent[i] = pu
        dep[i] = dep[pu] + 1
        nkid[pu] += 1
    new_parent, _ = dfs_renumber(parent)
    return new_parent


def gumbel_max_draw(rng: np.random.Generator, logits_row: np.ndarray, count: int) -> np.ndarray:
    """`count` i.i.d. draws from the distribution whose logits are `logits_row`
    (Gumbel-max: argmax of logits plus standard Gumbel noise)."""
    out = np.empty(count, dtype=np.int32)
    z = logits_row.astype(np.float64)
    for k in range(count):
        g = -np.log(-np.log(rng.random(z.shape[0]) + 1e-300) + 1e-300)
        out[k] = int(np.argmax(z + g))
    return out


# --------------------------------------------------------------------------
# workload container
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                 # "bf16" or "f32"
    batch: int
    n_max: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    vocab: int
    num_blocks: int
    max_blocks: int
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_table: np.ndarray
    prefix_len: np.ndarray
    n_nodes: np.ndarray
    parent: np.ndarray
    tokens: np.ndarray
    target_logits: np.ndarray | None
    draft_logits: np.ndarray | None
    u_accept: np.ndarray
    u_sample: np.ndarray
    temperature: float = 1.0
    seed: int = 0

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def make_workload(name: str, seed: int | None = None, *, batch=None, prefix=None, n_nodes=None,
                  vocab=None, tree=None, width="cfg", depth="cfg", n_max=None, paged=None,
                  with_logits=True, kv_fill="normal", logits_dtype=np.float32) -> Workload:
    """Build one seeded workload.  Keyword overrides shrink or reshape a named
    config (parity tests use smaller prefixes / vocabularies of the same kind)."""
    cfg = dict(CONFIGS[name])
    if seed is None:
        seed = seed_for(name)
    rng = np.random.default_rng(seed)
    B = cfg["batch"] if batch is None else batch
    Hq, Hkv, D = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    bs = cfg["block_size"]
    V = cfg["vocab"] if vocab is None else vocab
    pre = cfg["prefix"] if prefix is None else prefix
    if isinstance(pre, int):
        pre = (pre, pre)
    nn = cfg["n_nodes"] if n_nodes is None else n_nodes
    kind = cfg["tree"] if tree is None else tree
    w = cfg["width"] if width == "cfg" else width
    d = cfg["depth"] if depth == "cfg" else depth
    is_paged = cfg["paged"] if paged is None else paged

    # request shapes
    P = rng.integers(pre[0], pre[1] + 1, size=B).astype(np.int32)
    if isinstance(nn, tuple):
        N = rng.integers(nn[0], nn[1] + 1, size=B).astype(np.int32)
    else:
        N = np.full(B, nn, dtype=np.int32)
    Nmax = int(N.max()) if B > 0 else 1
    if n_max is not None:
        Nmax = max(Nmax, n_max)

    parent = np.full((B, Nmax), -1, dtype=np.int32)
    for b in range(B):
        parent[b, :N[b]] = random_tree(rng, int(N[b]), kind, w, d)

    # paged KV pool: each request owns ceil((P + N) / bs) blocks
    need = [(int(P[b]) + int(N[b]) + bs - 1) // bs for b in range(B)]
    num_blocks = max(1, sum(need))
    max_blocks = max([1] + need)
    pool = np.arange(num_blocks, dtype=np.int32)
    if is_paged:
        pool = rng.permutation(pool).astype(np.int32)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :need[b]] = pool[off:off + need[b]]
        off += need[b]

    dt = cfg["dtype"]

    def draw(shape):
        if kv_fill == "normal":
            x = rng.standard_normal(size=shape, dtype=np.float32)
        else:
            raise ValueError(kv_fill)
        return round_to_bf16(x) if dt == "bf16" else x

    q = draw((B, Nmax, Hq, D))
    k_cache = draw((num_blocks, Hkv, bs, D))
    v_cache = draw((num_blocks, Hkv, bs, D))

    tokens = np.zeros((B, Nmax), dtype=np.int32)
    tl = dl = None
    if with_logits:
        tl = np.zeros((B, Nmax, V), dtype=logits_dtype)
        dl = np.zeros((B, Nmax, V), dtype=logits_dtype)
        for b in range(B):
            n = int(N[b])
            t = rng.standard_normal(size=(n, V), dtype=np.float32) * np.float32(cfg["target_sd"])
            e = rng.standard_normal(size=(n, V), dtype=np.float32) * np.float32(cfg["draft_noise_sd"])
            tl[b, :n] = t
            dl[b, :n] = t + e
    for b in range(B):
        n = int(N[b])
        tokens[b, 0] = rng.integers(V)
        for c in range(1, n):
            if dl is not None:
                tokens[b, c] = gumbel_max_draw(rng, dl[b, parent[b, c]], 1)[0]
            else:
                tokens[b, c] = rng.integers(V)
    u_accept = rng.random(size=(B, Nmax), dtype=np.float32)
    u_sample = rng.random(size=(B, Nmax), dtype=np.float32)

    return Workload(name=name, dtype=dt, batch=B, n_max=Nmax, n_q_heads=Hq, n_kv_heads=Hkv,
                    head_dim=D, block_size=bs, vocab=V, num_blocks=num_blocks, max_blocks=max_blocks,
                    q=q, k_cache=k_cache, v_cache=v_cache, block_table=table, prefix_len=P,
                    n_nodes=N, parent=parent, tokens=tokens, target_logits=tl, draft_logits=dl,
                    u_accept=u_accept, u_sample=u_sample, seed=seed)


def dominate_tree_keys(wl: Workload, seed: int, strength: float = 16.0, noise: float = 0.25) -> Workload:
    """Rewrite the queries and the tree positions' keys so that the tree keys a
    row may see dominate its softmax (a mask-sensitive attention input).

    Per (request, KV head) a random unit direction e is drawn; every key at the
    request's tree positions [P, P + n) and every query of the KV head's
    q-heads become strength * e + noise * N(0, 1) (bf16-rounded for bf16
    workloads).  Tree scores then sit near strength^2 / sqrt(D) while prefix
    scores stay O(strength / sqrt(D)) wide, so each row's output is a weighted
    mean of the values at its visible tree positions, and adding or dropping
    one of them moves the row by a sizeable fraction of its norm.  In place;
    returns wl.
    """
    rng = np.random.default_rng(seed)
    D, Hkv = wl.head_dim, wl.n_kv_heads
    G = wl.n_q_heads // Hkv
    bs = wl.block_size
    rnd = round_to_bf16 if wl.dtype == "bf16" else (lambda x: np.asarray(x, dtype=np.float32))
    for b in range(wl.batch):
        P, n = int(wl.prefix_len[b]), int(wl.n_nodes[b])
        for g in range(Hkv):
            e = rng.standard_normal(D)
            e /= np.linalg.norm(e)
            keys = strength * e[None, :] + noise * rng.standard_normal((n, D))
            for i in range(n):
                pos = P + i
                blk = int(wl.block_table[b, pos // bs])
                wl.k_cache[blk, g, pos % bs, :] = rnd(keys[i].astype(np.float32))
            qs = strength * e[None, None, :] + noise * rng.standard_normal((wl.n_max, G, D))
            wl.q[b, :, g * G:(g + 1) * G, :] = rnd(qs.astype(np.float32))
    return wl


# ---------------------------------------------------------------------------
# token-tree construction inputs
# ---------------------------------------------------------------------------

def make_candidates(batch: int, n_cand: int, max_len: int, vocab: int, seed: int, share: float = 0.7,
                    min_len: int = 0):
    """Candidate continuations for a merge, as several draft models would propose them.

    Returns (cand_tokens [B][M][Lmax] int32, zero past each length; cand_len [B][M]
    int32; root_token [B] int32).  Lengths are uniform in [min_len, max_len].  With
    probability `share` a candidate copies a random earlier candidate of its
    request up to a random cut and continues from there (draft models agreeing on a
    prefix); otherwise it starts fresh.  Tokens are uniform in [0, vocab).
    """
    rng = np.random.default_rng(seed)
    toks = np.zeros((batch, n_cand, max_len), dtype=np.int32)
    lens = np.zeros((batch, n_cand), dtype=np.int32)
    for b in range(batch):
        for i in range(n_cand):
            L = int(rng.integers(min_len, max_len + 1))
            seq = []
            if i > 0 and rng.random() < share:
                src = int(rng.integers(i))
                cut = int(rng.integers(0, lens[b, src] + 1))
                seq = list(toks[b, src, :cut])
            while len(seq) < L:
                seq.append(int(rng.integers(vocab)))
            seq = seq[:L]
            toks[b, i, :L] = seq
            lens[b, i] = L
    root = rng.integers(0, vocab, size=batch).astype(np.int32)
    return toks, lens, root


def make_expand_rows(batch: int, f_max: int, vocab: int, seed: int, sd: float = 3.0, ties: bool = False):
    """Draft logit rows of one expansion level, [B][F][V] float32 ~ N(0, sd) (the spread
    of the configurations' target rows).  ties=True rounds them to multiples of 0.5 so
    that equal logits occur and the tie order is exercised."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((batch, f_max, vocab)) * sd).astype(np.float32)
    if ties:
        x = (np.round(x * 2.0) / 2.0).astype(np.float32)
    return x


def schedule_tree(schedule) -> np.ndarray:
    """Parent array of the tree an expansion schedule <k_1, ..., k_m> builds below
    the root: every node of level i - 1 gets k_i children, appended level by level
    (frontier order, then rank).  Shape only; no tokens."""
    parent = [-1]
    frontier = [0]
    for k in schedule:
        nxt = []
        for f in frontier:
            for _ in range(int(k)):
                nxt.append(len(parent))
                parent.append(f)
        frontier = nxt
    return np.asarray(parent, dtype=np.int32)


def make_budget_trees(batch: int, n_max: int, seed: int):
    """Trees and per-node acceptance probabilities for the expected-length
    calculation: [B][n_max] int32 parents (padding -1), [B] int32 node counts,
    [B][n_max] float64 probabilities (root and padding entries 0).  Node counts
    are uniform in 1..n_max with every fifth request full; shapes cycle through
    capped, recursive, chain and star trees; probabilities are U(0, 1) with
    about one in eight set to exactly 0 or 1."""
    rng = np.random.default_rng(seed)
    parent = np.full((batch, n_max), -1, dtype=np.int32)
    n_nodes = np.empty(batch, dtype=np.int32)
    prob = np.zeros((batch, n_max), dtype=np.float64)
    kinds = ("capped", "recursive", "chain", "star")
    for b in range(batch):
        n = n_max if b % 5 == 0 else int(rng.integers(1, n_max + 1))
        kind = kinds[b % 4]
        if kind == "capped":
            par = random_tree(rng, n, "capped", width=int(rng.integers(2, 9)), depth=None)
        else:
            par = random_tree(rng, n, kind)
        parent[b, :n] = par
        n_nodes[b] = n
        a = rng.random(n)
        pick = rng.random(n)
        a[pick < 1 / 16] = 0.0
        a[(pick >= 1 / 16) & (pick < 1 / 8)] = 1.0
        a[0] = 0.0
        prob[b, :n] = a
    return parent, n_nodes, prob
