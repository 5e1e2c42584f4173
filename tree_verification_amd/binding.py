"""ctypes binding of libtreeverify.so: argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks their
shapes/dtypes, passes raw device pointers plus torch's current HIP stream to
the C interface (include/tree_verify.h) and returns the output tensors.  All
computation happens in the library's kernels; there is no fallback path: if
the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtreeverify.so")

TV_F32, TV_BF16 = 0, 1

# per-request status flags (include/tree_verify.h)
REQ_BAD_PARENT = 1
REQ_BAD_NNODES = 2
REQ_BAD_KV = 4
REQ_NONFINITE = 8
REQ_BAD_TOKEN = 16
REQ_BAD_PATH = 32
REQ_TIMEOUT = 64
REQ_TREE_OVERFLOW = 128
REQ_BAD_LEN = 256
REQ_POOL_EXHAUSTED = 512
REQ_BAD_PROB = 1024
REQ_BAD_WORKSPACE = 2048


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_max", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("sm_scale", ctypes.c_float)]


class VerifyDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_max", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("temperature", ctypes.c_float)]


class MergeDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_cand", ctypes.c_int32),
                ("max_len", ctypes.c_int32), ("n_max", ctypes.c_int32)]


class ExpandDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("f_max", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("n_max", ctypes.c_int32), ("k", ctypes.c_int32)]


class BudgetDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_max", ctypes.c_int32)]


class TreeVerifyError(RuntimeError):
    pass


_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_SIGS = {
    "tree_attn_workspace_size": (_SZ, [ctypes.POINTER(AttnDesc)]),
    "tree_attn_forward": (ctypes.c_int, [ctypes.POINTER(AttnDesc)] + [_P] * 10 + [_SZ, _P]),
    "tree_verify_workspace_size": (_SZ, [ctypes.POINTER(VerifyDesc)]),
    "tree_verify_greedy": (ctypes.c_int, [ctypes.POINTER(VerifyDesc)] + [_P] * 9 + [_SZ, _P]),
    "tree_verify_stochastic": (ctypes.c_int, [ctypes.POINTER(VerifyDesc)] + [_P] * 12 + [_SZ, _P]),
    "tree_verify_greedy_noalloc": (ctypes.c_int, [ctypes.POINTER(VerifyDesc)] + [_P] * 9),
    "tree_verify_workspace_init": (ctypes.c_int, [_P, _SZ, _P]),
    "tree_verify_greedy_noalloc_max_scratch": (_SZ, []),
    "kv_compact_accepted": (ctypes.c_int, [ctypes.POINTER(AttnDesc)] + [_P] * 10),
    "tree_verify_stochastic_compact": (ctypes.c_int, [ctypes.POINTER(VerifyDesc), ctypes.POINTER(AttnDesc)]
                                       + [_P] * 19 + [_SZ, _P]),
    "kv_alloc_tree_blocks": (ctypes.c_int, [ctypes.POINTER(AttnDesc)] + [_P] * 9),
    "kv_release_blocks": (ctypes.c_int, [ctypes.POINTER(AttnDesc)] + [_P] * 7),
    "tree_merge_candidates": (ctypes.c_int, [ctypes.POINTER(MergeDesc)] + [_P] * 9),
    "tree_expand_workspace_size": (_SZ, [ctypes.POINTER(ExpandDesc)]),
    "tree_expand_topk": (ctypes.c_int, [ctypes.POINTER(ExpandDesc)] + [_P] * 10 + [_SZ, _P]),
    "tree_expected_accept_length": (ctypes.c_int, [ctypes.POINTER(BudgetDesc)] + [_P] * 7),
    "tree_budget_select": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "tv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

_lib = None
_lock = threading.Lock()


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load (once) and return the C library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise TreeVerifyError(f"{p} is missing: build it with `python -m tree_verification_amd.build`")
        lib = ctypes.CDLL(p)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


def _check(rc: int, name: str):
    if rc != 0:
        msg = load_library().tv_status_string(rc).decode()
        raise TreeVerifyError(f"{name} returned {rc} ({msg})")


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


# Workspaces: each (device, stream, kind, descriptor) gets its own buffer.  The
# verifiers', the attention's and the expansion's are prepared once with
# tree_verify_workspace_init (every call leaves their slots and counters at
# zero again).
_ws: dict = {}


def _desc_key(desc) -> tuple:
    return tuple(getattr(desc, f) for f, _ in desc._fields_)


def workspace(nbytes: int, device: torch.device, kind: str, desc=None) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    key = (device.index, torch.cuda.current_stream(device).cuda_stream, kind,
           None if desc is None else _desc_key(desc))
    buf = _ws.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        if kind in ("stochastic", "greedy", "attn", "expand"):
            init_verify_workspace(buf)
        _ws[key] = buf
    return buf


def init_verify_workspace(buf: torch.Tensor) -> torch.Tensor:
    """Prepare a verifier workspace (uint8 GPU tensor) in place."""
    lib = load_library()
    rc = lib.tree_verify_workspace_init(_ptr(buf), buf.numel(), _stream(buf.device))
    _check(rc, "tree_verify_workspace_init")
    return buf


def attn_desc(q, k_cache, block_table, n_kv_heads=None, sm_scale=None) -> AttnDesc:
    B, n_max, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    d = AttnDesc()
    d.batch, d.n_max, d.n_q_heads, d.n_kv_heads = B, n_max, Hq, Hkv
    d.head_dim, d.block_size = D, bs
    d.max_blocks_per_seq = block_table.shape[1]
    d.num_blocks = nb
    d.dtype = TV_BF16 if q.dtype == torch.bfloat16 else TV_F32
    d.sm_scale = 0.0 if sm_scale is None else float(sm_scale)
    return d


def tree_attn_forward(q, k_cache, v_cache, block_table, prefix_len, n_nodes, parent, *,
                      sm_scale=None, out=None, status=None, ws=None):
    """Tree attention (include/tree_verify.h).  Shapes:
    q [B, n_max, Hq, D]; k_cache and v_cache [num_blocks, Hkv, bs, D];
    block_table [B, max_blocks] int32; prefix_len, n_nodes [B] int32; parent [B, n_max] int32.
    Returns (out [B, n_max, Hq, D], status [B] int32)."""
    lib = load_library()
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("q must be float32 or bfloat16")
    dev = q.device
    B, n_max, Hq, D = q.shape
    _need(q, "q", q.dtype)
    _need(k_cache, "k_cache", q.dtype, device=dev)
    nb, Hkv, bs, _ = k_cache.shape
    _need(v_cache, "v_cache", q.dtype, (nb, Hkv, bs, D), dev)
    if k_cache.shape[3] != D:
        raise ValueError("k_cache head_dim differs from q")
    _need(block_table, "block_table", torch.int32, device=dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    _need(prefix_len, "prefix_len", torch.int32, (B,), dev)
    _need(n_nodes, "n_nodes", torch.int32, (B,), dev)
    _need(parent, "parent", torch.int32, (B, n_max), dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, tuple(q.shape), dev)
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=dev)
    _need(status, "status", torch.int32, (B,), dev)
    desc = attn_desc(q, k_cache, block_table, sm_scale=sm_scale)
    need = lib.tree_attn_workspace_size(ctypes.byref(desc))
    if ws is None:
        ws = workspace(need, dev, "attn", desc)
    nbytes = 0 if ws is None else ws.numel()
    rc = lib.tree_attn_forward(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(block_table), _ptr(prefix_len), _ptr(n_nodes), _ptr(parent),
                               _ptr(out), _ptr(status), _ptr(ws), nbytes, _stream(dev))
    _check(rc, "tree_attn_forward")
    return out, status


def _verify_outputs(B, n_max, dev, path, path_len, out_tokens, status):
    if path is None:
        path = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    if path_len is None:
        path_len = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=dev)
    _need(path, "path", torch.int32, (B, n_max), dev)
    _need(path_len, "path_len", torch.int32, (B,), dev)
    _need(out_tokens, "out_tokens", torch.int32, (B, n_max), dev)
    _need(status, "status", torch.int32, (B,), dev)
    return path, path_len, out_tokens, status


def verify_desc(target_logits, temperature=1.0) -> VerifyDesc:
    B, n_max, V = target_logits.shape
    d = VerifyDesc()
    d.batch, d.n_max, d.vocab, d.temperature = B, n_max, V, float(temperature)
    return d


def tree_verify_greedy(target_logits, tokens, parent, n_nodes, *, path=None, path_len=None,
                       out_tokens=None, status=None, ws=None):
    """Greedy tree verification.  target_logits [B, n_max, V] float32; tokens, parent
    [B, n_max] int32; n_nodes [B] int32.  Returns (path, path_len, out_tokens, status)."""
    lib = load_library()
    dev = target_logits.device
    B, n_max, V = target_logits.shape
    _need(target_logits, "target_logits", torch.float32)
    _need(tokens, "tokens", torch.int32, (B, n_max), dev)
    _need(parent, "parent", torch.int32, (B, n_max), dev)
    _need(n_nodes, "n_nodes", torch.int32, (B,), dev)
    path, path_len, out_tokens, status = _verify_outputs(B, n_max, dev, path, path_len, out_tokens, status)
    desc = verify_desc(target_logits)
    need = lib.tree_verify_workspace_size(ctypes.byref(desc))
    if ws is None:
        ws = workspace(need, dev, "greedy", desc)
    rc = lib.tree_verify_greedy(ctypes.byref(desc), _ptr(target_logits), _ptr(tokens), _ptr(parent),
                                _ptr(n_nodes), _ptr(path), _ptr(path_len), _ptr(out_tokens),
                                _ptr(status), _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev))
    _check(rc, "tree_verify_greedy")
    return path, path_len, out_tokens, status


def tree_verify_greedy_noalloc(target_logits, tokens, parent, n_nodes, *, path=None, path_len=None,
                               out_tokens=None, status=None):
    """tree_verify_greedy without a workspace: the library's static per-device
    scratch (tree_verify_greedy_noalloc_max_scratch() bytes) serves instead.
    Output tensors that are not given are allocated here; pass them in to
    allocate nothing.  Same arguments and results as tree_verify_greedy."""
    lib = load_library()
    dev = target_logits.device
    B, n_max, V = target_logits.shape
    _need(target_logits, "target_logits", torch.float32)
    _need(tokens, "tokens", torch.int32, (B, n_max), dev)
    _need(parent, "parent", torch.int32, (B, n_max), dev)
    _need(n_nodes, "n_nodes", torch.int32, (B,), dev)
    path, path_len, out_tokens, status = _verify_outputs(B, n_max, dev, path, path_len, out_tokens, status)
    desc = verify_desc(target_logits)
    rc = lib.tree_verify_greedy_noalloc(ctypes.byref(desc), _ptr(target_logits), _ptr(tokens), _ptr(parent),
                                        _ptr(n_nodes), _ptr(path), _ptr(path_len), _ptr(out_tokens),
                                        _ptr(status), _stream(dev))
    _check(rc, "tree_verify_greedy_noalloc")
    return path, path_len, out_tokens, status


def tree_verify_stochastic(target_logits, draft_logits, tokens, parent, n_nodes, u_accept, u_sample, *,
                           temperature=1.0, path=None, path_len=None, out_tokens=None, status=None,
                           ws=None):
    """Stochastic tree verification.  target/draft logits [B, n_max, V] float32; tokens,
    parent [B, n_max] int32; n_nodes [B] int32; u_accept, u_sample [B, n_max] float32.
    Returns (path, path_len, out_tokens, status)."""
    lib = load_library()
    dev = target_logits.device
    B, n_max, V = target_logits.shape
    _need(target_logits, "target_logits", torch.float32)
    _need(draft_logits, "draft_logits", torch.float32, (B, n_max, V), dev)
    _need(tokens, "tokens", torch.int32, (B, n_max), dev)
    _need(parent, "parent", torch.int32, (B, n_max), dev)
    _need(n_nodes, "n_nodes", torch.int32, (B,), dev)
    _need(u_accept, "u_accept", torch.float32, (B, n_max), dev)
    _need(u_sample, "u_sample", torch.float32, (B, n_max), dev)
    path, path_len, out_tokens, status = _verify_outputs(B, n_max, dev, path, path_len, out_tokens, status)
    desc = verify_desc(target_logits, temperature)
    need = lib.tree_verify_workspace_size(ctypes.byref(desc))
    if ws is None:
        ws = workspace(need, dev, "stochastic", desc)
    rc = lib.tree_verify_stochastic(ctypes.byref(desc), _ptr(target_logits), _ptr(draft_logits),
                                    _ptr(tokens), _ptr(parent), _ptr(n_nodes), _ptr(u_accept),
                                    _ptr(u_sample), _ptr(path), _ptr(path_len), _ptr(out_tokens),
                                    _ptr(status), _ptr(ws), 0 if ws is None else ws.numel(),
                                    _stream(dev))
    _check(rc, "tree_verify_stochastic")
    return path, path_len, out_tokens, status


def _compact_args(k_cache, v_cache, block_table, prefix_len, B, n_max, src_pos, new_len, status):
    """Checks of the compaction's cache arguments; returns (desc, src_pos, new_len, status)."""
    dev = k_cache.device
    if k_cache.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("caches must be float32 or bfloat16")
    nb, Hkv, bs, D = k_cache.shape
    _need(k_cache, "k_cache", k_cache.dtype)
    _need(v_cache, "v_cache", k_cache.dtype, (nb, Hkv, bs, D), dev)
    _need(block_table, "block_table", torch.int32, device=dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    _need(prefix_len, "prefix_len", torch.int32, (B,), dev)
    if src_pos is None:
        src_pos = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    if new_len is None:
        new_len = torch.empty(B, dtype=torch.int32, device=dev)
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=dev)
    _need(src_pos, "src_pos", torch.int32, (B, n_max), dev)
    _need(new_len, "new_len", torch.int32, (B,), dev)
    _need(status, "status", torch.int32, (B,), dev)
    d = AttnDesc()
    d.batch, d.n_max, d.n_q_heads, d.n_kv_heads = B, n_max, Hkv, Hkv
    d.head_dim, d.block_size = D, bs
    d.max_blocks_per_seq, d.num_blocks = block_table.shape[1], nb
    d.dtype = TV_BF16 if k_cache.dtype == torch.bfloat16 else TV_F32
    d.sm_scale = 0.0
    return d, src_pos, new_len, status


def kv_compact_accepted(k_cache, v_cache, block_table, prefix_len, path, path_len, *, src_pos=None,
                        new_len=None, status=None):
    """In-place accepted-path KV compaction.  Returns (src_pos [B, n_max], new_len [B], status [B])."""
    lib = load_library()
    dev = k_cache.device
    B, n_max = path.shape
    d, src_pos, new_len, status = _compact_args(k_cache, v_cache, block_table, prefix_len, B, n_max, src_pos,
                                                new_len, status)
    _need(path, "path", torch.int32, (B, n_max), dev)
    _need(path_len, "path_len", torch.int32, (B,), dev)
    rc = lib.kv_compact_accepted(ctypes.byref(d), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                 _ptr(prefix_len), _ptr(path), _ptr(path_len), _ptr(src_pos),
                                 _ptr(new_len), _ptr(status), _stream(dev))
    _check(rc, "kv_compact_accepted")
    return src_pos, new_len, status


def tree_verify_stochastic_compact(target_logits, draft_logits, tokens, parent, n_nodes, u_accept, u_sample,
                                   k_cache, v_cache, block_table, prefix_len, *, temperature=1.0, path=None,
                                   path_len=None, out_tokens=None, status=None, src_pos=None, new_len=None,
                                   kv_status=None, ws=None):
    """Stochastic verification and the accepted path's KV compaction in one call (arguments as
    tree_verify_stochastic, then as kv_compact_accepted without the path).
    Returns (path, path_len, out_tokens, status, src_pos, new_len, kv_status)."""
    lib = load_library()
    dev = target_logits.device
    B, n_max, V = target_logits.shape
    _need(target_logits, "target_logits", torch.float32)
    _need(draft_logits, "draft_logits", torch.float32, (B, n_max, V), dev)
    _need(tokens, "tokens", torch.int32, (B, n_max), dev)
    _need(parent, "parent", torch.int32, (B, n_max), dev)
    _need(n_nodes, "n_nodes", torch.int32, (B,), dev)
    _need(u_accept, "u_accept", torch.float32, (B, n_max), dev)
    _need(u_sample, "u_sample", torch.float32, (B, n_max), dev)
    path, path_len, out_tokens, status = _verify_outputs(B, n_max, dev, path, path_len, out_tokens, status)
    kd, src_pos, new_len, kv_status = _compact_args(k_cache, v_cache, block_table, prefix_len, B, n_max, src_pos,
                                                    new_len, kv_status)
    if k_cache.device != dev:
        raise ValueError("caches and logits must be on one device")
    desc = verify_desc(target_logits, temperature)
    need = lib.tree_verify_workspace_size(ctypes.byref(desc))
    if ws is None:
        ws = workspace(need, dev, "stochastic", desc)
    rc = lib.tree_verify_stochastic_compact(ctypes.byref(desc), ctypes.byref(kd), _ptr(target_logits),
                                            _ptr(draft_logits), _ptr(tokens), _ptr(parent), _ptr(n_nodes),
                                            _ptr(u_accept), _ptr(u_sample), _ptr(path), _ptr(path_len),
                                            _ptr(out_tokens), _ptr(status), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(block_table), _ptr(prefix_len), _ptr(src_pos), _ptr(new_len),
                                            _ptr(kv_status), _ptr(ws), 0 if ws is None else ws.numel(),
                                            _stream(dev))
    _check(rc, "tree_verify_stochastic_compact")
    return path, path_len, out_tokens, status, src_pos, new_len, kv_status


def tree_merge_candidates(cand_tokens, cand_len, root_token, n_max, *, tokens=None, parent=None,
                          n_nodes=None, node_of=None, status=None):
    """Merge candidate sequences into one token tree.  cand_tokens [B, M, Lmax] int32,
    cand_len [B, M] int32, root_token [B] int32.  Returns (tokens [B, n_max],
    parent [B, n_max], n_nodes [B], node_of [B, M, Lmax], status [B])."""
    lib = load_library()
    dev = cand_tokens.device
    B, M, L = cand_tokens.shape
    _need(cand_tokens, "cand_tokens", torch.int32)
    _need(cand_len, "cand_len", torch.int32, (B, M), dev)
    _need(root_token, "root_token", torch.int32, (B,), dev)
    out = []
    for t, name, shape in ((tokens, "tokens", (B, n_max)), (parent, "parent", (B, n_max)),
                           (n_nodes, "n_nodes", (B,)), (node_of, "node_of", (B, M, L)),
                           (status, "status", (B,))):
        if t is None:
            t = torch.empty(shape, dtype=torch.int32, device=dev)
        _need(t, name, torch.int32, shape, dev)
        out.append(t)
    d = MergeDesc()
    d.batch, d.n_cand, d.max_len, d.n_max = B, M, L, int(n_max)
    rc = lib.tree_merge_candidates(ctypes.byref(d), _ptr(cand_tokens), _ptr(cand_len), _ptr(root_token),
                                   *[_ptr(t) for t in out], _stream(dev))
    _check(rc, "tree_merge_candidates")
    return tuple(out)


def tree_expand_topk(draft_logits, frontier, n_frontier, tokens, parent, n_nodes, k, *, new_frontier=None,
                     n_new=None, status=None, ws=None):
    """One level of top-k expansion.  draft_logits [B, F, V] float32; frontier [B, F] int32;
    n_frontier [B] int32; tokens, parent [B, n_max] int32 and n_nodes [B] int32 are updated
    in place.  Returns (new_frontier [B, F * k], n_new [B], status [B])."""
    lib = load_library()
    dev = draft_logits.device
    B, F, V = draft_logits.shape
    n_max = tokens.shape[1]
    _need(draft_logits, "draft_logits", torch.float32)
    _need(frontier, "frontier", torch.int32, (B, F), dev)
    _need(n_frontier, "n_frontier", torch.int32, (B,), dev)
    _need(tokens, "tokens", torch.int32, (B, n_max), dev)
    _need(parent, "parent", torch.int32, (B, n_max), dev)
    _need(n_nodes, "n_nodes", torch.int32, (B,), dev)
    if new_frontier is None:
        new_frontier = torch.empty((B, F * int(k)), dtype=torch.int32, device=dev)
    if n_new is None:
        n_new = torch.empty(B, dtype=torch.int32, device=dev)
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=dev)
    _need(new_frontier, "new_frontier", torch.int32, (B, F * int(k)), dev)
    _need(n_new, "n_new", torch.int32, (B,), dev)
    _need(status, "status", torch.int32, (B,), dev)
    d = ExpandDesc()
    d.batch, d.f_max, d.vocab, d.n_max, d.k = B, F, V, n_max, int(k)
    need = lib.tree_expand_workspace_size(ctypes.byref(d))
    if ws is None:
        ws = workspace(need, dev, "expand", d)
    rc = lib.tree_expand_topk(ctypes.byref(d), _ptr(draft_logits), _ptr(frontier), _ptr(n_frontier),
                              _ptr(tokens), _ptr(parent), _ptr(n_nodes), _ptr(new_frontier), _ptr(n_new),
                              _ptr(status), _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev))
    _check(rc, "tree_expand_topk")
    return new_frontier, n_new, status


def _pool_desc(block_table, block_size, num_blocks) -> AttnDesc:
    d = AttnDesc()
    d.batch, d.max_blocks_per_seq = block_table.shape
    d.block_size, d.num_blocks = int(block_size), int(num_blocks)
    d.n_max, d.n_q_heads, d.n_kv_heads, d.head_dim, d.dtype, d.sm_scale = 1, 1, 1, 1, TV_F32, 0.0
    return d


def kv_alloc_tree_blocks(block_table, n_blocks, prefix_len, n_nodes, free_ids, free_count, *, block_size,
                         spec_from=None, status=None):
    """Pop the speculative blocks of every request's tree from the free stack.
    block_table [B, max_blocks], n_blocks [B] and free_count [1] (int32) are updated
    in place.  Returns (spec_from [B], status [B])."""
    lib = load_library()
    dev = block_table.device
    B, _ = block_table.shape
    nb = free_ids.shape[0]
    _need(block_table, "block_table", torch.int32)
    _need(n_blocks, "n_blocks", torch.int32, (B,), dev)
    _need(prefix_len, "prefix_len", torch.int32, (B,), dev)
    _need(n_nodes, "n_nodes", torch.int32, (B,), dev)
    _need(free_ids, "free_ids", torch.int32, (nb,), dev)
    _need(free_count, "free_count", torch.int32, (1,), dev)
    if spec_from is None:
        spec_from = torch.empty(B, dtype=torch.int32, device=dev)
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=dev)
    _need(spec_from, "spec_from", torch.int32, (B,), dev)
    _need(status, "status", torch.int32, (B,), dev)
    d = _pool_desc(block_table, block_size, nb)
    rc = lib.kv_alloc_tree_blocks(ctypes.byref(d), _ptr(block_table), _ptr(n_blocks), _ptr(prefix_len),
                                  _ptr(n_nodes), _ptr(free_ids), _ptr(free_count), _ptr(spec_from),
                                  _ptr(status), _stream(dev))
    _check(rc, "kv_alloc_tree_blocks")
    return spec_from, status


def kv_release_blocks(block_table, n_blocks, new_len, free_ids, free_count, *, block_size, status=None):
    """Push every block past the kept length back onto the free stack.  block_table,
    n_blocks, free_ids and free_count are updated in place.  Returns status [B]."""
    lib = load_library()
    dev = block_table.device
    B, _ = block_table.shape
    nb = free_ids.shape[0]
    _need(block_table, "block_table", torch.int32)
    _need(n_blocks, "n_blocks", torch.int32, (B,), dev)
    _need(new_len, "new_len", torch.int32, (B,), dev)
    _need(free_ids, "free_ids", torch.int32, (nb,), dev)
    _need(free_count, "free_count", torch.int32, (1,), dev)
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=dev)
    _need(status, "status", torch.int32, (B,), dev)
    d = _pool_desc(block_table, block_size, nb)
    rc = lib.kv_release_blocks(ctypes.byref(d), _ptr(block_table), _ptr(n_blocks), _ptr(new_len),
                               _ptr(free_ids), _ptr(free_count), _ptr(status), _stream(dev))
    _check(rc, "kv_release_blocks")
    return status


def tree_expected_accept_length(parent, n_nodes, accept_prob, *, reach=None, expected_len=None, status=None):
    """Expected acceptance length of each tree under the per-node independence
    model.  parent [B, n_max] int32, n_nodes [B] int32, accept_prob [B, n_max]
    float64.  Returns (reach [B, n_max], expected_len [B], status [B])."""
    lib = load_library()
    dev = parent.device
    B, n_max = parent.shape
    _need(parent, "parent", torch.int32)
    _need(n_nodes, "n_nodes", torch.int32, (B,), dev)
    _need(accept_prob, "accept_prob", torch.float64, (B, n_max), dev)
    if reach is None:
        reach = torch.empty(B, n_max, dtype=torch.float64, device=dev)
    if expected_len is None:
        expected_len = torch.empty(B, dtype=torch.float64, device=dev)
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=dev)
    _need(reach, "reach", torch.float64, (B, n_max), dev)
    _need(expected_len, "expected_len", torch.float64, (B,), dev)
    _need(status, "status", torch.int32, (B,), dev)
    d = BudgetDesc()
    d.batch, d.n_max = B, n_max
    rc = lib.tree_expected_accept_length(ctypes.byref(d), _ptr(parent), _ptr(n_nodes), _ptr(accept_prob),
                                         _ptr(reach), _ptr(expected_len), _ptr(status), _stream(dev))
    _check(rc, "tree_expected_accept_length")
    return reach, expected_len, status


def tree_budget_select(al, itl):
    """Best shape per batch size by goodput al[s] / itl[i][s] (host arrays:
    al of length S, itl of I rows of S latencies).  Returns a list of I shape
    indices (-1 where no latency is positive and finite)."""
    lib = load_library()
    al = [float(x) for x in al]
    rows = [[float(x) for x in r] for r in itl]
    S, I = len(al), len(rows)
    if any(len(r) != S for r in rows):
        raise ValueError("every latency row needs one entry per shape")
    al_c = (ctypes.c_double * max(S, 1))(*al)
    itl_c = (ctypes.c_double * max(S * I, 1))(*[x for r in rows for x in r])
    best = (ctypes.c_int32 * max(I, 1))()
    rc = lib.tree_budget_select(I, S, ctypes.cast(al_c, _P), ctypes.cast(itl_c, _P), ctypes.cast(best, _P))
    _check(rc, "tree_budget_select")
    return [int(best[i]) for i in range(I)]
