// Token-tree construction for gfx950 ([guide] "Token Tree Construction:
// Expansion vs. Merge").
//
// Merge (Method B), tree_merge_kernel: one workgroup per request.  The
// candidates sit in LDS; for every pair of candidates the length of their
// common token prefix (lcp) is computed once.  Position j of candidate i is a
// new node exactly when no earlier candidate shares its first j + 1 tokens;
// otherwise it belongs to the node of the first candidate that does (its
// creator).  Depth-first preorder ranks follow from pairwise comparisons of
// the new nodes: two nodes either lie on one root path (the shallower first)
// or diverge below a common prefix of length d, where the two subtrees are
// ordered by the creators of their depth-d prefixes (siblings in
// first-candidate order).
//
// Expansion (Method A), one level, as one launch: topk_kernel's grid holds one
// workgroup per (frontier row, 8192-logit chunk), which finds the chunk's k
// best 64-bit keys (value order, then lower index) by k rounds of a workgroup
// maximum, each removing the winner from the thread that holds it, and then
// one workgroup per request.  Workgroups are dispatched in id order, so a
// request's workgroup takes a slot only after every chunk workgroup has one;
// one wave per frontier row polls (bounded) until the row's key slots are
// written, merges them the same way, and clears them for the next call, and
// the request's children are appended after its last node.  A key slot is a
// 64-bit word written with one agent-scope store and never 0 once written
// (reserved small values mark "no element left" and "non-finite logit"), so a
// slot carries its own "written" mark and no ordering between addresses is
// needed.

#include "tv_common.h"

#include <math.h>

namespace {

constexpr int kMergeThreads = 256;
constexpr int kMaxCand = 64;
constexpr int kMaxCandLen = 32;
constexpr int kMaxTreeNodes = 1024;

constexpr int kTopkThreads = 256;
constexpr int kTopkChunk = kTopkThreads * 32;   // 8192 logits per workgroup
constexpr int kMaxK = 16;
constexpr long long kAppendSpinLimit = 1LL << 21;   // a request workgroup's bounded wait (~2 s)

// ===========================================================================
// merge
// ===========================================================================

struct MergeParams {
  const int32_t* cand_tokens;   // [B][M][L]
  const int32_t* cand_len;      // [B][M]
  const int32_t* root_token;    // [B]
  int32_t* tokens;              // [B][n_max]
  int32_t* parent;              // [B][n_max]
  int32_t* n_nodes;             // [B]
  int32_t* node_of;             // [B][M][L] or null
  int32_t* status;              // [B]
  int M, L, n_max;
};

struct MergeSmem {
  int tok[kMaxCand][kMaxCandLen];
  int len[kMaxCand];
  uint8_t lcp[kMaxCand][kMaxCand];
  uint8_t creator[kMaxCand][kMaxCandLen];
  uint16_t nodes[kMaxCand * kMaxCandLen];     // new nodes as (i << 5) | j, any order
  int16_t rank[kMaxCand][kMaxCandLen];        // node id of each new node (i, j)
  int wcount[kMergeThreads / 64];
  int count, bad;
};

// Does new node y = (i2, j2) come before new node x = (i, j) in depth-first
// preorder?  d = common prefix length of candidates i and i2.
__device__ __forceinline__ bool precedes(const MergeSmem& sm, int i2, int j2, int i, int j) {
  const int d = sm.lcp[i][i2];
  if (j < d && j2 < d) return j2 < j;    // both on the shared prefix: the shallower first
  if (j2 < d) return true;               // y is a prefix of x: an ancestor
  if (j < d) return false;               // x is an ancestor of y
  return sm.creator[i2][d] < sm.creator[i][d];   // diverging below the shared prefix
}

__global__ __launch_bounds__(kMergeThreads) void tree_merge_kernel(MergeParams p) {
  __shared__ MergeSmem sm;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, b = blockIdx.x;
  const int M = p.M, L = p.L;
  if (t == 0) sm.bad = 0;
  __syncthreads();
  if (t < M) {
    const int len = p.cand_len[(size_t)b * M + t];
    sm.len[t] = (len >= 0 && len <= L) ? len : 0;
    if (len < 0 || len > L) sm.bad = 1;
  }
  __syncthreads();
  for (int q = t; q < M * L; q += kMergeThreads) {
    const int i = q / L, j = q % L;
    sm.tok[i][j] = j < sm.len[i] ? p.cand_tokens[(size_t)b * M * L + q] : 0;
  }
  __syncthreads();
  if (sm.bad) {
    if (t == 0) {
      p.status[b] = TV_REQ_BAD_LEN;
      p.n_nodes[b] = 0;
    }
    return;
  }
  // common prefix lengths of every pair (the diagonal is the length itself)
  for (int q = t; q < M * M; q += kMergeThreads) {
    const int i = q / M, i2 = q % M;
    if (i2 > i) continue;
    const int lim = min(sm.len[i], sm.len[i2]);
    int d = 0;
    while (d < lim && sm.tok[i][d] == sm.tok[i2][d]) ++d;
    sm.lcp[i][i2] = (uint8_t)d;
    sm.lcp[i2][i] = (uint8_t)d;
  }
  __syncthreads();
  // creator: the first candidate holding the same first j + 1 tokens
  for (int q = t; q < M * L; q += kMergeThreads) {
    const int i = q / L, j = q % L;
    if (j >= sm.len[i]) continue;
    int c = 0;
    while (sm.lcp[i][c] < j + 1) ++c;   // stops at c = i at the latest
    sm.creator[i][j] = (uint8_t)c;
  }
  __syncthreads();
  // compact the new nodes (ballot prefix counts per pass of 256 positions)
  int base = 0;
  for (int q0 = 0; q0 < M * L; q0 += kMergeThreads) {
    const int q = q0 + t;
    bool isnew = false;
    int i = 0, j = 0;
    if (q < M * L) {
      i = q / L;
      j = q % L;
      isnew = j < sm.len[i] && sm.creator[i][j] == i;
    }
    const unsigned long long bal = __ballot(isnew);
    if (l == 0) sm.wcount[w] = __popcll(bal);
    __syncthreads();
    int off = base;
    for (int k = 0; k < w; ++k) off += sm.wcount[k];
    if (isnew) sm.nodes[off + __popcll(bal & ((1ull << l) - 1ull))] = (uint16_t)((i << 5) | j);
    for (int k = 0; k < kMergeThreads / 64; ++k) base += sm.wcount[k];
    __syncthreads();
  }
  const int count = base;
  if (1 + count > p.n_max) {
    if (t == 0) {
      p.status[b] = TV_REQ_TREE_OVERFLOW;
      p.n_nodes[b] = 0;
    }
    return;
  }
  // depth-first preorder ranks: 1 + the number of new nodes before each one
  for (int x = t; x < count; x += kMergeThreads) {
    const int i = sm.nodes[x] >> 5, j = sm.nodes[x] & 31;
    int r = 1;
    for (int y = 0; y < count; ++y) r += precedes(sm, sm.nodes[y] >> 5, sm.nodes[y] & 31, i, j) ? 1 : 0;
    sm.rank[i][j] = (int16_t)r;
  }
  __syncthreads();
  int32_t* tokens = p.tokens + (size_t)b * p.n_max;
  int32_t* parent = p.parent + (size_t)b * p.n_max;
  for (int q = t; q < M * L; q += kMergeThreads) {
    const int i = q / L, j = q % L;
    int id = -1;
    if (j < sm.len[i]) {
      const int c = sm.creator[i][j];
      id = sm.rank[c][j];
      if (c == i) {
        tokens[id] = sm.tok[i][j];
        parent[id] = j == 0 ? 0 : sm.rank[sm.creator[i][j - 1]][j - 1];
      }
    }
    if (p.node_of) p.node_of[(size_t)b * M * L + q] = id;
  }
  if (t == 0) {
    tokens[0] = p.root_token[b];
    parent[0] = -1;
    p.n_nodes[b] = 1 + count;
    p.status[b] = 0;
  }
}

// ===========================================================================
// expansion
// ===========================================================================

struct ExpandParams {
  const float* logits;        // [B][F][V]
  const int32_t* frontier;    // [B][F]
  const int32_t* n_frontier;  // [B]
  int32_t* tokens;            // [B][n_max]
  int32_t* parent;            // [B][n_max]
  int32_t* n_nodes;           // [B]
  int32_t* new_frontier;      // [B][F * k]
  int32_t* n_new;             // [B]
  int32_t* status;            // [B]
  unsigned long long* header; // workspace [2]: kWsMagic, bytes zero-filled by tree_verify_workspace_init
  unsigned long long need;    // bytes this call's layout uses (header included)
  unsigned long long* keys;   // workspace [B][F][chunks][k], zero between calls
  int B, F, V, n_max, k, chunks;
  int G;                      // chunk workgroups; the B workgroups after them append the children
  long long spin;             // polling rounds before a request workgroup gives up (negative: at once)
};

// Order-preserving key: larger value first, then lower index.  For a finite
// or infinite value and an index below 2^31 it exceeds 2^32, so the values
// below are free: 0 is an unwritten slot, kKeyNone a chunk with no element
// left, kKeyBad a chunk holding a NaN or an infinity.  -0 and +0 tie.
__device__ __forceinline__ unsigned long long topk_key(float v, int idx) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;
  const uint32_t hi = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)hi << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}

constexpr unsigned long long kKeyNone = 1ull;
constexpr unsigned long long kKeyBad = 2ull;

__device__ __forceinline__ int key_index(unsigned long long key) {
  return (int)(0xFFFFFFFFu - (uint32_t)key);
}

// 16 consecutive logits through a buffer resource over the row (reads past the
// row's end return 0 and are masked by index afterwards).
template <bool kVec>
__device__ __forceinline__ void row_load16(__amdgpu_buffer_rsrc_t rs, int e0, float* x) {
  if (kVec) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const tv_f32x4 a = __builtin_bit_cast(tv_f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * e0 + 16 * i, 0, 0));
      x[4 * i] = a[0];
      x[4 * i + 1] = a[1];
      x[4 * i + 2] = a[2];
      x[4 * i + 3] = a[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (e0 + i), 0, 0));
  }
}

// The thread's best remaining key among its 32 logits (elements e0 + j for
// j < 16, e1 + j - 16 above; removed or out-of-range ones hold -inf).
__device__ __forceinline__ unsigned long long thread_best(const float (&x)[32], int e0, int e1, int* jbest) {
  float bv = -__builtin_huge_valf();
  int bj = -1;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    if (x[j] > bv) {   // strict: the lowest j (lowest index) among equal values
      bv = x[j];
      bj = j;
    }
  }
  *jbest = bj;
  return bj < 0 ? 0ull : topk_key(bv, bj < 16 ? e0 + bj : e1 + bj - 16);
}

// One (frontier row, chunk) unit: the chunk's k best keys into its k slots
// (kKeyNone once the chunk has no element left; every slot kKeyBad when the
// chunk holds a non-finite logit).  Rows at or past the request's frontier
// size are skipped (the request workgroup reads only rows f < n_frontier).
template <bool kVec>
__device__ __forceinline__ void topk_chunk(const ExpandParams& p, unsigned long long (&red)[2][kTopkThreads / 64]) {
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  const int c = blockIdx.x % p.chunks;
  const int row = blockIdx.x / p.chunks;   // b * F + f
  const int b = row / p.F, f = row % p.F;
  const int nf = p.n_frontier[b];
  if (nf < 0 || nf > p.F || f >= nf) return;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.logits + (size_t)row * p.V), (short)0, p.V * 4, 0x00020000);
  const int lo = c * kTopkChunk, hi = min(p.V, lo + kTopkChunk);
  const int e0 = lo + 16 * t, e1 = e0 + 16 * kTopkThreads;
  float x[32];
  row_load16<kVec>(rs, e0, x);
  row_load16<kVec>(rs, e1, x + 16);
  int bad = 0;
  int jb;
  unsigned long long key;
  if (hi - lo == kTopkChunk) {
    // A full chunk: no per-entry bounds tests.  The thread's best is its largest
    // value (three-input maxima) at the first entry holding it, the same key
    // as thread_best gives when every entry is finite (a chunk with a
    // non-finite entry publishes kKeyBad instead).
#pragma unroll
    for (int j = 0; j < 32; ++j) bad |= !isfinite(x[j]);
    const float m = fmaxf(tv_max16(x), tv_max16(x + 16));
    int jm = 31;
#pragma unroll
    for (int j = 30; j >= 0; --j) jm = x[j] == m ? j : jm;
    jb = jm;
    key = topk_key(m, jm < 16 ? e0 + jm : e1 + jm - 16);
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int e = j < 16 ? e0 + j : e1 + j - 16;
      if (e < hi) bad |= !isfinite(x[j]);
      else x[j] = -__builtin_huge_valf();   // outside the chunk: never selected
    }
    key = thread_best(x, e0, e1, &jb);
  }
  unsigned long long* out = p.keys + ((size_t)row * p.chunks + c) * p.k;
  if (__syncthreads_or(bad)) {
    if (t < p.k) __hip_atomic_store(out + t, kKeyBad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  for (int r = 0; r < p.k; ++r) {
    const unsigned long long wmax = tv_wave_max_u64(key);
    if (l == 0) red[r & 1][w] = wmax;
    __syncthreads();
    unsigned long long m = red[r & 1][0];
#pragma unroll
    for (int i = 1; i < kTopkThreads / 64; ++i) m = red[r & 1][i] > m ? red[r & 1][i] : m;
    if (t == 0) __hip_atomic_store(out + r, m ? m : kKeyNone, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (m != 0ull && key == m) {   // keys are unique: exactly one thread holds the winner
#pragma unroll
      for (int j = 0; j < 32; ++j)
        if (j == jb) x[j] = -__builtin_huge_valf();
      key = thread_best(x, e0, e1, &jb);
    }
  }
}

struct AppendSmem {
  int flags;
  int win[kMaxTreeNodes];     // the appended tokens, in id order (at most n_max - 1 of them)
  int front[kMaxTreeNodes];   // the frontier ids (n_frontier * k < n_max once the checks pass)
};

// Request b's workgroup: status, then one wave per frontier row f <
// n_frontier waits for the row's chunks * k slots (at most 256: four per
// lane), merges them by k rounds of a wave maximum and clears them; the
// children are appended once every row is in.  The slots of rows f <
// n_frontier are drained whenever the chunk workgroups wrote them (the
// workspace is prepared and n_frontier is in range), also when the request
// fails its other checks, so that no slot stays set for the next call.  A row
// not complete within p.spin rounds fails the request with TV_REQ_TIMEOUT and
// invalidates the workspace header (its slots may still be written later):
// later calls report TV_REQ_BAD_WORKSPACE until the workspace is prepared
// again.
__device__ void topk_append(const ExpandParams& p, AppendSmem& sm, int b) {
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  const int n0 = p.n_nodes[b], nf = p.n_frontier[b];
  const unsigned long long magic = p.header[0], bytes = p.header[1];
  const bool wsok = (magic == kWsMagic) & (bytes >= p.need);
  if (t == 0) sm.flags = 0;
  __syncthreads();
  int fl = 0;
  if (!wsok) fl = TV_REQ_BAD_WORKSPACE;
  else if (nf < 0 || nf > p.F) fl = TV_REQ_BAD_LEN;
  else if (n0 < 1 || n0 > p.n_max) fl = TV_REQ_BAD_NNODES;
  else if (n0 + nf * p.k > p.n_max) fl = TV_REQ_TREE_OVERFLOW;
  if (fl == 0) {
    for (int f = t; f < nf; f += kTopkThreads) {
      const int u = p.frontier[(size_t)b * p.F + f];
      sm.front[f] = u;
      if (u < 0 || u >= n0) atomicOr(&sm.flags, TV_REQ_BAD_LEN);
    }
  }
  const bool drain = wsok && nf >= 0 && nf <= p.F;
  const int nk = p.chunks * p.k;
  for (int f = w; drain && f < nf; f += kTopkThreads / 64) {
    unsigned long long* keys = p.keys + ((size_t)b * p.F + f) * nk;
    unsigned long long kk[4] = {0ull, 0ull, 0ull, 0ull};
    bool done = p.spin >= 0;
    for (long long it = 0; done; ++it) {
      bool mine = true;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = l + 64 * i;
        if (s < nk && kk[i] == 0ull) kk[i] = __hip_atomic_load(keys + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        mine = mine && (s >= nk || kk[i] != 0ull);
      }
      if (__all(mine)) break;
      if (it >= p.spin) done = false;
      else __builtin_amdgcn_s_sleep(2);
    }
    if (!done) {
      if (l == 0) {
        atomicOr(&sm.flags, TV_REQ_TIMEOUT);
        p.header[0] = 0ull;
      }
      continue;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (l + 64 * i < nk) __hip_atomic_store(keys + l + 64 * i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) bad = bad || kk[i] == kKeyBad;
    if (__any(bad)) {
      if (l == 0) atomicOr(&sm.flags, TV_REQ_NONFINITE);
      continue;
    }
    if (fl) continue;   // drained only
    for (int r = 0; r < p.k; ++r) {
      unsigned long long mine = kk[0];
#pragma unroll
      for (int i = 1; i < 4; ++i) mine = kk[i] > mine ? kk[i] : mine;
      const unsigned long long m = tv_wave_max_u64(mine);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (kk[i] == m) kk[i] = 0ull;   // the k best are unique keys: one lane, one slot
      if (l == 0) sm.win[f * p.k + r] = key_index(m);
    }
  }
  __syncthreads();
  const int got = sm.flags;
  // Precedence as in the checks above: a request that fails them reports only
  // those flags (and a timeout); a non-finite row is reported otherwise.
  if (fl == 0) fl = got;
  else fl |= got & TV_REQ_TIMEOUT;
  if (fl) {
    if (t == 0) {
      p.status[b] = fl;
      p.n_new[b] = 0;
    }
    return;
  }
  const int nnew = nf * p.k;
  int32_t* tokens = p.tokens + (size_t)b * p.n_max + n0;
  int32_t* parent = p.parent + (size_t)b * p.n_max + n0;
  int32_t* nfr = p.new_frontier + (size_t)b * p.F * p.k;
  for (int i = t; i < nnew; i += kTopkThreads) {
    tokens[i] = sm.win[i];
    parent[i] = sm.front[i / p.k];
    nfr[i] = n0 + i;
  }
  if (t == 0) {
    p.n_nodes[b] = n0 + nnew;
    p.n_new[b] = nnew;
    p.status[b] = 0;
  }
}

template <bool kVec>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(ExpandParams p) {
  __shared__ union {
    unsigned long long red[2][kTopkThreads / 64];
    AppendSmem a;
  } sm;
  if ((int)blockIdx.x >= p.G) topk_append(p, sm.a, (int)blockIdx.x - p.G);
  else topk_chunk<kVec>(p, sm.red);
}

int check_expand(const tv_expand_desc* d) {
  if (!d) return TV_ERR_INVALID_ARG;
  if (d->batch < 0 || d->f_max < 1 || d->vocab < 1 || d->n_max < 1 || d->k < 1) return TV_ERR_INVALID_ARG;
  if (d->k > d->vocab) return TV_ERR_INVALID_ARG;
  if (d->k > kMaxK || d->n_max > kMaxTreeNodes) return TV_ERR_UNSUPPORTED;
  const long long chunks = (d->vocab + kTopkChunk - 1) / kTopkChunk;
  if (chunks * d->k > 256) return TV_ERR_UNSUPPORTED;   // a request workgroup's wave holds 4 slots per lane
  return TV_OK;
}

struct ExpandLayout {
  size_t keys, bytes;
  int chunks;
};

// The workspace: the prepared-workspace header, then the key slots.
ExpandLayout expand_layout(const tv_expand_desc* d) {
  ExpandLayout L;
  L.chunks = (d->vocab + kTopkChunk - 1) / kTopkChunk;
  const size_t rows = (size_t)d->batch * d->f_max;
  L.keys = kWsHeader;
  L.bytes = tv_align_up(L.keys + rows * L.chunks * d->k * sizeof(unsigned long long), 256);
  return L;
}

}  // namespace

static int tree_merge_candidates_impl(const tv_merge_desc* desc, const int32_t* cand_tokens,
                                     const int32_t* cand_len, const int32_t* root_token, int32_t* tokens,
                                     int32_t* parent, int32_t* n_nodes, int32_t* node_of, int32_t* status,
                                     hipStream_t stream) {
  if (!desc) return TV_ERR_INVALID_ARG;
  if (desc->batch < 0 || desc->n_cand < 1 || desc->max_len < 1 || desc->n_max < 1) return TV_ERR_INVALID_ARG;
  if (desc->n_cand > kMaxCand || desc->max_len > kMaxCandLen || desc->n_max > kMaxTreeNodes)
    return TV_ERR_UNSUPPORTED;
  if (desc->batch == 0) return TV_OK;
  if (!cand_tokens || !cand_len || !root_token || !tokens || !parent || !n_nodes || !status)
    return TV_ERR_INVALID_ARG;
  MergeParams p;
  p.cand_tokens = cand_tokens;
  p.cand_len = cand_len;
  p.root_token = root_token;
  p.tokens = tokens;
  p.parent = parent;
  p.n_nodes = n_nodes;
  p.node_of = node_of;
  p.status = status;
  p.M = desc->n_cand;
  p.L = desc->max_len;
  p.n_max = desc->n_max;
  hipLaunchKernelGGL(tree_merge_kernel, dim3((unsigned)desc->batch), dim3(kMergeThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

extern "C" int tree_merge_candidates(const tv_merge_desc* desc, const int32_t* cand_tokens,
                                     const int32_t* cand_len, const int32_t* root_token, int32_t* tokens,
                                     int32_t* parent, int32_t* n_nodes, int32_t* node_of, int32_t* status,
                                     hipStream_t stream) {
  TV_TRACE_SCOPE("tree_merge_candidates");
  return tv_debug_finish("tree_merge_candidates", tree_merge_candidates_impl(desc, cand_tokens, cand_len, root_token, tokens, parent, n_nodes, node_of, status, stream), stream);
}

extern "C" size_t tree_expand_workspace_size(const tv_expand_desc* desc) {
  if (check_expand(desc) != TV_OK) return 0;
  return expand_layout(desc).bytes;
}

static int tree_expand_topk_impl(const tv_expand_desc* desc, const float* draft_logits, const int32_t* frontier,
                                const int32_t* n_frontier, int32_t* tokens, int32_t* parent, int32_t* n_nodes,
                                int32_t* new_frontier, int32_t* n_new, int32_t* status, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  const int rc = check_expand(desc);
  if (rc != TV_OK) return rc;
  if (desc->batch == 0) return TV_OK;
  if (!draft_logits || !frontier || !n_frontier || !tokens || !parent || !n_nodes || !new_frontier || !n_new ||
      !status)
    return TV_ERR_INVALID_ARG;
  if (((uintptr_t)draft_logits & 15) != 0) return TV_ERR_INVALID_ARG;
  const ExpandLayout L = expand_layout(desc);
  if (!workspace || workspace_bytes < L.bytes) return TV_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255) != 0) return TV_ERR_INVALID_ARG;
  ExpandParams p;
  p.logits = draft_logits;
  p.frontier = frontier;
  p.n_frontier = n_frontier;
  p.tokens = tokens;
  p.parent = parent;
  p.n_nodes = n_nodes;
  p.new_frontier = new_frontier;
  p.n_new = n_new;
  p.status = status;
  p.header = (unsigned long long*)workspace;
  p.need = L.bytes;
  p.keys = (unsigned long long*)((char*)workspace + L.keys);
  p.B = desc->batch;
  p.F = desc->f_max;
  p.V = desc->vocab;
  p.n_max = desc->n_max;
  p.k = desc->k;
  p.chunks = L.chunks;
  const long long units = (long long)desc->batch * desc->f_max * L.chunks;
  const long long grid = units + desc->batch;
  if (grid > 0x7fffffff || (long long)desc->vocab * 4 > 0x7fffffff) return TV_ERR_UNSUPPORTED;
  p.G = (int)units;
  p.spin = tv_chase_spin_limit(kAppendSpinLimit);
  if ((desc->vocab & 3) == 0)
    hipLaunchKernelGGL(topk_kernel<true>, dim3((unsigned)grid), dim3(kTopkThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(topk_kernel<false>, dim3((unsigned)grid), dim3(kTopkThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

extern "C" int tree_expand_topk(const tv_expand_desc* desc, const float* draft_logits, const int32_t* frontier,
                                const int32_t* n_frontier, int32_t* tokens, int32_t* parent, int32_t* n_nodes,
                                int32_t* new_frontier, int32_t* n_new, int32_t* status, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  TV_TRACE_SCOPE("tree_expand_topk");
  return tv_debug_finish("tree_expand_topk", tree_expand_topk_impl(desc, draft_logits, frontier, n_frontier, tokens, parent, n_nodes, new_frontier, n_new, status, workspace, workspace_bytes, stream), stream);
}
