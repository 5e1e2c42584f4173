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
// Expansion (Method A), one level: topk_chunk_kernel gives every (frontier
// row, 8192-logit chunk) its k best 64-bit keys (value order, then lower
// index) by k rounds of a workgroup maximum, each removing the winner from the
// thread that holds it.  topk_append_kernel (one workgroup per request, one
// wave per frontier row) merges the chunks' keys of each row the same way and
// appends the children after the request's last node.

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
  unsigned long long* keys;   // workspace [B][F][chunks][k]
  int* flags;                 // workspace [B][F][chunks]: non-finite logit seen
  int B, F, V, n_max, k, chunks;
};

// Order-preserving key: larger value first, then lower index; never 0 for an
// index below 2^32 - 1, so 0 marks "no element".  -0 and +0 tie.
__device__ __forceinline__ unsigned long long topk_key(float v, int idx) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;
  const uint32_t hi = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)hi << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}

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

template <bool kVec>
__global__ __launch_bounds__(kTopkThreads) void topk_chunk_kernel(ExpandParams p) {
  __shared__ unsigned long long red[2][kTopkThreads / 64];
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  const int c = blockIdx.x % p.chunks;
  const int row = blockIdx.x / p.chunks;   // b * F + f
  const int b = row / p.F, f = row % p.F;
  const int nf = p.n_frontier[b];
  if (nf < 0 || nf > p.F || f >= nf) return;   // the append kernel reads only rows f < nf
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
    // as thread_best gives when every entry is finite (a row with a non-finite
    // entry is flagged, and its keys are not used).
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
  // written for every chunk of every row the append kernel reads, so the
  // workspace needs no clearing (a non-finite row yields unspecified keys; the
  // append kernel then writes nothing)
  if (__syncthreads_or(bad) && t == 0) p.flags[(size_t)row * p.chunks + c] = 1;
  else if (t == 0) p.flags[(size_t)row * p.chunks + c] = 0;
  unsigned long long* out = p.keys + ((size_t)row * p.chunks + c) * p.k;
  for (int r = 0; r < p.k; ++r) {
    const unsigned long long wmax = tv_wave_max_u64(key);
    if (l == 0) red[r & 1][w] = wmax;
    __syncthreads();
    unsigned long long m = red[r & 1][0];
#pragma unroll
    for (int i = 1; i < kTopkThreads / 64; ++i) m = red[r & 1][i] > m ? red[r & 1][i] : m;
    if (t == 0) out[r] = m;
    if (m != 0ull && key == m) {   // keys are unique: exactly one thread holds the winner
#pragma unroll
      for (int j = 0; j < 32; ++j)
        if (j == jb) x[j] = -__builtin_huge_valf();
      key = thread_best(x, e0, e1, &jb);
    }
  }
}

// One workgroup per request: status, then one wave per frontier row merges the
// chunks' keys (k rounds of a wave maximum) and appends the children.
__global__ __launch_bounds__(kTopkThreads) void topk_append_kernel(ExpandParams p) {
  __shared__ int s_bad;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, b = blockIdx.x;
  const int n0 = p.n_nodes[b], nf = p.n_frontier[b];
  if (t == 0) s_bad = 0;
  __syncthreads();
  int fl = 0;
  if (n0 < 1 || n0 > p.n_max) fl = TV_REQ_BAD_NNODES;
  else if (nf < 0 || nf > p.F) fl = TV_REQ_BAD_LEN;
  else if (n0 + nf * p.k > p.n_max) fl = TV_REQ_TREE_OVERFLOW;
  if (fl == 0) {
    for (int f = t; f < nf; f += kTopkThreads) {
      const int u = p.frontier[(size_t)b * p.F + f];
      if (u < 0 || u >= n0) atomicOr(&s_bad, TV_REQ_BAD_LEN);
    }
    for (int q = t; q < nf * p.chunks; q += kTopkThreads)
      if (p.flags[((size_t)b * p.F) * p.chunks + q]) atomicOr(&s_bad, TV_REQ_NONFINITE);
  }
  __syncthreads();
  fl |= s_bad;
  if (fl) {
    if (t == 0) {
      p.status[b] = fl;
      p.n_new[b] = 0;
    }
    return;
  }
  int32_t* tokens = p.tokens + (size_t)b * p.n_max;
  int32_t* parent = p.parent + (size_t)b * p.n_max;
  const int nk = p.chunks * p.k;   // candidate keys per row (<= 64 * 4 at V <= 2^21, k <= 16)
  for (int f = w; f < nf; f += kTopkThreads / 64) {
    const unsigned long long* keys = p.keys + ((size_t)b * p.F + f) * nk;
    unsigned long long kk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kk[i] = l + 64 * i < nk ? keys[l + 64 * i] : 0ull;
    const int u = p.frontier[(size_t)b * p.F + f];
    for (int r = 0; r < p.k; ++r) {
      unsigned long long mine = kk[0];
#pragma unroll
      for (int i = 1; i < 4; ++i) mine = kk[i] > mine ? kk[i] : mine;
      const unsigned long long m = tv_wave_max_u64(mine);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (kk[i] == m) kk[i] = 0ull;   // unique keys: one lane, one slot
      if (l == 0) {
        const int id = n0 + f * p.k + r;
        tokens[id] = key_index(m);
        parent[id] = u;
        p.new_frontier[(size_t)b * p.F * p.k + f * p.k + r] = id;
      }
    }
  }
  if (t == 0) {
    p.n_nodes[b] = n0 + nf * p.k;
    p.n_new[b] = nf * p.k;
    p.status[b] = 0;
  }
}

int check_expand(const tv_expand_desc* d) {
  if (!d) return TV_ERR_INVALID_ARG;
  if (d->batch < 0 || d->f_max < 1 || d->vocab < 1 || d->n_max < 1 || d->k < 1) return TV_ERR_INVALID_ARG;
  if (d->k > d->vocab) return TV_ERR_INVALID_ARG;
  if (d->k > kMaxK || d->n_max > kMaxTreeNodes) return TV_ERR_UNSUPPORTED;
  const long long chunks = (d->vocab + kTopkChunk - 1) / kTopkChunk;
  if (chunks * d->k > 256) return TV_ERR_UNSUPPORTED;   // the append kernel's wave holds 4 keys per lane
  return TV_OK;
}

struct ExpandLayout {
  size_t keys, flags, bytes;
  int chunks;
};

ExpandLayout expand_layout(const tv_expand_desc* d) {
  ExpandLayout L;
  L.chunks = (d->vocab + kTopkChunk - 1) / kTopkChunk;
  const size_t rows = (size_t)d->batch * d->f_max;
  L.keys = 0;
  size_t o = tv_align_up(rows * L.chunks * d->k * sizeof(unsigned long long), 256);
  L.flags = o;
  o = tv_align_up(o + rows * L.chunks * sizeof(int), 256);
  L.bytes = o;
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
  p.keys = (unsigned long long*)((char*)workspace + L.keys);
  p.flags = (int*)((char*)workspace + L.flags);
  p.B = desc->batch;
  p.F = desc->f_max;
  p.V = desc->vocab;
  p.n_max = desc->n_max;
  p.k = desc->k;
  p.chunks = L.chunks;
  const long long grid = (long long)desc->batch * desc->f_max * L.chunks;
  if (grid > 0x7fffffff || (long long)desc->vocab * 4 > 0x7fffffff) return TV_ERR_UNSUPPORTED;
  if ((desc->vocab & 3) == 0)
    hipLaunchKernelGGL(topk_chunk_kernel<true>, dim3((unsigned)grid), dim3(kTopkThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(topk_chunk_kernel<false>, dim3((unsigned)grid), dim3(kTopkThreads), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return TV_ERR_HIP;
  hipLaunchKernelGGL(topk_append_kernel, dim3((unsigned)desc->batch), dim3(kTopkThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

extern "C" int tree_expand_topk(const tv_expand_desc* desc, const float* draft_logits, const int32_t* frontier,
                                const int32_t* n_frontier, int32_t* tokens, int32_t* parent, int32_t* n_nodes,
                                int32_t* new_frontier, int32_t* n_new, int32_t* status, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  TV_TRACE_SCOPE("tree_expand_topk");
  return tv_debug_finish("tree_expand_topk", tree_expand_topk_impl(desc, draft_logits, frontier, n_frontier, tokens, parent, n_nodes, new_frontier, n_new, status, workspace, workspace_bytes, stream), stream);
}
