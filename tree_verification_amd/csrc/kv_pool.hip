// Paged speculative-block pool for gfx950 ([guide] "PagedKV Allocation with
// Zero-Copy Pruning": the tree's blocks come from the paged pool and are
// speculative; after verification the unselected branches' blocks return to
// the free pool in one metadata update).
//
// The pool is a stack of free block ids, free_ids[0 .. *free_count).  Each
// call is one workgroup that serves the batch in request order, 256 requests
// per pass, one thread per request: an exclusive scan of the block counts
// gives each request its segment of the stack, and *free_count changes once,
// at the end.  A request the pool cannot serve (too few free blocks, or a
// stack that would overflow) fails, and so does every later request that needs
// blocks moved; requests that move nothing always succeed.

#include "tv_common.h"

namespace {

constexpr int kPoolThreads = 256;

struct PoolParams {
  int32_t* table;             // [B][max_blocks]
  int32_t* n_blocks;          // [B]
  const int32_t* prefix_len;  // [B]  (allocation)
  const int32_t* n_nodes;     // [B]  (allocation)
  const int32_t* new_len;     // [B]  (release)
  int32_t* free_ids;          // [num_blocks]
  int32_t* free_count;        // [1]
  int32_t* spec_from;         // [B]  (allocation)
  int32_t* status;            // [B]
  int B, bs, max_blocks, num_blocks;
};

// Inclusive prefix sum of one int per thread over the workgroup; *total gets
// the sum of all.  Ends with a barrier, so `part` may be reused right after.
__device__ __forceinline__ int block_incl_scan(int x, int* part, int* total) {
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (l >= d) x += y;
  }
  if (l == 63) part[w] = x;
  __syncthreads();
  int off = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kPoolThreads / 64; ++i) {
    off += i < w ? part[i] : 0;
    all += part[i];
  }
  __syncthreads();
  *total = all;
  return x + off;
}

__device__ __forceinline__ int ceil_div(int a, int b) { return a / b + (a % b != 0 ? 1 : 0); }

__global__ __launch_bounds__(kPoolThreads) void alloc_kernel(PoolParams p) {
  __shared__ int part[kPoolThreads / 64];
  const int t = threadIdx.x;
  const int fc = *p.free_count;
  const bool pool_ok = fc >= 0 && fc <= p.num_blocks;
  int promised = 0, served = 0;   // over earlier passes (uniform)
  for (int b0 = 0; b0 < p.B; b0 += kPoolThreads) {
    const int b = b0 + t;
    int st = 0, extra = 0, nb = 0;
    if (b < p.B) {
      const int P = p.prefix_len[b], n = p.n_nodes[b];
      nb = p.n_blocks[b];
      if (!pool_ok || P < 0 || n < 0 || nb < 0 || nb > p.max_blocks || P > 0x7fffffff - n) {
        st = TV_REQ_BAD_KV;
      } else {
        const int need = ceil_div(P + n, p.bs);
        if (need > p.max_blocks) st = TV_REQ_BAD_KV;
        else extra = need > nb ? need - nb : 0;
      }
    }
    int total;
    const int cum = promised + block_incl_scan(extra, part, &total);
    const bool ok = b < p.B && st == 0 && (extra == 0 || cum <= fc);
    if (b < p.B && st == 0 && !ok) st = TV_REQ_POOL_EXHAUSTED;
    if (ok) {
      const int top = fc - (cum - extra);   // stack top before this request's pops
      int32_t* row = p.table + (size_t)b * p.max_blocks;
      for (int j = 0; j < extra; ++j) row[nb + j] = p.free_ids[top - 1 - j];
      p.n_blocks[b] = nb + extra;
    }
    if (b < p.B) {
      p.spec_from[b] = ok ? nb : -1;
      p.status[b] = st;
    }
    int got;
    block_incl_scan(ok ? extra : 0, part, &got);
    served += got;
    promised += total;
  }
  if (t == 0 && pool_ok) *p.free_count = fc - served;
}

__global__ __launch_bounds__(kPoolThreads) void release_kernel(PoolParams p) {
  __shared__ int part[kPoolThreads / 64];
  const int t = threadIdx.x;
  const int fc = *p.free_count;
  const bool pool_ok = fc >= 0 && fc <= p.num_blocks;
  int promised = 0, pushed = 0;
  for (int b0 = 0; b0 < p.B; b0 += kPoolThreads) {
    const int b = b0 + t;
    int st = 0, rel = 0, keep = 0;
    const int32_t* row = p.table + (size_t)b * p.max_blocks;
    if (b < p.B) {
      const int L = p.new_len[b], nb = p.n_blocks[b];
      if (!pool_ok || L < 0 || nb < 0 || nb > p.max_blocks) {
        st = TV_REQ_BAD_KV;
      } else {
        keep = ceil_div(L, p.bs);
        if (keep > nb) {
          st = TV_REQ_BAD_KV;
        } else {
          for (int j = keep; j < nb; ++j)
            if (row[j] < 0 || row[j] >= p.num_blocks) st = TV_REQ_BAD_KV;
          if (st == 0) rel = nb - keep;
        }
      }
    }
    int total;
    const int cum = promised + block_incl_scan(rel, part, &total);
    const bool ok = b < p.B && st == 0 && (rel == 0 || fc + cum <= p.num_blocks);
    if (b < p.B && st == 0 && !ok) st = TV_REQ_POOL_EXHAUSTED;
    if (ok) {
      const int base = fc + cum - rel;
      int32_t* wrow = p.table + (size_t)b * p.max_blocks;
      for (int j = 0; j < rel; ++j) {
        p.free_ids[base + j] = wrow[keep + j];
        wrow[keep + j] = -1;
      }
      p.n_blocks[b] = keep;
    }
    if (b < p.B) p.status[b] = st;
    int got;
    block_incl_scan(ok ? rel : 0, part, &got);
    pushed += got;
    promised += total;
  }
  if (t == 0 && pool_ok) *p.free_count = fc + pushed;
}

int check_pool_desc(const tv_attn_desc* d) {
  if (!d) return TV_ERR_INVALID_ARG;
  if (d->batch < 0 || d->block_size < 1 || d->max_blocks_per_seq < 1 || d->num_blocks < 1) return TV_ERR_INVALID_ARG;
  return TV_OK;
}

}  // namespace

static int kv_alloc_tree_blocks_impl(const tv_attn_desc* desc, int32_t* block_table, int32_t* n_blocks,
                                    const int32_t* prefix_len, const int32_t* n_nodes, const int32_t* free_ids,
                                    int32_t* free_count, int32_t* spec_from, int32_t* status, hipStream_t stream) {
  const int rc = check_pool_desc(desc);
  if (rc != TV_OK) return rc;
  if (desc->batch == 0) return TV_OK;
  if (!block_table || !n_blocks || !prefix_len || !n_nodes || !free_ids || !free_count || !spec_from || !status)
    return TV_ERR_INVALID_ARG;
  PoolParams p{};
  p.table = block_table;
  p.n_blocks = n_blocks;
  p.prefix_len = prefix_len;
  p.n_nodes = n_nodes;
  p.free_ids = const_cast<int32_t*>(free_ids);   // read only by this kernel
  p.free_count = free_count;
  p.spec_from = spec_from;
  p.status = status;
  p.B = desc->batch;
  p.bs = desc->block_size;
  p.max_blocks = desc->max_blocks_per_seq;
  p.num_blocks = desc->num_blocks;
  hipLaunchKernelGGL(alloc_kernel, dim3(1), dim3(kPoolThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

extern "C" int kv_alloc_tree_blocks(const tv_attn_desc* desc, int32_t* block_table, int32_t* n_blocks,
                                    const int32_t* prefix_len, const int32_t* n_nodes, const int32_t* free_ids,
                                    int32_t* free_count, int32_t* spec_from, int32_t* status, hipStream_t stream) {
  TV_TRACE_SCOPE("kv_alloc_tree_blocks");
  return tv_debug_finish("kv_alloc_tree_blocks", kv_alloc_tree_blocks_impl(desc, block_table, n_blocks, prefix_len, n_nodes, free_ids, free_count, spec_from, status, stream), stream);
}

static int kv_release_blocks_impl(const tv_attn_desc* desc, int32_t* block_table, int32_t* n_blocks,
                                 const int32_t* new_len, int32_t* free_ids, int32_t* free_count, int32_t* status,
                                 hipStream_t stream) {
  const int rc = check_pool_desc(desc);
  if (rc != TV_OK) return rc;
  if (desc->batch == 0) return TV_OK;
  if (!block_table || !n_blocks || !new_len || !free_ids || !free_count || !status) return TV_ERR_INVALID_ARG;
  PoolParams p{};
  p.table = block_table;
  p.n_blocks = n_blocks;
  p.new_len = new_len;
  p.free_ids = free_ids;
  p.free_count = free_count;
  p.status = status;
  p.B = desc->batch;
  p.bs = desc->block_size;
  p.max_blocks = desc->max_blocks_per_seq;
  p.num_blocks = desc->num_blocks;
  hipLaunchKernelGGL(release_kernel, dim3(1), dim3(kPoolThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

extern "C" int kv_release_blocks(const tv_attn_desc* desc, int32_t* block_table, int32_t* n_blocks,
                                 const int32_t* new_len, int32_t* free_ids, int32_t* free_count, int32_t* status,
                                 hipStream_t stream) {
  TV_TRACE_SCOPE("kv_release_blocks");
  return tv_debug_finish("kv_release_blocks", kv_release_blocks_impl(desc, block_table, n_blocks, new_len, free_ids, free_count, status, stream), stream);
}
