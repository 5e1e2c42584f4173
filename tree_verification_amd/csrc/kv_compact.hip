// Accepted-path KV compaction for gfx950.
//
// [guide] "Depth-First Flattening and KV Cache Reuse": after verification only
// the winning root path stays in the cache.  Position P + j receives the K/V
// of position P + path[j] (j = 0..L), all KV heads, in place.  Path ids
// increase strictly and path[j] >= j, so a source can coincide with an
// earlier destination only when it belongs to a later step: a batch of steps
// is hazard-free when every source of the batch is read before any of its
// destinations is written, and the sources of later batches lie past every
// destination of earlier ones.  One workgroup per (request, KV head); thread d
// owns element d of the key rows and of the transposed value rows.

#include "tv_common.h"

namespace {

constexpr int kStage = 16;   // path steps staged in registers per batch

struct CompactParams {
  void* k;
  void* v;
  const int32_t* table;
  const int32_t* prefix_len;
  const int32_t* path;
  const int32_t* path_len;
  int32_t* src_pos;
  int32_t* new_len;
  int32_t* status;
  int B, n_max, Hkv, D, bs, max_blocks, num_blocks, esize;
};

template <typename T>
__global__ __launch_bounds__(128) void compact_kernel(CompactParams p) {
  __shared__ int s_bad;
  const int b = blockIdx.x / p.Hkv, g = blockIdx.x % p.Hkv;
  const int t = threadIdx.x;
  const int P = p.prefix_len[b];
  const int L1 = p.path_len[b];
  const int32_t* path = p.path + (size_t)b * p.n_max;
  const int32_t* trow = p.table + (size_t)b * p.max_blocks;

  if (t == 0) s_bad = 0;
  __syncthreads();
  int flags = 0;
  if (L1 < 0 || L1 > p.n_max) {
    flags = TV_REQ_BAD_PATH;
  } else if (L1 > 0) {
    for (int j = t; j < L1; j += blockDim.x) {
      int pj = path[j];
      bool ok = (j == 0) ? (pj == 0) : (pj > path[j - 1] && pj < p.n_max);
      if (!ok) s_bad = 1;
    }
    __syncthreads();
    if (s_bad) {
      flags = TV_REQ_BAD_PATH;
    } else if (P < 0 || (long long)P + path[L1 - 1] >= (long long)p.max_blocks * p.bs) {
      flags = TV_REQ_BAD_KV;
    } else {
      int nblk = (P + path[L1 - 1]) / p.bs + 1;
      __syncthreads();
      for (int i = t; i < nblk; i += blockDim.x) {
        int blk = trow[i];
        if (blk < 0 || blk >= p.num_blocks) s_bad = 1;
      }
      __syncthreads();
      if (s_bad) flags = TV_REQ_BAD_KV;
    }
  }
  const bool active = (flags == 0 && L1 > 0);
  if (g == 0) {
    for (int j = t; j < p.n_max; j += blockDim.x)
      p.src_pos[(size_t)b * p.n_max + j] = (active && j < L1) ? P + path[j] : -1;
    if (t == 0) {
      p.new_len[b] = active ? P + L1 : P;
      if (p.status) p.status[b] = flags;
    }
  }
  if (!active || t >= p.D) return;

  T* K = (T*)p.k;
  T* V = (T*)p.v;
  for (int j0 = 1; j0 < L1; j0 += kStage) {
    T kreg[kStage], vreg[kStage];
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      int j = j0 + i;
      if (j < L1 && path[j] != j) {
        int s = P + path[j];
        size_t blk = (size_t)trow[s / p.bs];
        int slot = s % p.bs;
        kreg[i] = K[((blk * p.Hkv + g) * p.bs + slot) * p.D + t];
        vreg[i] = V[((blk * p.Hkv + g) * p.D + t) * p.bs + slot];
      }
    }
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      int j = j0 + i;
      if (j < L1 && path[j] != j) {
        int d = P + j;
        size_t blk = (size_t)trow[d / p.bs];
        int slot = d % p.bs;
        K[((blk * p.Hkv + g) * p.bs + slot) * p.D + t] = kreg[i];
        V[((blk * p.Hkv + g) * p.D + t) * p.bs + slot] = vreg[i];
      }
    }
  }
}

}  // namespace

extern "C" int kv_compact_accepted(const tv_attn_desc* desc, void* k_cache, void* v_cache,
                                   const int32_t* block_table, const int32_t* prefix_len,
                                   const int32_t* path, const int32_t* path_len, int32_t* src_pos,
                                   int32_t* new_len, int32_t* status, hipStream_t stream) {
  if (!desc) return TV_ERR_INVALID_ARG;
  if (desc->batch < 0 || desc->n_kv_heads < 1 || desc->max_blocks_per_seq < 1 || desc->num_blocks < 1)
    return TV_ERR_INVALID_ARG;
  if (desc->n_max < 1 || desc->n_max > 128) return TV_ERR_UNSUPPORTED;
  if (desc->head_dim != 64 && desc->head_dim != 128) return TV_ERR_UNSUPPORTED;
  if (desc->dtype != TV_F32 && desc->dtype != TV_BF16) return TV_ERR_UNSUPPORTED;
  if (desc->block_size != 16 && desc->block_size != 32 && desc->block_size != 64 && desc->block_size != 128)
    return TV_ERR_UNSUPPORTED;
  if (desc->batch == 0) return TV_OK;
  if (!k_cache || !v_cache || !block_table || !prefix_len || !path || !path_len || !src_pos || !new_len)
    return TV_ERR_INVALID_ARG;
  CompactParams p;
  p.k = k_cache;
  p.v = v_cache;
  p.table = block_table;
  p.prefix_len = prefix_len;
  p.path = path;
  p.path_len = path_len;
  p.src_pos = src_pos;
  p.new_len = new_len;
  p.status = status;
  p.B = desc->batch;
  p.n_max = desc->n_max;
  p.Hkv = desc->n_kv_heads;
  p.D = desc->head_dim;
  p.bs = desc->block_size;
  p.max_blocks = desc->max_blocks_per_seq;
  p.num_blocks = desc->num_blocks;
  long long grid = (long long)desc->batch * desc->n_kv_heads;
  if (grid > 0x7fffffff) return TV_ERR_UNSUPPORTED;
  if (desc->dtype == TV_BF16)
    hipLaunchKernelGGL(compact_kernel<uint16_t>, dim3((unsigned)grid), dim3(128), 0, stream, p);
  else
    hipLaunchKernelGGL(compact_kernel<float>, dim3((unsigned)grid), dim3(128), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}
