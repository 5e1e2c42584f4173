// Accepted-path KV compaction of one (request, KV head), shared by the
// stand-alone compaction kernel and the verify-and-compact chase workgroups of
// the stochastic verifier, so that both give the same caches, src_pos, new_len
// and status.
//
// [guide] "Depth-First Flattening and KV Cache Reuse": after verification only
// the winning root path stays in the cache.  Position P + j receives the K/V
// of position P + path[j] (j = 0..L), all KV heads, in place.  Path ids
// increase strictly and path[j] >= j, so a source can coincide with an
// earlier destination only when it belongs to a later step: a batch of steps
// is hazard-free when every source of the batch is read before any of its
// destinations is written, and the sources of later batches lie past every
// destination of earlier ones.  Each unit of the key and value rows (both
// token-major) -- one element, or 8 bytes of consecutive elements of one KV
// head -- is moved by one thread, independently of the others.
#pragma once

#include "tv_common.h"

#include <type_traits>

struct TvCompactArgs {
  void* k;
  void* v;
  const int32_t* table;
  const int32_t* prefix_len;
  int32_t* src_pos;
  int32_t* new_len;
  int32_t* status;   // may be null
  int n_max, Hkv, D, bs, max_blocks, num_blocks;
};

constexpr int kTvCompactStage = 16;   // path steps staged in registers per batch
constexpr int kTvNoBadBlock = 0x7fffffff;

// Block-table entries read before the path is known (the fused
// verify-and-compact kernel reads them while it walks the path): the first
// entry among [0, nblk_max) that names no pool block, and the entries of the
// blocks that hold positions [P, P + n) (stage[i] = entry stage0 + i).
struct TvTablePrefetch {
  int first_bad;
  int stage0;
  const int* stage;
};

// The unit one thread moves: W elements of type T (W = 1: the element itself;
// otherwise 8 bytes, which needs caches aligned to 8 bytes).
template <typename T, int W>
struct TvMoveUnit {
  static_assert(W == 1 || sizeof(T) * W == 8, "a move unit is one element or 8 bytes");
  using type = typename std::conditional<W == 1, T, uint2>::type;
};

// Compacts KV heads g0 .. g0 + ng - 1 of request b.  Every thread of the
// workgroup calls this (it synchronises); thread t owns the units of W
// consecutive (head, element) pairs t, t + blockDim.x, ... of the ng * D / W.
// path: the request's path (global or LDS), L1 its length (0: nothing
// accepted), P its prefix_len.  pre: table entries read ahead (null: read
// here).  The workgroup holding head 0 writes src_pos, new_len and status.
template <typename T, int W = 1>
__device__ void tv_compact_heads(const TvCompactArgs& p, int b, int g0, int ng, const int32_t* path, int L1, int P,
                                 const TvTablePrefetch* pre, int* s_bad) {
  const int t = threadIdx.x;
  const int32_t* trow = p.table + (size_t)b * p.max_blocks;

  if (t == 0) *s_bad = kTvNoBadBlock;
  __syncthreads();
  int flags = 0;
  if (L1 < 0 || L1 > p.n_max) {
    flags = TV_REQ_BAD_PATH;
  } else if (L1 > 0) {
    for (int j = t; j < L1; j += blockDim.x) {
      int pj = path[j];
      bool ok = (j == 0) ? (pj == 0) : (pj > path[j - 1] && pj < p.n_max);
      if (!ok) *s_bad = 1;
    }
    __syncthreads();
    if (*s_bad != kTvNoBadBlock) {
      flags = TV_REQ_BAD_PATH;
    } else if (P < 0 || (long long)P + path[L1 - 1] >= (long long)p.max_blocks * p.bs) {
      flags = TV_REQ_BAD_KV;
    } else {
      // every block id used by positions [0, P + path[L - 1]] must name a pool block
      const int nblk = (P + path[L1 - 1]) / p.bs + 1;
      int first_bad;
      if (pre) {
        first_bad = pre->first_bad;
      } else {
        __syncthreads();   // every thread has read *s_bad above before it is reused
        for (int i = t; i < nblk; i += blockDim.x) {
          int blk = trow[i];
          if (blk < 0 || blk >= p.num_blocks) atomicMin(s_bad, i);
        }
        __syncthreads();
        first_bad = *s_bad;
      }
      if (first_bad < nblk) flags = TV_REQ_BAD_KV;
    }
  }
  const bool active = (flags == 0 && L1 > 0);
  if (g0 == 0) {
    for (int j = t; j < p.n_max; j += blockDim.x)
      p.src_pos[(size_t)b * p.n_max + j] = (active && j < L1) ? P + path[j] : -1;
    if (t == 0) {
      p.new_len[b] = active ? P + L1 : P;
      if (p.status) p.status[b] = flags;
    }
  }
  if (!active) return;

  using U = typename TvMoveUnit<T, W>::type;
  // a batch of steps keeps 2 * kStage units in registers
  constexpr int kStage = W == 1 ? kTvCompactStage : kTvCompactStage / 2;
  U* K = (U*)p.k;
  U* V = (U*)p.v;
  const int DW = p.D / W;
  for (int e = t; e < ng * DW; e += blockDim.x) {
    const int g = g0 + e / DW, d = e % DW;
    for (int j0 = 1; j0 < L1; j0 += kStage) {
      U kreg[kStage], vreg[kStage];
#pragma unroll
      for (int i = 0; i < kStage; ++i) {
        int j = j0 + i;
        if (j < L1 && path[j] != j) {
          int s = P + path[j];
          size_t blk = (size_t)(pre ? pre->stage[s / p.bs - pre->stage0] : trow[s / p.bs]);
          int slot = s % p.bs;
          kreg[i] = K[((blk * p.Hkv + g) * p.bs + slot) * DW + d];
          vreg[i] = V[((blk * p.Hkv + g) * p.bs + slot) * DW + d];
        }
      }
#pragma unroll
      for (int i = 0; i < kStage; ++i) {
        int j = j0 + i;
        if (j < L1 && path[j] != j) {
          int dst = P + j;
          size_t blk = (size_t)(pre ? pre->stage[dst / p.bs - pre->stage0] : trow[dst / p.bs]);
          int slot = dst % p.bs;
          K[((blk * p.Hkv + g) * p.bs + slot) * DW + d] = kreg[i];
          V[((blk * p.Hkv + g) * p.bs + slot) * DW + d] = vreg[i];
        }
      }
    }
  }
}

// Descriptor checks of the compaction (shared by both entry points).
static inline int tv_compact_check_desc(const tv_attn_desc* desc) {
  if (!desc) return TV_ERR_INVALID_ARG;
  if (desc->batch < 0 || desc->n_kv_heads < 1 || desc->max_blocks_per_seq < 1 || desc->num_blocks < 1)
    return TV_ERR_INVALID_ARG;
  if (desc->n_max < 1 || desc->n_max > 128) return TV_ERR_UNSUPPORTED;
  if (desc->head_dim != 64 && desc->head_dim != 128) return TV_ERR_UNSUPPORTED;
  if (desc->dtype != TV_F32 && desc->dtype != TV_BF16) return TV_ERR_UNSUPPORTED;
  if (desc->block_size != 16 && desc->block_size != 32 && desc->block_size != 64 && desc->block_size != 128)
    return TV_ERR_UNSUPPORTED;
  return TV_OK;
}

static inline TvCompactArgs tv_compact_args(const tv_attn_desc* desc, void* k_cache, void* v_cache,
                                            const int32_t* block_table, const int32_t* prefix_len,
                                            int32_t* src_pos, int32_t* new_len, int32_t* status) {
  TvCompactArgs a;
  a.k = k_cache;
  a.v = v_cache;
  a.table = block_table;
  a.prefix_len = prefix_len;
  a.src_pos = src_pos;
  a.new_len = new_len;
  a.status = status;
  a.n_max = desc->n_max;
  a.Hkv = desc->n_kv_heads;
  a.D = desc->head_dim;
  a.bs = desc->block_size;
  a.max_blocks = desc->max_blocks_per_seq;
  a.num_blocks = desc->num_blocks;
  return a;
}
