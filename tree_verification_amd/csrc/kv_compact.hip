// Accepted-path KV compaction for gfx950: one workgroup per (request, KV
// head) runs the shared per-head compaction (tv_compact.h).

#include "tv_compact.h"

namespace {

// One workgroup per (request, KV head).
template <typename T>
__global__ __launch_bounds__(128) void compact_kernel(TvCompactArgs p, const int32_t* path, const int32_t* path_len) {
  __shared__ int s_bad;
  const int b = blockIdx.x / p.Hkv, g = blockIdx.x % p.Hkv;
  tv_compact_heads<T>(p, b, g, 1, path + (size_t)b * p.n_max, path_len[b], p.prefix_len[b], nullptr, &s_bad);
}

}  // namespace

static int kv_compact_accepted_impl(const tv_attn_desc* desc, void* k_cache, void* v_cache,
                                   const int32_t* block_table, const int32_t* prefix_len,
                                   const int32_t* path, const int32_t* path_len, int32_t* src_pos,
                                   int32_t* new_len, int32_t* status, hipStream_t stream) {
  const int rc = tv_compact_check_desc(desc);
  if (rc != TV_OK) return rc;
  if (desc->batch == 0) return TV_OK;
  if (!k_cache || !v_cache || !block_table || !prefix_len || !path || !path_len || !src_pos || !new_len)
    return TV_ERR_INVALID_ARG;
  const TvCompactArgs p = tv_compact_args(desc, k_cache, v_cache, block_table, prefix_len, src_pos, new_len, status);
  long long grid = (long long)desc->batch * desc->n_kv_heads;
  if (grid > 0x7fffffff) return TV_ERR_UNSUPPORTED;
  if (desc->dtype == TV_BF16)
    hipLaunchKernelGGL(compact_kernel<uint16_t>, dim3((unsigned)grid), dim3(128), 0, stream, p, path, path_len);
  else
    hipLaunchKernelGGL(compact_kernel<float>, dim3((unsigned)grid), dim3(128), 0, stream, p, path, path_len);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

extern "C" int kv_compact_accepted(const tv_attn_desc* desc, void* k_cache, void* v_cache,
                                   const int32_t* block_table, const int32_t* prefix_len,
                                   const int32_t* path, const int32_t* path_len, int32_t* src_pos,
                                   int32_t* new_len, int32_t* status, hipStream_t stream) {
  TV_TRACE_SCOPE("kv_compact_accepted");
  return tv_debug_finish("kv_compact_accepted", kv_compact_accepted_impl(desc, k_cache, v_cache, block_table, prefix_len, path, path_len, src_pos, new_len, status, stream), stream);
}
