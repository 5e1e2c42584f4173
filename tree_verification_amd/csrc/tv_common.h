// Internal helpers shared by the gfx950 kernels of libtreeverify.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tree_verify.h"

#define TV_WAVE 64

typedef __bf16 tv_bf16x8 __attribute__((ext_vector_type(8)));
typedef float tv_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t tv_u32x4 __attribute__((ext_vector_type(4)));

// A workspace whose slots must start at zero begins with a header that
// tree_verify_workspace_init writes after zero-filling the rest: a magic word
// and the number of bytes it cleared.  Kernels that use such slots check it and
// fail their requests with TV_REQ_BAD_WORKSPACE instead of reading a buffer
// that was never prepared (or is too small for the call's layout).
constexpr unsigned long long kWsMagic = 0x7476777370616365ull;
constexpr size_t kWsHeader = 256;

// ---- host-side helpers ----------------------------------------------------

// Number of compute units of the current device (cached per device).
int tv_device_cu_count(int* cu_out);

// ---- tracing and debug validation (host side, tv_api.hip) ------------------
//
// TV_TRACE=1 in the environment: every entry point is a roctx range (the
// roctx library is loaded at run time when present; rocprofv3 --marker-trace
// shows the ranges).  TV_DEBUG=1: entry points copy their tree and KV
// metadata to the host, print every malformed request to stderr before
// launching (the per-request status flags are produced as usual), and
// synchronise after launching, returning TV_ERR_HIP when the GPU reported an
// error.  Both are read once per process.
struct TvTraceScope {
  bool on;
  explicit TvTraceScope(const char* name);
  ~TvTraceScope();
};
#define TV_TRACE_SCOPE(name) TvTraceScope tv_trace_scope_(name)

bool tv_debug_enabled();
// Polling rounds after which a verifier's path-chasing workgroup gives up
// (TV_CHASE_SPIN_LIMIT, read once per process; `dflt` when unset; negative:
// give up without waiting).
long long tv_chase_spin_limit(long long dflt);
// Malformed trees (n_nodes outside [1, n_max], parent[0] != -1, parent[i]
// outside [0, i)) reported on stderr; returns how many requests were reported.
int tv_debug_trees(const char* entry, const int32_t* parent, const int32_t* n_nodes, int batch, int n_max,
                   hipStream_t stream);
// Requests whose positions [0, prefix_len + n_nodes) leave the block table or
// name a block outside the pool, reported on stderr.
int tv_debug_kv(const char* entry, const int32_t* block_table, const int32_t* prefix_len, const int32_t* n_nodes,
                int batch, int max_blocks, int block_size, int num_blocks, hipStream_t stream);
// After the launches: synchronise and turn a GPU error into TV_ERR_HIP (rc otherwise).
int tv_debug_finish(const char* entry, int rc, hipStream_t stream);

#define TV_HIP_TRY(expr)                    \
  do {                                      \
    if ((expr) != hipSuccess) return TV_ERR_HIP; \
  } while (0)

static inline size_t tv_align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- device helpers -------------------------------------------------------

__device__ __forceinline__ float tv_bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// float32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t tv_f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Full-wave butterflies without LDS traffic: four DPP patterns inside each row
// of 16 lanes (quad swaps, half-row and row mirrors), then the row swaps of
// v_permlane16_swap / v_permlane32_swap.  Every lane ends with the same value,
// combined in the same order (each step pairs a with b and b with a), so the
// result does not depend on the lane.
template <int CTRL>
__device__ __forceinline__ uint32_t tv_dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <class Op>
__device__ __forceinline__ uint32_t tv_wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, tv_dpp<0xB1>(v));    // quad_perm [1,0,3,2]
  v = op(v, tv_dpp<0x4E>(v));    // quad_perm [2,3,0,1]
  v = op(v, tv_dpp<0x141>(v));   // row_half_mirror
  v = op(v, tv_dpp<0x140>(v));   // row_mirror
  auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(r16[0], r16[1]);
  auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(r32[0], r32[1]);
}

template <class Op>
__device__ __forceinline__ uint64_t tv_wave_reduce_u64(uint64_t v, Op op) {
  auto step = [&](uint32_t lo, uint32_t hi) { return ((uint64_t)hi << 32) | lo; };
  v = op(v, step(tv_dpp<0xB1>((uint32_t)v), tv_dpp<0xB1>((uint32_t)(v >> 32))));
  v = op(v, step(tv_dpp<0x4E>((uint32_t)v), tv_dpp<0x4E>((uint32_t)(v >> 32))));
  v = op(v, step(tv_dpp<0x141>((uint32_t)v), tv_dpp<0x141>((uint32_t)(v >> 32))));
  v = op(v, step(tv_dpp<0x140>((uint32_t)v), tv_dpp<0x140>((uint32_t)(v >> 32))));
  {
    auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    v = op(step(lo[0], hi[0]), step(lo[1], hi[1]));
  }
  {
    auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    v = op(step(lo[0], hi[0]), step(lo[1], hi[1]));
  }
  return v;
}

__device__ __forceinline__ float tv_wave_max(float v) {
  return __uint_as_float(tv_wave_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    const float x = __uint_as_float(a), y = __uint_as_float(b);
    return __float_as_uint(x > y ? x : y);
  }));
}

__device__ __forceinline__ float tv_wave_sum(float v) {
  return __uint_as_float(tv_wave_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}

__device__ __forceinline__ double tv_wave_sum_d(double v) {
  return __longlong_as_double((long long)tv_wave_reduce_u64((uint64_t)__double_as_longlong(v), [](uint64_t a, uint64_t b) {
    return (uint64_t)__double_as_longlong(__longlong_as_double((long long)a) + __longlong_as_double((long long)b));
  }));
}

// Reductions inside each row of 16 lanes (every lane of a row gets its row's result).
__device__ __forceinline__ float tv_row16_max(float v) {
  auto mx = [](float a, float b) { return a > b ? a : b; };
  v = mx(v, __uint_as_float(tv_dpp<0xB1>(__float_as_uint(v))));
  v = mx(v, __uint_as_float(tv_dpp<0x4E>(__float_as_uint(v))));
  v = mx(v, __uint_as_float(tv_dpp<0x141>(__float_as_uint(v))));
  return mx(v, __uint_as_float(tv_dpp<0x140>(__float_as_uint(v))));
}

__device__ __forceinline__ double tv_row16_sum_d(double v) {
  auto part = [](double x, auto sel) {
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    return __longlong_as_double((long long)(((uint64_t)sel((uint32_t)(b >> 32)) << 32) | sel((uint32_t)b)));
  };
  v += part(v, [](uint32_t x) { return tv_dpp<0xB1>(x); });
  v += part(v, [](uint32_t x) { return tv_dpp<0x4E>(x); });
  v += part(v, [](uint32_t x) { return tv_dpp<0x141>(x); });
  v += part(v, [](uint32_t x) { return tv_dpp<0x140>(x); });
  return v;
}

// The double held by lane `src` (wave-uniform), to every lane.
__device__ __forceinline__ double tv_readlane_d(double v, int src) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), src);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive prefix sums of doubles over the wave: shifts by 1, 2, 4 and 8
// lanes inside each row of 16 (lanes shifted in from outside the row read 0),
// then the rows' totals (lanes 15, 31, 47) added in row order.
__device__ __forceinline__ double tv_wave_incl_scan_d(double x, int lane) {
  auto shifted = [](double v, auto sel) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    return __longlong_as_double((long long)(((uint64_t)sel((uint32_t)(b >> 32)) << 32) | sel((uint32_t)b)));
  };
  x += shifted(x, [](uint32_t v) { return tv_dpp<0x111>(v); });   // row_shr:1
  x += shifted(x, [](uint32_t v) { return tv_dpp<0x112>(v); });   // row_shr:2
  x += shifted(x, [](uint32_t v) { return tv_dpp<0x114>(v); });   // row_shr:4
  x += shifted(x, [](uint32_t v) { return tv_dpp<0x118>(v); });   // row_shr:8
  const double r0 = tv_readlane_d(x, 15), r1 = tv_readlane_d(x, 31), r2 = tv_readlane_d(x, 47);
  const double o1 = r0, o2 = r0 + r1, o3 = o2 + r2;
  const int row = lane >> 4;
  return x + (row == 0 ? 0.0 : row == 1 ? o1 : row == 2 ? o2 : o3);
}

// Combine the four rows of 16 lanes (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float tv_rows_max(float v) {
  auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

__device__ __forceinline__ float tv_rows_sum(float v) {
  auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Unsigned 64-bit maximum over the wave.
__device__ __forceinline__ unsigned long long tv_wave_max_u64(unsigned long long v) {
  return tv_wave_reduce_u64(v, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
}

// LDS-only workgroup barrier: unlike __syncthreads it does not first wait for
// the wave's outstanding global loads, so loads issued earlier stay in flight.
// Largest of 16 floats by three-input maxima (NaN entries are skipped, as by
// fmaxf; -0 and +0 compare equal).
__device__ __forceinline__ float tv_max16(const float* x) {
  const float a = fmaxf(fmaxf(x[0], x[1]), x[2]), b = fmaxf(fmaxf(x[3], x[4]), x[5]);
  const float c = fmaxf(fmaxf(x[6], x[7]), x[8]), d = fmaxf(fmaxf(x[9], x[10]), x[11]);
  const float e = fmaxf(fmaxf(x[12], x[13]), x[14]);
  return fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), x[15]));
}

__device__ __forceinline__ void tv_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Acquire/release helpers for inter-workgroup hand-offs through global memory.
__device__ __forceinline__ int tv_atomic_add_release(int* p, int v) {
  __threadfence();
  return atomicAdd(p, v);
}

__device__ __forceinline__ int tv_load_acquire(const int* p) {
  int v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __threadfence();
  return v;
}

// Remap a linear workgroup id so that consecutive logical ids land on the same
// XCD (the hardware deals workgroups to the 8 XCDs round-robin), keeping tiles
// that share data inside one L2.
__device__ __forceinline__ int tv_xcd_remap(int pid, int total) {
  const int nx = 8;
  int x = pid % nx, local = pid / nx;
  int per = total / nx, rem = total % nx;
  return x * per + (x < rem ? x : rem) + local;
}
