// Internal helpers shared by the gfx950 kernels of libtreeverify.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tree_verify.h"

#define TV_WAVE 64

typedef __bf16 tv_bf16x8 __attribute__((ext_vector_type(8)));
typedef float tv_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t tv_u32x4 __attribute__((ext_vector_type(4)));

// ---- host-side helpers ----------------------------------------------------

// Number of compute units of the current device (cached per device).
int tv_device_cu_count(int* cu_out);

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

__device__ __forceinline__ float tv_wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ double tv_wave_sum_d(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float tv_wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

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
