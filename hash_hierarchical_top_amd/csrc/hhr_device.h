// Device helpers for the gfx950 kernels of libhhr: storage-format conversions,
// wave64 reductions and scans, orderable float keys.  Internal header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hhr_consts.h"

namespace hhr {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- formats
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// f32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Split x into bf16 hi + lo with x - hi - lo within 2^-17 |x|.
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_rne(x);
  lo = f32_to_bf16_rne(x - bf16_to_f32(hi));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Monotone map f32 -> u32 (larger float -> larger key); -0 is folded onto +0.
__device__ __forceinline__ uint32_t orderable_key(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Lanes below this one in the wave.
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ int popc64(uint64_t x) { return __popcll(x); }

// Inclusive scan across the wave.
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T x) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    T t = __shfl_up(x, off);
    if (l >= off) x += t;
  }
  return x;
}

// Exclusive scan over a whole workgroup of NT threads (NT/64 waves <= 64).
// `lds` needs NT/64 + 1 elements.  Returns the exclusive prefix; *total gets
// the block total.  Contains two barriers.
template <int NT, typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* lds, T* total) {
  constexpr int NWAVES = NT / kWave;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = tid % kWave;
  T inc = wave_inclusive_scan(v);
  if (l == kWave - 1) lds[w] = inc;
  __syncthreads();
  if (w == 0) {
    T t = (l < NWAVES) ? lds[l] : T(0);
    T ti = wave_inclusive_scan(t);
    if (l < NWAVES) lds[l] = ti - t;  // exclusive wave offsets
    if (l == NWAVES - 1) lds[NWAVES] = ti;
  }
  __syncthreads();
  *total = lds[NWAVES];
  return lds[w] + inc - v;
}

}  // namespace hhr
