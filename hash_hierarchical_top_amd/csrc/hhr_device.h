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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// f32 -> bf16 bits of a (low half) and b (high half), rounded to nearest
// even: one v_cvt_pk_bf16_f32 (finite inputs).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  return f32x2_to_bf16x2_rne(x, 0.f) & 0xFFFFu;
}

// Split x into bf16 hi + lo with x - hi - lo within 2^-17 |x| (x - hi is
// exact in f32).
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_rne(x);
  lo = f32_to_bf16_rne(x - bf16_to_f32(hi));
}
// The same for a pair, packed as the MFMA operands hold them (a low, b high):
// {hi, lo}.
__device__ __forceinline__ u32x2 split_bf16x2(float a, float b) {
  const uint32_t hi = f32x2_to_bf16x2_rne(a, b);
  return u32x2{hi, f32x2_to_bf16x2_rne(a - __uint_as_float(hi << 16),
                                       b - __uint_as_float(hi & 0xFFFF0000u))};
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// min / max by med3 against an infinity: med3(x, y, -inf) = min(x, y) and
// med3(x, y, +inf) = max(x, y) for non-NaN x, y.  v_med3 needs no NaN
// canonicalisation of its operands, which IEEE-mode minnum / maxnum add.  The
// infinity must come from opaque_inf(): a literal would let the compiler fold
// med3 back into minnum / maxnum.
__device__ __forceinline__ float opaque_inf() {
  float r;
  asm volatile("v_mov_b32 %0, 0x7f800000" : "=v"(r));
  return r;
}
__device__ __forceinline__ float med_min(float a, float b, float inf) {
  return __builtin_amdgcn_fmed3f(a, b, -inf);
}
__device__ __forceinline__ float med_max(float a, float b, float inf) {
  return __builtin_amdgcn_fmed3f(a, b, inf);
}

// gfx950 lane swaps: with both operands x, v_permlane32_swap leaves {x[l],
// x[l ^ 32]} in the two results of every lane l, v_permlane16_swap {x[l],
// x[l ^ 16]}.  One VALU instruction each, no LDS.
__device__ __forceinline__ float fmin_swap32(float x, float inf) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return med_min(__uint_as_float(p[0]), __uint_as_float(p[1]), inf);
}
__device__ __forceinline__ float fmax_swap32(float x, float inf) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return med_max(__uint_as_float(p[0]), __uint_as_float(p[1]), inf);
}
__device__ __forceinline__ float fmin_swap16(float x, float inf) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return med_min(__uint_as_float(p[0]), __uint_as_float(p[1]), inf);
}
__device__ __forceinline__ float fmax_swap16(float x, float inf) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return med_max(__uint_as_float(p[0]), __uint_as_float(p[1]), inf);
}
__device__ __forceinline__ uint32_t or_swap32(uint32_t x) {
  const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return p[0] | p[1];
}
__device__ __forceinline__ uint32_t or_swap16(uint32_t x) {
  const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return p[0] | p[1];
}

// Directed rounding f32 -> bf16 bits.  A bf16 value is the upper half of an
// f32 pattern, so dropping the lower half rounds the magnitude down (toward
// zero).  Rounding toward -inf is that for x >= 0 and one step up in magnitude
// for negative x with a nonzero lower half; toward +inf the other way round.
// Past the largest finite bf16 the step lands on the infinity of that sign;
// infinities stay as they are.  Inputs are never NaN here.
__device__ __forceinline__ uint32_t f32_to_bf16_down(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u >> 16) + ((u >> 31) & ((u & 0xFFFFu) != 0u));
}
__device__ __forceinline__ uint32_t f32_to_bf16_up(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u >> 16) + ((~u >> 31) & ((u & 0xFFFFu) != 0u));
}

// Monotone map f32 -> u32 (larger float -> larger key); -0 is folded onto +0.
__device__ __forceinline__ uint32_t orderable_key(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Cross-lane exchanges use DPP (a VALU operand modifier, a few cycles) rather
// than __shfl (an LDS permute, ~100 cycles).  gfx9 DPP controls: quad_perm,
// row_shr:n (lane i of a 16-lane row reads lane i-n, zero past the row
// start), row_half_mirror / row_mirror (lane j of 8 / 16 reads lane 7-j /
// 15-j), row_bcast:15 / :31 (lane 15 / 31 feeds the following rows).  Every
// wave op here needs all 64 lanes active.
namespace dpp {
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowShr = 0x110;   // + n, 1 <= n <= 15
constexpr int kRowMirror = 0x140;
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;
}  // namespace dpp

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}
__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Butterfly inside each 16-lane row, then the four row results combined in
// scalar registers; every lane returns the same bits.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<dpp::kQuadXor1>(v);
  v += dpp_f<dpp::kQuadXor2>(v);
  v += dpp_f<dpp::kRowHalfMirror>(v);
  v += dpp_f<dpp::kRowMirror>(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

// Sum over the 16 lanes of each row; every lane of the row gets the same bits.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<dpp::kQuadXor1>(v);
  v += dpp_f<dpp::kQuadXor2>(v);
  v += dpp_f<dpp::kRowHalfMirror>(v);
  v += dpp_f<dpp::kRowMirror>(v);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<dpp::kQuadXor1>(v));
  v = fmaxf(v, dpp_f<dpp::kQuadXor2>(v));
  v = fmaxf(v, dpp_f<dpp::kRowHalfMirror>(v));
  v = fmaxf(v, dpp_f<dpp::kRowMirror>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)),
               fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

__device__ __forceinline__ float wave_min(float v) { return -wave_max(-v); }

__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_i<dpp::kQuadXor1>(v);
  v += dpp_i<dpp::kQuadXor2>(v);
  v += dpp_i<dpp::kRowHalfMirror>(v);
  v += dpp_i<dpp::kRowMirror>(v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) {
  int x = (int)v;
  x = (int)min((uint32_t)x, (uint32_t)dpp_i<dpp::kQuadXor1>(x));
  x = (int)min((uint32_t)x, (uint32_t)dpp_i<dpp::kQuadXor2>(x));
  x = (int)min((uint32_t)x, (uint32_t)dpp_i<dpp::kRowHalfMirror>(x));
  x = (int)min((uint32_t)x, (uint32_t)dpp_i<dpp::kRowMirror>(x));
  return min(min((uint32_t)__builtin_amdgcn_readlane(x, 0), (uint32_t)__builtin_amdgcn_readlane(x, 16)),
             min((uint32_t)__builtin_amdgcn_readlane(x, 32), (uint32_t)__builtin_amdgcn_readlane(x, 48)));
}

__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
  int x = (int)v;
  x = (int)max((uint32_t)x, (uint32_t)dpp_i<dpp::kQuadXor1>(x));
  x = (int)max((uint32_t)x, (uint32_t)dpp_i<dpp::kQuadXor2>(x));
  x = (int)max((uint32_t)x, (uint32_t)dpp_i<dpp::kRowHalfMirror>(x));
  x = (int)max((uint32_t)x, (uint32_t)dpp_i<dpp::kRowMirror>(x));
  return max(max((uint32_t)__builtin_amdgcn_readlane(x, 0), (uint32_t)__builtin_amdgcn_readlane(x, 16)),
             max((uint32_t)__builtin_amdgcn_readlane(x, 32), (uint32_t)__builtin_amdgcn_readlane(x, 48)));
}

__device__ __forceinline__ int popc64(uint64_t x) { return __popcll(x); }

// Set bits of the wave-uniform mask m below this lane.
__device__ __forceinline__ uint32_t mbcnt64(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive scan across the wave (32-bit integers): Hillis-Steele inside
// each 16-lane row with row_shr 1, 2, 4, 8, then row totals carried forward
// with row_bcast:15 (rows 1, 3) and row_bcast:31 (rows 2, 3).
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T x) {
  static_assert(sizeof(T) == 4, "32-bit scan");
  int v = __builtin_bit_cast(int, x);
  v += dpp_i<dpp::kRowShr + 1>(v);
  v += dpp_i<dpp::kRowShr + 2>(v);
  v += dpp_i<dpp::kRowShr + 4>(v);
  v += dpp_i<dpp::kRowShr + 8>(v);
  v += dpp_i<dpp::kRowBcast15, 0xA>(v);
  v += dpp_i<dpp::kRowBcast31, 0xC>(v);
  return __builtin_bit_cast(T, v);
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

// ---------------------------------------------------------------- coherence
// Data handed from one workgroup to another inside a kernel crosses XCDs,
// whose L2 caches are not coherent with each other.  A device-scope fence
// (__threadfence) writes back and invalidates a whole L2, which costs tens of
// microseconds when every workgroup does it; instead such data is written
// and read with agent-scope (sc1) accesses, which the L2 does not hold stale,
// and a producer publishes with s_waitcnt(0) + a relaxed agent-scope atomic.
// Mem<false> is the plain path for data that only crosses kernel boundaries.
//
// Why the relaxed hand-off (arrive_last) is ordered.  The HIP memory model
// would express it as a release (producer) and an acquire (consumer) at agent
// scope; on this part those compile to an L2 writeback (release) and an L2
// invalidate (acquire) around the atomic, which only matter for data that may
// sit in an L2 line: data written by plain stores (dirty in the producer's
// XCD's L2) or read by plain loads (possibly stale in the consumer's).  Every
// value handed over inside a launch here is written with agent-scope stores
// and read with agent-scope loads (Mem<true>, ld_sc1_x4): such accesses are
// performed at the memory side, never through a stale or dirty L2 line, so
// there is nothing to write back or invalidate.  What remains is completion
// order: each producer wave waits with s_waitcnt(0) until its agent-scope
// stores are acknowledged (performed at the memory side), the workgroup meets
// at a barrier (which the compiler does not move memory accesses across),
// and only then does one thread add to the counter with an agent-scope
// atomic, itself performed at the memory side after those stores.  The
// workgroup that reads the final count therefore issues its agent-scope
// loads after every producer's stores were performed.  Nobody waits for
// anybody: the last arriver is the one that finds all the others done, so
// there is no scheduling hazard either.
template <bool COH>
struct Mem {
  template <typename T>
  static __device__ __forceinline__ T ld(const T* p) {
    if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *p;
  }
  template <typename T>
  static __device__ __forceinline__ void st(T* p, T v) {
    if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
  }
};

__device__ __forceinline__ uint32_t ld_agent_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_agent_u32(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A compiler-only barrier for memory operations (no instruction, no wait):
// loads written before it are issued before it.  Used after a batch of
// independent loads whose values are consumed under conditions, which the
// compiler would otherwise turn into one branch per load, each load waited
// for on its own before the next is issued.
__device__ __forceinline__ void issue_loads_here() { asm volatile("" ::: "memory"); }

// Wait until every memory access this wave issued has completed.
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Publishes this workgroup's agent-scope stores and counts it in on *counter;
// returns its place in the arrival order (0 = first, n_wg - 1 = last; the
// last also puts the counter back to zero for the next call).  All threads
// call.
__device__ __forceinline__ uint32_t arrive_order(uint32_t* counter, uint32_t n_wg,
                                                 uint32_t* s_order) {
  wait_all_mem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = add_agent_u32(counter, 1u);
    *s_order = prev;
    if (prev == n_wg - 1u) st_agent_u32(counter, 0u);
  }
  __syncthreads();
  return *s_order;
}

// Publishes this workgroup's agent-scope stores and counts it in on *counter;
// true in the workgroup that arrives last (n_wg arrivals), which also puts the
// counter back to zero for the next call.  All threads call.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t n_wg, int* s_last) {
  wait_all_mem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = add_agent_u32(counter, 1u);
    *s_last = prev == n_wg - 1u;
    if (*s_last) st_agent_u32(counter, 0u);
  }
  __syncthreads();
  return *s_last != 0;
}

}  // namespace hhr

