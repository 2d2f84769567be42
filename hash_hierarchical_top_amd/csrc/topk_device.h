// Ordered exact top-P inside one workgroup: the P largest keys, ties to the
// lower candidate index, emitted in ascending candidate order.  Internal header.
#pragma once

#include "hhr_device.h"

namespace hhr {

struct TopScratch {
  int hist[256];
  int digit, above, valid;
  long long scan[17];
};

// Digit d* (one wave): count(digits > d*) < remaining <= count(digits >= d*).
__device__ __forceinline__ void find_digit_desc(const int* hist, int remaining, int* out_digit,
                                                int* out_above) {
  const int l = threadIdx.x & 63;
  int local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) local += hist[255 - 4 * l - i];
  const int excl = wave_inclusive_scan(local) - local;
  int run = excl;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = 255 - 4 * l - i;
    const int c = hist[d];
    if (run < remaining && run + c >= remaining) {
      *out_digit = d;
      *out_above = run;
    }
    run += c;
  }
}

// Candidates c = tid*items + i (i < items) hold key[i]; key 0 marks "absent"
// (orderable_key() of any non-NaN float is >= 0x007FFFFF).  Selects the
// min(P, #present) largest present keys, ties to the lower c, and calls
// emit(pos, c) with pos = rank of c among the selected in ascending c.
// Returns the number selected.  Radix select: four 8-bit digits, most
// significant first; then an ordered block scan.  NT threads, NT <= 1024.
template <int NT, int ITEMS, typename Emit>
__device__ int top_largest_ordered(const uint32_t (&key)[ITEMS], int items, int P,
                                   TopScratch& sh, Emit emit) {
  const int tid = threadIdx.x;
  const int i0 = tid * items;
  int present = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) present += (i < items && key[i] != 0u);
  long long tot;
  block_exclusive_scan<NT, long long>((long long)present, sh.scan, &tot);
  const int n_valid = (int)tot;
  const int Pe = min(P, n_valid);
  if (Pe <= 0) return 0;

  uint32_t T = 0;  // select key > T, and key == T among the first need_eq
  int need_eq = 0;
  if (Pe < n_valid) {
    uint32_t prefix = 0, pmask = 0;
    int remaining = Pe;
    for (int shift = 24; shift >= 0; shift -= 8) {
      __syncthreads();
      for (int i = tid; i < 256; i += NT) sh.hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < ITEMS; ++i)
        if (i < items && key[i] != 0u && (key[i] & pmask) == prefix)
          atomicAdd(&sh.hist[(key[i] >> shift) & 255], 1);
      __syncthreads();
      if (tid < kWave) find_digit_desc(sh.hist, remaining, &sh.digit, &sh.above);
      __syncthreads();
      prefix |= (uint32_t)sh.digit << shift;
      pmask |= 255u << shift;
      remaining -= sh.above;
    }
    T = prefix;
    need_eq = remaining;
  }

  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    if (i < items && key[i] != 0u) {
      gt += key[i] > T;
      eq += key[i] == T;
    }
  }
  __syncthreads();
  const long long ex =
      block_exclusive_scan<NT, long long>(((long long)gt << 32) | (long long)eq, sh.scan, &tot);
  const int gt_before = (int)(ex >> 32);
  const int eq_before = (int)(ex & 0xFFFFFFFFll);
  int pos = gt_before + min(eq_before, need_eq);
  int eq_seen = eq_before;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    if (i < items && key[i] != 0u) {
      bool take = key[i] > T;
      if (key[i] == T) {
        take = eq_seen < need_eq;
        ++eq_seen;
      }
      if (take) emit(pos++, i0 + i);
    }
  }
  return Pe;
}

}  // namespace hhr
