// Ordered exact top-P inside one workgroup: the P largest scores, ties to the
// lower candidate index, emitted in ascending candidate order.  Internal header.
//
// Layout: candidate c = i*NT + tid sits in register slot i of thread tid, so
// a workgroup's loads of a contiguous score array are coalesced.
//
// The selection is described by a cut-off (T, need_eq) on orderable keys:
// candidate c is taken iff key > T, or key == T and fewer than need_eq keys
// equal to T precede it (in c order).  Two ways find the cut-off:
//   * linear histogram (the usual case): after a block min / max, one pass
//     bins the scores into 2048 bins linear in value -- bin(v) = (int)((v -
//     vmin) * 2048 / (vmax - vmin)) is non-decreasing in v because each step
//     of the float arithmetic is monotone, so a higher bin holds only larger
//     scores -- and the threshold bin b* (count above < P <= count through
//     b*) usually holds a handful of scores, whose exact value ranks give T;
//   * radix select over orderable keys (when b* holds more than 1024 scores,
//     e.g. many equal values): 11-bit digits of key - kmin from the highest
//     bit in which keys differ.
// Then an ordered compaction: wave ballots give ranks inside each (slot,
// wave) group and one scan over the groups gives their offsets.
#pragma once

#include "hhr_device.h"

namespace hhr {

constexpr int kLinBins = 2048;
constexpr int kLinListMax = 1024;
constexpr int kTopMaxGroups = 1024;  // ITEMS * (NT / 64)

struct TopScratch {
  int hist[kLinBins];
  float list_v[kLinListMax];
  int list_n;
  int grp_gt[kTopMaxGroups];
  int grp_eq[kTopMaxGroups];
  float w_min[16], w_max[16];
  int w_n[16];
  uint32_t w_kmin[16], w_kmax[16];
  float vmin, vmax;
  uint32_t kmin, kmax;
  int n_valid, bstar, above, digit;
  uint32_t T;
  int need_eq;
  int scan[17];
};

// Cut-off of the K largest present keys (key 0 = absent), 1 <= K < #present.
template <int NT, int ITEMS>
__device__ void radix_cutoff(const uint32_t (&key)[ITEMS], int K, TopScratch& sh) {
  constexpr int NWAVES = NT / kWave;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = tid % kWave;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    if (key[i] != 0u) {
      mn = min(mn, key[i]);
      mx = max(mx, key[i]);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, off));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
  }
  __syncthreads();
  if (l == 0) {
    sh.w_kmin[w] = mn;
    sh.w_kmax[w] = mx;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t a = 0xFFFFFFFFu, z = 0u;
    for (int k = 0; k < NWAVES; ++k) {
      a = min(a, sh.w_kmin[k]);
      z = max(z, sh.w_kmax[k]);
    }
    sh.kmin = a;
    sh.kmax = z;
  }
  __syncthreads();
  const uint32_t kmin = sh.kmin;
  const uint32_t range = sh.kmax - kmin;
  if (range == 0u) {
    if (tid == 0) {
      sh.T = kmin;
      sh.need_eq = K;
    }
    __syncthreads();
    return;
  }
  const int nbits = 32 - __clz((int)range);
  uint32_t prefix = 0, pmask = 0;
  int remaining = K;
  for (int hi = nbits; hi > 0; hi -= 11) {
    const int width = hi < 11 ? hi : 11;
    const int shift = hi - width;
    const int nb = 1 << width;
    const uint32_t dmask = (uint32_t)nb - 1u;
    __syncthreads();
    for (int i = tid; i < nb; i += NT) sh.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      if (key[i] != 0u) {
        const uint32_t rel = key[i] - kmin;
        if ((rel & pmask) == prefix) atomicAdd(&sh.hist[(rel >> shift) & dmask], 1);
      }
    }
    __syncthreads();
    const int per = (nb + NT - 1) / NT;
    int local = 0;
    for (int j = 0; j < per; ++j) {
      const int d = nb - 1 - (tid * per + j);
      if (d >= 0) local += sh.hist[d];
    }
    int tot;
    int run = block_exclusive_scan<NT, int>(local, sh.scan, &tot);
    for (int j = 0; j < per; ++j) {
      const int d = nb - 1 - (tid * per + j);
      if (d >= 0) {
        const int c = sh.hist[d];
        if (run < remaining && run + c >= remaining) {
          sh.digit = d;
          sh.above = run;
        }
        run += c;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh.digit << shift;
    pmask |= dmask << shift;
    remaining -= sh.above;
  }
  __syncthreads();
  if (tid == 0) {
    sh.T = kmin + prefix;
    sh.need_eq = remaining;
  }
  __syncthreads();
}

// Ordered compaction: emit(pos, c) for every taken candidate, pos ascending in c.
template <int NT, int ITEMS, typename Emit>
__device__ void compact_strided(const uint32_t (&key)[ITEMS], uint32_t T, int need_eq,
                                TopScratch& sh, Emit emit) {
  constexpr int NWAVES = NT / kWave;
  static_assert(ITEMS * NWAVES <= kTopMaxGroups, "too many (slot, wave) groups");
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = tid % kWave;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const uint64_t bgt = __ballot(key[i] != 0u && key[i] > T);
    const uint64_t beq = __ballot(key[i] != 0u && key[i] == T);
    if (l == 0) {
      sh.grp_gt[i * NWAVES + w] = popc64(bgt);
      sh.grp_eq[i * NWAVES + w] = popc64(beq);
    }
  }
  __syncthreads();
  if (w == 0) {
    constexpr int m = ITEMS * NWAVES;
    constexpr int per = (m + kWave - 1) / kWave;
    int a = 0, e = 0;
#pragma unroll
    for (int k = 0; k < per; ++k) {
      const int j = l * per + k;
      if (j < m) {
        a += sh.grp_gt[j];
        e += sh.grp_eq[j];
      }
    }
    int ra = wave_inclusive_scan(a) - a;
    int re = wave_inclusive_scan(e) - e;
#pragma unroll
    for (int k = 0; k < per; ++k) {
      const int j = l * per + k;
      if (j < m) {
        const int ta = sh.grp_gt[j], te = sh.grp_eq[j];
        sh.grp_gt[j] = ra;
        sh.grp_eq[j] = re;
        ra += ta;
        re += te;
      }
    }
  }
  __syncthreads();
  const uint64_t mlt = lanemask_lt();
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const bool gt = key[i] != 0u && key[i] > T;
    const bool eq = key[i] != 0u && key[i] == T;
    const uint64_t bgt = __ballot(gt);
    const uint64_t beq = __ballot(eq);
    const int gt_before = sh.grp_gt[i * NWAVES + w] + popc64(bgt & mlt);
    const int eq_before = sh.grp_eq[i * NWAVES + w] + popc64(beq & mlt);
    if (gt || (eq && eq_before < need_eq))
      emit(gt_before + min(eq_before, need_eq), i * NT + tid);
  }
}

// The min(P, #present) largest of the present scores x[i] (present[i]),
// ties to the lower candidate c = i*NT + tid; emit(pos, c) in ascending c.
// Returns the number selected.  Scores must be finite.
template <int NT, int ITEMS, typename Emit>
__device__ int top_largest_strided(const float (&x)[ITEMS], const bool (&present)[ITEMS], int P,
                                   TopScratch& sh, Emit emit) {
  constexpr int NWAVES = NT / kWave;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = tid % kWave;

  float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    if (present[i]) {
      mn = fminf(mn, x[i]);
      mx = fmaxf(mx, x[i]);
      ++cnt;
    }
  }
  mn = -wave_max(-mn);
  mx = wave_max(mx);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
  if (l == 0) {
    sh.w_min[w] = mn;
    sh.w_max[w] = mx;
    sh.w_n[w] = cnt;
  }
  for (int i = tid; i < kLinBins; i += NT) sh.hist[i] = 0;
  if (tid == 0) sh.list_n = 0;
  __syncthreads();
  if (w == 0) {
    float a = l < NWAVES ? sh.w_min[l] : __builtin_huge_valf();
    float z = l < NWAVES ? sh.w_max[l] : -__builtin_huge_valf();
    int c = l < NWAVES ? sh.w_n[l] : 0;
    a = -wave_max(-a);
    z = wave_max(z);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
    if (l == 0) {
      sh.vmin = a;
      sh.vmax = z;
      sh.n_valid = c;
    }
  }
  __syncthreads();
  const int n_valid = sh.n_valid;
  const int Pe = min(P, n_valid);
  if (Pe <= 0) return 0;

  uint32_t key[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) key[i] = present[i] ? orderable_key(x[i]) : 0u;

  uint32_t T = 0u;  // Pe == n_valid: every present key (>= 0x007FFFFF) is > 0
  int need_eq = 0;
  if (Pe < n_valid) {
    const float vmin = sh.vmin;
    const float range = sh.vmax - vmin;
    const float inv = range > 0.f ? (float)kLinBins / range : 0.f;
    auto bin_of = [&](float v) {
      const float f = (v - vmin) * inv;
      const int bb = f < (float)kLinBins ? (int)f : kLinBins - 1;
      return min(max(bb, 0), kLinBins - 1);
    };
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
      if (present[i]) atomicAdd(&sh.hist[bin_of(x[i])], 1);
    __syncthreads();
    {
      constexpr int PER = kLinBins / NT > 0 ? kLinBins / NT : 1;
      int local = 0;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int d = kLinBins - 1 - (tid * PER + j);
        if (d >= 0) local += sh.hist[d];
      }
      int tot;
      int run = block_exclusive_scan<NT, int>(local, sh.scan, &tot);
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int d = kLinBins - 1 - (tid * PER + j);
        if (d >= 0) {
          const int c = sh.hist[d];
          if (run < Pe && run + c >= Pe) {
            sh.bstar = d;
            sh.above = run;
          }
          run += c;
        }
      }
    }
    __syncthreads();
    const int bstar = sh.bstar;
    const int need = Pe - sh.above;  // 1 <= need <= hist[b*]
    const int cstar = sh.hist[bstar];
    if (cstar <= kLinListMax) {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        if (present[i] && bin_of(x[i]) == bstar) {
          const int slot = atomicAdd(&sh.list_n, 1);
          sh.list_v[slot] = x[i];
        }
      }
      __syncthreads();
      // T = the value with (#greater in b*) < need <= (#greater) + (#equal)
      for (int j = tid; j < cstar; j += NT) {
        const float vj = sh.list_v[j];
        int gtr = 0, eql = 0;
        for (int k = 0; k < cstar; ++k) {
          const float vk = sh.list_v[k];
          gtr += vk > vj;
          eql += vk == vj;
        }
        if (gtr < need && need <= gtr + eql) {  // all equal copies agree
          sh.T = orderable_key(vj);
          sh.need_eq = need - gtr;
        }
      }
      __syncthreads();
      T = sh.T;
      need_eq = sh.need_eq;
    } else {
      radix_cutoff<NT, ITEMS>(key, Pe, sh);
      T = sh.T;
      need_eq = sh.need_eq;
    }
  }
  compact_strided<NT, ITEMS>(key, T, need_eq, sh, emit);
  return Pe;
}

}  // namespace hhr
