// Ordered exact top-P inside one workgroup: the P largest scores, ties to the
// lower candidate index, emitted in ascending candidate order.  Internal header.
//
// Layout: the scores sit in LDS; thread tid owns a run of consecutive
// candidates, read as float4, so the whole selection works from registers and
// the output order follows from one block scan.
//
// The selection is described by a cut-off (T, need_eq) on orderable keys:
// candidate c is taken iff key > T, or key == T and fewer than need_eq keys
// equal to T precede it (in c order).  Two ways find the cut-off:
//   * linear histogram (the usual case): after a block min / max, one pass
//     bins the scores into 2048 bins linear in value -- bin(v) = (int)((v -
//     vmin) * 2048 / (vmax - vmin)) is non-decreasing in v because each step
//     of the float arithmetic is monotone, so a higher bin holds only larger
//     scores.  If the whole threshold bin b* (count above < P <= count
//     through b*) is taken, the cut is "bin >= b*"; otherwise b* usually
//     holds a handful of scores, whose exact value ranks give T;
//   * radix select over orderable keys (when b* holds more than
//     kLinListMax scores, e.g. many equal values): 11-bit digits of
//     key - kmin from the highest bit in which keys differ.
// Then an ordered compaction over the per-thread runs: each thread counts
// its taken candidates (strictly inside the cut, and on it) and one block
// scan of the packed pair gives every run its output offset.
#pragma once

#include "hhr_device.h"

namespace hhr {

constexpr int kLinBins = 2048;
constexpr int kLinListMax = 512;

constexpr int kStridedCnt = 256;  // (slot, wave) counts of top_largest_strided

struct TopScratch {
  int hist[kLinBins];
  uint32_t cnt[kStridedCnt];
  float list_v[kLinListMax];
  int list_n;
  float w_min[16], w_max[16];
  int w_n[16];
  uint32_t w_kmin[16], w_kmax[16];
  uint32_t kmin, kmax;
  int bstar, above, digit;
  uint32_t T;
  int need_eq;
  int scan[17];
  uint32_t uscan[17];
};

// Cut-off of the K largest present keys (key 0 = absent), 1 <= K < #present.
// key_of(i) gives this thread's key i of n_items (the loops stay rolled: this
// runs once per selection, so small code matters more than loop overhead).
template <int NT, typename KeyOf>
__device__ void radix_cutoff(KeyOf key_of, int n_items, int K, TopScratch& sh) {
  constexpr int NWAVES = NT / kWave;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = tid % kWave;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll 1
  for (int i = 0; i < n_items; ++i) {
    const uint32_t k = key_of(i);
    if (k != 0u) {
      mn = min(mn, k);
      mx = max(mx, k);
    }
  }
  mn = wave_min_u(mn);
  mx = wave_max_u(mx);
  __syncthreads();
  if (l == 0) {
    sh.w_kmin[w] = mn;
    sh.w_kmax[w] = mx;
  }
  __syncthreads();
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll 1
  for (int k = 0; k < NWAVES; ++k) {
    kmin = min(kmin, sh.w_kmin[k]);
    kmax = max(kmax, sh.w_kmax[k]);
  }
  const uint32_t range = kmax - kmin;
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
#pragma unroll 1
  for (int hi = nbits; hi > 0; hi -= 11) {
    const int width = hi < 11 ? hi : 11;
    const int shift = hi - width;
    const int nb = 1 << width;
    const uint32_t dmask = (uint32_t)nb - 1u;
    __syncthreads();
    for (int i = tid; i < nb; i += NT) sh.hist[i] = 0;
    __syncthreads();
#pragma unroll 1
    for (int i = 0; i < n_items; ++i) {
      const uint32_t k = key_of(i);
      if (k != 0u) {
        const uint32_t rel = k - kmin;
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

// Output offsets of this thread's run in an ordered compaction: gt and eq
// count the run's candidates strictly inside the cut and on it; returns the
// counts over all earlier runs (one block scan of gt | eq << 16: both totals
// stay below 65536).
template <int NT>
__device__ __forceinline__ void run_offsets(int gt, int eq, TopScratch& sh, int& gt0, int& eq0) {
  uint32_t tot;
  const uint32_t ex =
      block_exclusive_scan<NT, uint32_t>((uint32_t)gt | ((uint32_t)eq << 16), sh.uscan, &tot);
  gt0 = (int)(ex & 0xFFFFu);
  eq0 = (int)(ex >> 16);
}

// Emits one candidate of a run in order: cls 1 = inside the cut (always
// taken), 2 = on the cut (taken while fewer than need_eq on-cut candidates
// precede it).  The output slot is the number of taken candidates before it.
template <typename Emit>
__device__ __forceinline__ void emit_ordered(int cls, int c, int need_eq, int& gb, int& eb,
                                             Emit& emit) {
  const bool take = cls == 1 || (cls == 2 && eb < need_eq);
  if (take) emit(gb + min(eb, need_eq), c);
  gb += cls == 1 ? 1 : 0;
  eb += cls == 2 ? 1 : 0;
}

// The min(P, #present) largest present scores of sbuf[0..n), ties to the
// lower index; emit(pos, c) for each taken candidate c, pos = its rank in
// ascending c.  present(c) tells whether candidate c < n exists.  Thread tid
// owns candidates [4*nv4*tid, 4*nv4*(tid+1)) with nv4 = ceil(n / (4*NT)) <=
// MAXV4; sbuf must hold 4*NT*MAXV4 floats, 16-byte aligned (slots past n are
// read but never used).  Scores must be finite (-0 counts as +0).  Returns
// the number taken.  All threads call.
//
// Every pass over the data is vector-throughput bound on one CU, so each
// slot's bin is computed once and kept in registers (16 bits per slot):
// the cut is then decided from the bins, and only members of the threshold
// bin compare values.
template <int NT, int MAXV4, typename Present, typename Emit>
__device__ int top_largest_ranged(const float* sbuf, int n, Present present, int P, float vmin,
                                  float vmax, int n_valid, TopScratch& sh, Emit emit,
                                  bool hist_clear = false);

template <int NT, int MAXV4, typename Present, typename Emit>
__device__ int top_largest_lds(const float* sbuf, int n, Present present, int P, TopScratch& sh,
                               Emit emit) {
  constexpr int NWAVES = NT / kWave;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = tid % kWave;
  const int nv4 = (n + 4 * NT - 1) / (4 * NT);
  const int c0 = 4 * nv4 * tid;
  const float4* run4 = reinterpret_cast<const float4*>(sbuf) + nv4 * tid;
  auto val = [&](const float4& t, int e) { return e == 0 ? t.x : e == 1 ? t.y : e == 2 ? t.z : t.w; };

  float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < MAXV4; ++j) {
    if (j < nv4) {
      const float4 t = run4[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = c0 + 4 * j + e;
        if (c < n && present(c)) {
          mn = fminf(mn, val(t, e));
          mx = fmaxf(mx, val(t, e));
          ++cnt;
        }
      }
    }
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  cnt = wave_sum_i(cnt);
  if (l == 0) {
    sh.w_min[w] = mn;
    sh.w_max[w] = mx;
    sh.w_n[w] = cnt;
  }
  __syncthreads();
  float vmin = __builtin_huge_valf(), vmax = -__builtin_huge_valf();
  int n_valid = 0;
#pragma unroll
  for (int k = 0; k < NWAVES; ++k) {
    vmin = fminf(vmin, sh.w_min[k]);
    vmax = fmaxf(vmax, sh.w_max[k]);
    n_valid += sh.w_n[k];
  }
  return top_largest_ranged<NT, MAXV4>(sbuf, n, present, P, vmin, vmax, n_valid, sh, emit);
}

// The same selection with the range of the present scores given: vmin <=
// every present score <= vmax, and n_valid = #present.  Each thread reads only
// its own run of sbuf, so a caller that writes its own run needs no barrier
// before the call.  hist_clear: the caller has already zeroed sh.hist and
// sh.list_n before a barrier (saving a barrier here).
template <int NT, int NV4, typename Present, typename Emit>
__device__ int top_largest_fixed(const float* sbuf, int n, Present present, int P, float vmin,
                                 float vmax, int n_valid, TopScratch& sh, Emit& emit,
                                 bool hist_clear);

// Dispatch on the run length nv4 = ceil(n / (4 NT)) (block-uniform), so that
// every per-slot loop is exactly as long as the live run: these passes are
// vector-throughput bound, and dead slots cost as much as live ones.
template <int NT, int MAXV4, typename Present, typename Emit>
__device__ int top_largest_ranged(const float* sbuf, int n, Present present, int P, float vmin,
                                  float vmax, int n_valid, TopScratch& sh, Emit emit,
                                  bool hist_clear) {
  static_assert(MAXV4 >= 1 && MAXV4 <= 8, "run length");
  const int nv4 = max((n + 4 * NT - 1) / (4 * NT), 1);
#define HHR_TOP_CASE(k)                                                                      \
  if (MAXV4 >= (k) && nv4 == (k))                                                            \
    return top_largest_fixed<NT, ((k) <= MAXV4 ? (k) : 1)>(sbuf, n, present, P, vmin, vmax, \
                                                           n_valid, sh, emit, hist_clear);
  HHR_TOP_CASE(1)
  HHR_TOP_CASE(2)
  HHR_TOP_CASE(3)
  HHR_TOP_CASE(4)
  HHR_TOP_CASE(5)
  HHR_TOP_CASE(6)
  HHR_TOP_CASE(7)
  HHR_TOP_CASE(8)
#undef HHR_TOP_CASE
  return 0;  // unreachable for n <= 4 NT MAXV4
}

template <int NT, int NV4, typename Present, typename Emit>
__device__ int top_largest_fixed(const float* sbuf, int n, Present present, int P, float vmin,
                                 float vmax, int n_valid, TopScratch& sh, Emit& emit,
                                 bool hist_clear) {
  constexpr int MAXV4 = NV4;
  constexpr int MAXV = 4 * MAXV4;
  static_assert(MAXV <= 32, "2 class bits per slot in 64 bits");
  constexpr uint32_t kAbsent = 0xFFFFu;  // bin code of an absent slot
  const int tid = threadIdx.x;
  constexpr int nv4 = NV4;
  const int c0 = 4 * nv4 * tid;
  const float4* run4 = reinterpret_cast<const float4*>(sbuf) + nv4 * tid;
  auto val = [&](const float4& t, int e) { return e == 0 ? t.x : e == 1 ? t.y : e == 2 ? t.z : t.w; };
  auto is_present = [&](int c) { return c < n && present(c); };

  const int Pe = min(P, n_valid);
  if (Pe <= 0) return 0;  // block-uniform
  if (!hist_clear) {
    for (int i = tid; i < kLinBins; i += NT) sh.hist[i] = 0;
    if (tid == 0) sh.list_n = 0;
    __syncthreads();
  }

  // bins: bin(v) = (int)((v - vmin) * 2048 / (vmax - vmin)) is monotone in v
  const float range = vmax - vmin;
  const float inv = range > 0.f ? (float)kLinBins / range : 0.f;
  uint32_t bins[MAXV / 2];  // two 16-bit bin codes per word
  const bool all = Pe >= n_valid;
#pragma unroll
  for (int j = 0; j < MAXV4; ++j) {
    uint32_t b4[4];
    if (j < nv4) {
      const float4 t = run4[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t bb = kAbsent;
        if (is_present(c0 + 4 * j + e)) {
          const float f = (val(t, e) - vmin) * inv;
          bb = (uint32_t)min(max(f < (float)kLinBins ? (int)f : kLinBins - 1, 0), kLinBins - 1);
          if (!all) atomicAdd(&sh.hist[bb], 1);
        }
        b4[e] = bb;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) b4[e] = kAbsent;
    }
    bins[2 * j] = b4[0] | (b4[1] << 16);
    bins[2 * j + 1] = b4[2] | (b4[3] << 16);
  }
  auto bin_at = [&](int i) { return (bins[i >> 1] >> (16 * (i & 1))) & 0xFFFFu; };

  // cut-off: mode 0 = every present slot, 1 = bin >= bstar, 2 = bin > bstar or
  // (bin == bstar and key >= T, ties by need_eq)
  int mode = 0, need_eq = 0;
  uint32_t bstar = 0, T = 0u;
  if (!all) {
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
    bstar = (uint32_t)sh.bstar;
    const int need = Pe - sh.above;  // 1 <= need <= hist[b*]
    const int cstar = sh.hist[bstar];
    if (need == cstar) {
      mode = 1;
    } else if (cstar <= kLinListMax) {
      mode = 2;
#pragma unroll
      for (int i = 0; i < MAXV; ++i)
        if (bin_at(i) == bstar) sh.list_v[atomicAdd(&sh.list_n, 1)] = sbuf[c0 + i];
      __syncthreads();
      // T = the value with (#greater in b*) < need <= (#greater) + (#equal)
      for (int j = tid; j < cstar; j += NT) {
        const float vj = sh.list_v[j];
        int gtr = 0, eql = 0;
#pragma unroll 1
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
      mode = 3;  // radix over the keys of the whole set
      radix_cutoff<NT>(
          [&](int i) -> uint32_t {
            const int c = c0 + i;
            return is_present(c) ? orderable_key(sbuf[c]) : 0u;
          },
          4 * nv4, Pe, sh);
      T = sh.T;
      need_eq = sh.need_eq;
    }
  }
  // classify each slot once (2 bits: 1 = inside the cut, 2 = on it)
  uint64_t cls = 0;
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const uint32_t bb = bin_at(i);
    int k = 0;
    if (bb != kAbsent) {
      if (mode == 0) {
        k = 1;
      } else if (mode == 1) {
        k = bb >= bstar ? 1 : 0;
      } else if (mode == 2 && bb != bstar) {
        k = bb > bstar ? 1 : 0;
      } else {  // key comparison: mode 3, or a member of the threshold bin
        const uint32_t key = orderable_key(sbuf[c0 + i]);
        k = key > T ? 1 : (key == T ? 2 : 0);
      }
    }
    cls |= (uint64_t)k << (2 * i);
    gt += k == 1;
    eq += k == 2;
  }
  int gb, eb;
  run_offsets<NT>(gt, eq, sh, gb, eb);
#pragma unroll 1
  for (int i = 0; i < 4 * nv4; ++i) {
    const int k = (int)(cls >> (2 * i)) & 3;
    if (k != 0) emit_ordered(k, c0 + i, need_eq, gb, eb, emit);
  }
  return Pe;
}

// ---------------------------------------------------------------------------
// The same selection with the scores in registers and strided ownership:
// thread t of NT holds candidate j NT + t in x[j] (j < NV), the layout that
// coalesced loads give, so the scores are never staged through LDS.  Output
// positions come from per-slot wave ballots (a lane's rank among the wave's
// taken candidates of slot j) and one exclusive prefix over the (slot, wave)
// counts, whose order j, wave, lane is the candidate order.  This costs a few
// vector instructions per candidate where the run-based compaction spends
// tens, and the top-P of one (b, g) runs on a single CU bound by its vector
// throughput.  vmin <= every score <= vmax; sh.hist and sh.list_n must be
// zero behind a barrier; sbuf (4 NT NV floats in LDS) is used only by the
// radix fallback.  Candidates c >= n are absent.  Returns min(P, n).  All NT
// threads call.
template <int NT, int NV, typename Emit>
__device__ int top_largest_strided(const float (&x)[NV], int n, int P, float vmin, float vmax,
                                   float* sbuf, TopScratch& sh, Emit& emit) {
  constexpr int NWAVES = NT / kWave;
  constexpr int NE = NV * NWAVES;  // (slot, wave) entries
  static_assert(NE <= kStridedCnt, "slot counts fit TopScratch::cnt");
  constexpr int PER = (NE + kWave - 1) / kWave;
  static_assert(PER <= 4, "at most 4 entries per lane");
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l = tid % kWave;
  const int Pe = min(P, n);
  if (Pe <= 0) return 0;  // block-uniform
  const bool all = Pe >= n;

  // bins, linear in value: bin(v) = (int)((v - vmin) * 2048 / (vmax - vmin)),
  // non-decreasing in v; -1 for an absent candidate
  const float range = vmax - vmin;
  const float inv = range > 0.f ? (float)kLinBins / range : 0.f;
  int bin[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const float f = (x[j] - vmin) * inv;
    const int bb = f < (float)kLinBins ? max((int)f, 0) : kLinBins - 1;
    const bool present = j * NT + tid < n;
    bin[j] = present ? bb : -1;
    if (present && !all) atomicAdd(&sh.hist[bb], 1);
  }

  // cut-off: mode 0 = every present candidate, 1 = bin >= bstar, 2 = bin >
  // bstar or (bin == bstar and key >= T, ties by need_eq), 3 = key >= T
  int mode = 0, need_eq = 0, bstar = 0;
  uint32_t T = 0u;
  if (!all) {
    __syncthreads();
    {
      constexpr int PERB = kLinBins / NT > 0 ? kLinBins / NT : 1;
      int local = 0;
#pragma unroll
      for (int j = 0; j < PERB; ++j) {
        const int d = kLinBins - 1 - (tid * PERB + j);
        if (d >= 0) local += sh.hist[d];
      }
      int tot;
      int run = block_exclusive_scan<NT, int>(local, sh.scan, &tot);
#pragma unroll
      for (int j = 0; j < PERB; ++j) {
        const int d = kLinBins - 1 - (tid * PERB + j);
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
    bstar = sh.bstar;
    const int need = Pe - sh.above;  // 1 <= need <= hist[b*]
    const int cstar = sh.hist[bstar];
    if (need == cstar) {
      mode = 1;
    } else if (cstar <= kLinListMax) {
      mode = 2;
#pragma unroll
      for (int j = 0; j < NV; ++j)
        if (bin[j] == bstar) sh.list_v[atomicAdd(&sh.list_n, 1)] = x[j];
      __syncthreads();
      // T = the value with (#greater in b*) < need <= (#greater) + (#equal)
      for (int j = tid; j < cstar; j += NT) {
        const float vj = sh.list_v[j];
        int gtr = 0, eql = 0;
#pragma unroll 1
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
      mode = 3;  // radix over the keys of the whole set, read back from LDS
#pragma unroll
      for (int j = 0; j < NV; ++j) sbuf[j * NT + tid] = x[j];
      __syncthreads();
      radix_cutoff<NT>(
          [&](int i) -> uint32_t {
            const int c = i * NT + tid;
            return c < n ? orderable_key(sbuf[c]) : 0u;
          },
          NV, Pe, sh);
      T = sh.T;
      need_eq = sh.need_eq;
    }
  }

  // classes (1 = inside the cut, 2 = on it) and each lane's rank among its
  // wave's candidates of the same class and slot
  int cls[NV];
  uint32_t rank[NV];  // rank in class 1 | rank in class 2 << 16
  const uint64_t below = lanemask_lt();
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    int k = 0;
    if (bin[j] >= 0) {
      if (mode == 0) {
        k = 1;
      } else if (mode == 1) {
        k = bin[j] >= bstar ? 1 : 0;
      } else if (mode == 2 && bin[j] != bstar) {
        k = bin[j] > bstar ? 1 : 0;
      } else {
        const uint32_t key = orderable_key(x[j]);
        k = key > T ? 1 : (key == T ? 2 : 0);
      }
    }
    cls[j] = k;
    const uint64_t b1 = __ballot(k == 1);
    const uint64_t b2 = __ballot(k == 2);
    rank[j] = (uint32_t)popc64(b1 & below) | ((uint32_t)popc64(b2 & below) << 16);
    if (l == 0) sh.cnt[j * NWAVES + w] = (uint32_t)popc64(b1) | ((uint32_t)popc64(b2) << 16);
  }
  __syncthreads();
  // exclusive prefix over entries e = j NWAVES + w (lane l holds entries
  // PER l .. PER l + PER - 1); both 16-bit halves stay below 65536
  uint32_t pre[PER];
  {
    uint32_t v[PER], local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = PER * l + i;
      v[i] = e < NE ? sh.cnt[e] : 0u;
      local += v[i];
    }
    uint32_t run = wave_inclusive_scan(local) - local;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      pre[i] = run;
      run += v[i];
    }
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e = j * NWAVES + w;  // wave-uniform
    const int r = e % PER;
    uint32_t p = pre[0];
#pragma unroll
    for (int i = 1; i < PER; ++i)
      if (r == i) p = pre[i];
    const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)p, e / PER) + rank[j];
    const int gb = (int)(base & 0xFFFFu), eb = (int)(base >> 16);
    if (cls[j] == 1 || (cls[j] == 2 && eb < need_eq)) emit(gb + min(eb, need_eq), j * NT + tid);
  }
  return Pe;
}

}  // namespace hhr
