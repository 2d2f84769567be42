// Ordered exact top-P inside one workgroup: the P largest scores, ties to the
// lower candidate index, emitted in ascending candidate order.  Internal header.
//
// Layout: thread t of NT holds candidates j NT + t (j < NV) in registers, the
// layout that coalesced loads give, so the scores are never staged through
// LDS; the selection is bound by one CU's vector throughput, so it spends as
// few instructions per candidate as it can.
//
// The selection is described by a cut-off (T, need_eq) on orderable keys:
// candidate c is taken iff key > T, or key == T and fewer than need_eq keys
// equal to T precede it (in c order).  Two ways find the cut-off:
//   * linear histogram (the usual case): given the range [vmin, vmax], one
//     pass bins the scores into 2048 bins linear in value -- bin(v) = (int)((v
//     - vmin) * 2048 / (vmax - vmin)) is non-decreasing in v because each step
//     of the float arithmetic is monotone, so a higher bin holds only larger
//     scores.  If the whole threshold bin b* (count above < P <= count
//     through b*) is taken, the cut is "bin >= b*"; otherwise b* usually
//     holds a handful of scores, whose exact value ranks give T;
//   * radix select over orderable keys (when b* holds more than
//     kLinListMax scores, e.g. many equal values): 11-bit digits of
//     key - kmin from the highest bit in which keys differ.
// Output positions come from per-slot wave ballots and one prefix over the
// (slot, wave) counts, whose order is the candidate order.  run_offsets and
// emit_ordered serve the per-thread-run compaction of the fine top-k.
#pragma once

#include "hhr_device.h"

namespace hhr {

constexpr int kLinBins = 2048;
constexpr int kLinListMax = 512;

constexpr int kStridedCnt = 256;  // (slot, wave) counts of top_largest_strided

struct TopScratch {
  int hist[kLinBins];
  uint32_t cnt[kStridedCnt];
  __attribute__((aligned(16))) float list_v[kLinListMax + 4];  // + 4: whole 16-byte reads
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

// ---------------------------------------------------------------------------
// The same selection with the scores in registers and strided ownership:
// thread t of NT holds candidate j NT + t in x[j] (j < NV), the layout that
// coalesced loads give, so the scores are never staged through LDS.  Output
// positions come from per-slot wave ballots (a lane's rank among the wave's
// taken candidates of slot j) and one exclusive prefix over the (slot, wave)
// counts, whose order j, wave, lane is the candidate order.  This costs a few
// vector instructions per candidate where the run-based compaction spends
// tens, and the top-P of one (b, g) runs on a single CU bound by its vector
// throughput.  Candidate j NT + t is present iff it is below n and
// present(x[j]); n_valid counts the present ones, and vmin <= every present
// score <= vmax.  sh.hist and sh.list_n must be zero behind a barrier; sbuf
// (NT NV floats in LDS) is used only by the radix fallback.  Returns
// min(P, n_valid).  All NT threads call.
template <int NT, int NV, typename Present, typename Emit>
__device__ int top_largest_strided(const float (&x)[NV], int n, int n_valid, Present present,
                                   int P, float vmin, float vmax, float* sbuf, TopScratch& sh,
                                   Emit& emit) {
  constexpr int NWAVES = NT / kWave;
  constexpr int NE = NV * NWAVES;  // (slot, wave) entries
  static_assert(NE <= kStridedCnt, "slot counts fit TopScratch::cnt");
  constexpr int PER = (NE + kWave - 1) / kWave;
  static_assert(PER <= 4, "at most 4 entries per lane");
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l = tid % kWave;
  const int Pe = min(P, n_valid);
  if (Pe <= 0) return 0;  // block-uniform
  const bool all = Pe >= n_valid;

  // bins, linear in value: bin(v) = (int)((v - vmin) * 2048 / (vmax - vmin)),
  // non-decreasing in v; -1 for an absent candidate
  const float range = vmax - vmin;
  const float inv = range > 0.f ? (float)kLinBins / range : 0.f;
  int bin[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const float f = (x[j] - vmin) * inv;
    const int bb = f < (float)kLinBins ? max((int)f, 0) : kLinBins - 1;
    const bool pres = j * NT + tid < n && present(x[j]);
    bin[j] = pres ? bb : -1;
    if (pres && !all) atomicAdd(&sh.hist[bb], 1);
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
      // T = the value with (#greater in b*) < need <= (#greater) + (#equal);
      // the list is read four entries per LDS load (entries past cstar are
      // masked; the list has room for them)
      for (int j = tid; j < cstar; j += NT) {
        const float vj = sh.list_v[j];
        int gtr = 0, eql = 0;
#pragma unroll 2
        for (int k0 = 0; k0 < cstar; k0 += 4) {
          const floatx4 v4 = *(const floatx4*)&sh.list_v[k0];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool in = k0 + i < cstar;
            gtr += (in && v4[i] > vj) ? 1 : 0;
            eql += (in && v4[i] == vj) ? 1 : 0;
          }
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
            return c < n && present(sbuf[c]) ? orderable_key(sbuf[c]) : 0u;
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
    rank[j] = mbcnt64(b1) | (mbcnt64(b2) << 16);
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

// ---------------------------------------------------------------------------
// Loading front end of top_largest_strided.  mid() runs once, after the loads
// are issued and before their values are used, so that work of the caller's
// with loads of its own shares their round trip.
struct NoMid {
  __device__ void operator()() const {}
};
struct AllPresent {
  __device__ bool operator()(float) const { return true; }
};

// Loads candidates j NT + t (j < NV) of src into registers (COH: agent-scope;
// addresses clamped to src[0 .. n_load)), runs mid(), then reduces the range
// of the present candidates (below n, with the given pieces lo, hi) and their
// count in one barrier, and selects with top_largest_strided.  The caller
// must have zeroed sh.hist and sh.list_n.
template <int NT, int NV, bool COH, typename Present, typename Emit, typename Mid>
__device__ int top_strided_nv(const float* src, int n_load, int n, int P, Present& present,
                              float lo, float hi, float* sbuf, TopScratch& sh, Emit& emit,
                              Mid& mid) {
  const int tid = threadIdx.x;
  const int last = max(n_load - 1, 0);
  float x[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) x[j] = Mem<COH>::ld(src + min(j * NT + tid, last));
  mid();
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const bool pres = j * NT + tid < n && present(x[j]);
    cnt += __popcll(__ballot(pres));
    if (pres) {
      lo = fminf(lo, x[j]);
      hi = fmaxf(hi, x[j]);
    }
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if ((tid & (kWave - 1)) == 0) {
    sh.w_min[tid / kWave] = lo;
    sh.w_max[tid / kWave] = hi;
    sh.w_n[tid / kWave] = cnt;
  }
  __syncthreads();  // also orders the caller's clearing of sh.hist and sh.list_n
  float vmin = __builtin_huge_valf(), vmax = -__builtin_huge_valf();
  int n_valid = 0;
#pragma unroll
  for (int k = 0; k < NT / kWave; ++k) {
    vmin = fminf(vmin, sh.w_min[k]);
    vmax = fmaxf(vmax, sh.w_max[k]);
    n_valid += sh.w_n[k];
  }
  return top_largest_strided<NT, NV>(x, n, n_valid, present, P, vmin, vmax, sbuf, sh, emit);
}

// The P largest of src[0 .. n) (those present), ties to the lower index,
// emitted in ascending index.  n_load (>= n, <= NVMAX NT, block-uniform and
// known before n may be) bounds the loads, so they need not wait for n.
// NVMAX (1, 2, 4, 8 or 16) caps the registers a caller reserves for it.
template <int NT, bool COH, typename Present, typename Emit, typename Mid = NoMid,
          int NVMAX = 16>
__device__ __forceinline__ int top_strided(const float* src, int n_load, int n, int P, Present present, float lo,
                           float hi, float* sbuf, TopScratch& sh, Emit emit, Mid mid = Mid()) {
  static_assert(NVMAX == 1 || NVMAX == 2 || NVMAX == 4 || NVMAX == 8 || NVMAX == 16, "NVMAX");
  const int tid = threadIdx.x;
  for (int i = tid; i < kLinBins; i += NT) sh.hist[i] = 0;  // ready after the range barrier
  if (tid == 0) sh.list_n = 0;
  const int nv = (n_load + NT - 1) / NT;
#define HHR_TOP_STRIDED(V) \
  return top_strided_nv<NT, V, COH>(src, n_load, n, P, present, lo, hi, sbuf, sh, emit, mid)
  if (NVMAX == 1 || nv <= 1) HHR_TOP_STRIDED(1);
  if (NVMAX == 2 || nv <= 2) HHR_TOP_STRIDED(NVMAX < 2 ? NVMAX : 2);
  if (NVMAX == 4 || nv <= 4) HHR_TOP_STRIDED(NVMAX < 4 ? NVMAX : 4);
  if (NVMAX == 8 || nv <= 8) HHR_TOP_STRIDED(NVMAX < 8 ? NVMAX : 8);
  HHR_TOP_STRIDED(NVMAX);
#undef HHR_TOP_STRIDED
}

// ---------------------------------------------------------------------------
// Exact top-P of n <= kPrefilterMaxPages candidates when a lower bound lb of
// the cut is known: each of the J producing workgroups has published (thr) a
// value that q of its own candidates reach, with (J - 1) q >= P, so the P
// largest candidates are all >= the smallest published value.  Candidates
// below it cannot be taken: the rest are compacted into LDS in candidate
// order (ballots, one prefix over the (slot, wave) counts) and the top-P is
// taken among them with top_largest_strided, with a quarter of the registers
// per thread when about a quarter survive.  sc[c] is loaded with agent-scope
// loads (c < n_load, clamped); present(v) says whether candidate c < n takes
// part; sbuf holds the compacted values (and serves the radix fallback), cidx
// their candidate indices.  emit(pos, c) with pos ascending in c.  All NT
// threads call; returns min(P, present candidates).
constexpr int kPrefilterMaxPages = 8192;

template <int NT, int NV2, typename Emit>
__device__ __forceinline__ int top_compacted(int n, int P, float lb, float vmax, float* sbuf,
                                             const uint16_t* cidx, TopScratch& sh, Emit& emit) {
  const int tid = threadIdx.x;
  float x2[NV2];
#pragma unroll
  for (int j = 0; j < NV2; ++j) x2[j] = sbuf[min(j * NT + tid, n - 1)];
  auto emit2 = [&](int pos, int c) { emit(pos, (int)cidx[c]); };
  return top_largest_strided<NT, NV2>(x2, n, n, AllPresent(), P, lb, vmax, sbuf, sh, emit2);
}

template <int NT, typename Present, typename Emit>
__device__ __forceinline__ int top_prefiltered(const float* sc, int n_load, int n, int P,
                                               Present present, const float* thr, int J,
                                               float* sbuf, uint16_t* cidx, TopScratch& sh,
                                               Emit emit) {
  constexpr int NV = kPrefilterMaxPages / NT;
  constexpr int NWAVES = NT / kWave;
  constexpr int NE = NV * NWAVES;
  constexpr int PER = (NE + kWave - 1) / kWave;
  static_assert(NE <= kStridedCnt && PER <= 4, "slot counts fit TopScratch::cnt");
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = tid % kWave;
  const int last = max(n_load - 1, 0);
  float x[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) x[j] = Mem<true>::ld(sc + min(j * NT + tid, last));
  const float t = Mem<true>::ld(thr + min(tid, J - 1));
  issue_loads_here();
  for (int i = tid; i < kLinBins; i += NT) sh.hist[i] = 0;  // for the selection below
  if (tid == 0) sh.list_n = 0;
  const float tm = wave_min(tid < J ? t : __builtin_huge_valf());
  if (l == 0) sh.w_min[w] = tm;
  __syncthreads();
  float lb = __builtin_huge_valf();
#pragma unroll
  for (int k = 0; k < NWAVES; ++k) lb = fminf(lb, sh.w_min[k]);
  // compaction of the survivors (present, >= lb) in candidate order, and their maximum
  uint32_t rank[NV];
  bool keep[NV];
  float hm = -__builtin_huge_valf();
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    keep[j] = j * NT + tid < n && present(x[j]) && x[j] >= lb;
    const uint64_t m = __ballot(keep[j]);
    rank[j] = mbcnt64(m);
    if (l == 0) sh.cnt[j * NWAVES + w] = (uint32_t)popc64(m);
    if (keep[j]) hm = fmaxf(hm, x[j]);
  }
  hm = wave_max(hm);
  if (l == 0) sh.w_max[w] = hm;
  __syncthreads();
  float vmax = -__builtin_huge_valf();
#pragma unroll
  for (int k = 0; k < NWAVES; ++k) vmax = fmaxf(vmax, sh.w_max[k]);
  uint32_t pre[PER], tot;
  {
    uint32_t v[PER], local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = PER * l + i;
      v[i] = e < NE ? sh.cnt[e] : 0u;
      local += v[i];
    }
    const uint32_t inc = wave_inclusive_scan(local);
    tot = (uint32_t)__builtin_amdgcn_readlane((int)inc, kWave - 1);
    uint32_t run = inc - local;
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
    const uint32_t pos = (uint32_t)__builtin_amdgcn_readlane((int)p, e / PER) + rank[j];
    if (keep[j]) {
      sbuf[pos] = x[j];
      cidx[pos] = (uint16_t)(j * NT + tid);
    }
  }
  __syncthreads();
  const int nc = (int)tot;  // >= min(P, present) by the choice of the published values
  if (nc <= 0) return 0;
  if (nc <= NT) return top_compacted<NT, 1>(nc, P, lb, vmax, sbuf, cidx, sh, emit);
  if (nc <= 2 * NT) return top_compacted<NT, 2>(nc, P, lb, vmax, sbuf, cidx, sh, emit);
  if (nc <= 4 * NT) return top_compacted<NT, 4>(nc, P, lb, vmax, sbuf, cidx, sh, emit);
  return top_compacted<NT, 8>(nc, P, lb, vmax, sbuf, cidx, sh, emit);
}

// The lower bound a producing workgroup publishes for top_prefiltered: a
// value that min(q, its present candidates) of its candidates reach, namely
// the smallest candidate of the bin of a 64-bin histogram over its
// candidates' range (wlo, whi) in which the count from the top reaches q (its
// smallest candidate when it has fewer than q).  Thread t holds candidate v
// when has; s_cnt and s_min are 64 words of LDS that the caller has set to
// 0 and 0xFFFFFFFF behind a barrier (lower_bound_init).  Every thread of the
// workgroup calls (one barrier); thread 0 stores the value to *dst.
__device__ __forceinline__ void lower_bound_init(int* s_cnt, uint32_t* s_min) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    s_cnt[tid] = 0;
    s_min[tid] = 0xFFFFFFFFu;
  }
}

__device__ __forceinline__ void publish_lower_bound(float v, bool has, float wlo, float whi,
                                                    int q, int* s_cnt, uint32_t* s_min,
                                                    float* dst) {
  const int tid = threadIdx.x;
  const float inv = whi > wlo ? 64.f / (whi - wlo) : 0.f;
  if (has) {
    const float f = (v - wlo) * inv;
    const int bin = f < 64.f ? max((int)f, 0) : 63;
    atomicAdd(&s_cnt[bin], 1);
    atomicMin(&s_min[bin], orderable_key(v));
  }
  __syncthreads();
  if (tid < 64) {  // wave 0: bins from the top
    const int c = s_cnt[63 - tid];
    const int inc = wave_inclusive_scan(c);
    const uint64_t hit = __ballot(inc >= q && inc - c < q);
    float t = wlo;  // fewer than q here: every candidate counts
    if (hit != 0ull) {
      const uint32_t key = s_min[63 - __builtin_ctzll(hit)];
      t = __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
    }
    if (tid == 0) Mem<true>::st(dst, t);
  }
}

}  // namespace hhr
