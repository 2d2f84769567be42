// S3 page-bound scorer, S4 top-P page pruning, S5 Hamming scan + S6 exact top-k.
//
// [HHR abstract] GKR derives page-level logit bounds from the rotated keys and
// prunes low-bound pages; LHP then ranks the keys of the surviving pages by
// the Hamming distance of their codes to the query's code.  [HATA abstract]
// only the relative order matters, so the fine stage is an exact top-k on the
// integer distance with a lowest-position tie-break.

#include "hhr_device.h"
#include "hhr_internal.h"
#include "topk_device.h"

namespace hhr {

namespace {

__device__ __forceinline__ int checked_len(const int32_t* seq_len, int b, int Lcap,
                                           uint32_t* status) {
  const int L = seq_len[b];
  if (L < 0 || L > Lcap) {
    if (status && threadIdx.x == 0) atomicOr(status, HHR_DEV_BAD_SEQ_LEN);
    return 0;
  }
  return L;
}

// ------------------------------------------------------------------ S3
// Per page p of (b, g):  s(p) = sum_h sum_d max(q'_hd mn_pd, q'_hd mx_pd).
// Because mn <= mx, max(q mn, q mx) = max(q,0) mx + min(q,0) mn, so per
// dimension the group reduces to A_d = sum_h max(q'_hd, 0) and
// B_d = sum_h min(q'_hd, 0), and s(p) = sum_d (A_d mx_pd + B_d mn_pd).
//
// One wave streams 16 pages at a time: lane l reads dims {2l, 2l+1} of each
// page (16 bytes; the wave reads the page's 1 KiB in one coalesced load),
// keeps 16 partial sums, and a butterfly reduce-scatter leaves the sum of
// page 8*b5 + 4*b4 + 2*b3 + b2 (b_i = bit i of the lane id) in every lane.
constexpr int kScoreWaves = 4;
constexpr int kPagesPerWaveIter = 16;

__global__ __launch_bounds__(256) void k_page_scores(const float* __restrict__ q_rot,
                                                     const int32_t* __restrict__ seq_len,
                                                     const float* __restrict__ meta,
                                                     float* __restrict__ scores,
                                                     uint32_t* __restrict__ status, int Hq,
                                                     int Hkv, int Lcap, int pages_per_wg) {
  const int bg = blockIdx.y;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  const int G = Hq / Hkv;
  const int NpCap = Lcap / kPS;
  const int L = checked_len(seq_len, b, Lcap, blockIdx.x == 0 && g == 0 ? status : nullptr);
  const int Np = (L + kPS - 1) / kPS;
  const int p_begin = blockIdx.x * pages_per_wg;
  if (p_begin >= Np) return;
  const int p_end = min(Np, p_begin + pages_per_wg);

  const int w = threadIdx.x >> 6;
  const int l = threadIdx.x & 63;
  float A0 = 0.f, B0 = 0.f, A1 = 0.f, B1 = 0.f;
  const float* qr = q_rot + ((size_t)b * Hq + (size_t)g * G) * kD + 2 * l;
  for (int h = 0; h < G; ++h) {
    const float2 v = *(const float2*)(qr + (size_t)h * kD);
    A0 += fmaxf(v.x, 0.f);
    B0 += fminf(v.x, 0.f);
    A1 += fmaxf(v.y, 0.f);
    B1 += fminf(v.y, 0.f);
  }
  const float* mbase = meta + (size_t)bg * NpCap * kD * 2 + 4 * l;
  float* sbase = scores + (size_t)bg * NpCap;

  for (int pb = p_begin + w * kPagesPerWaveIter; pb < p_end;
       pb += kScoreWaves * kPagesPerWaveIter) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int p = pb + i;
      v[i] = 0.f;
      if (p < p_end) {
        const floatx4 m = __builtin_nontemporal_load((const floatx4*)(mbase + (size_t)p * kD * 2));
        // m = {mn[2l], mx[2l], mn[2l+1], mx[2l+1]}
        v[i] = A0 * m[1] + B0 * m[0] + A1 * m[3] + B1 * m[2];
      }
    }
    const bool b5 = l & 32, b4 = l & 16, b3 = l & 8, b2 = l & 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float send = b5 ? v[i] : v[i + 8];
      const float keep = b5 ? v[i + 8] : v[i];
      v[i] = keep + __shfl_xor(send, 32);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float send = b4 ? v[i] : v[i + 4];
      const float keep = b4 ? v[i + 4] : v[i];
      v[i] = keep + __shfl_xor(send, 16);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float send = b3 ? v[i] : v[i + 2];
      const float keep = b3 ? v[i + 2] : v[i];
      v[i] = keep + __shfl_xor(send, 8);
    }
    {
      const float send = b2 ? v[0] : v[1];
      const float keep = b2 ? v[1] : v[0];
      v[0] = keep + __shfl_xor(send, 4);
    }
    v[0] += __shfl_xor(v[0], 2);
    v[0] += __shfl_xor(v[0], 1);
    const int idx = (b5 ? 8 : 0) + (b4 ? 4 : 0) + (b3 ? 2 : 0) + (b2 ? 1 : 0);
    if ((l & 3) == 0 && pb + idx < p_end) sbase[pb + idx] = v[0];
  }
}

// ------------------------------------------------------------------ S4
// Exact top-P of the page scores of one (b, g) in one 1024-thread workgroup
// (radix select on orderable float keys, then an ordered block scan), kept
// pages written ascending.
constexpr int kSelThreads = 1024;
constexpr int kTopPItems = 16;  // NpCap <= 16384

__global__ __launch_bounds__(kSelThreads) void k_top_pages(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_len, int keep_num,
    int keep_den, int keep_abs, int p_max, int Hkv, int Lcap, int32_t* __restrict__ kept,
    int32_t* __restrict__ kept_count, uint32_t* __restrict__ status) {
  __shared__ TopScratch sh;
  const int bg = blockIdx.x;
  const int b = bg / Hkv;
  const int NpCap = Lcap / kPS;
  const int L = checked_len(seq_len, b, Lcap, (bg % Hkv) == 0 ? status : nullptr);
  const int Np = (L + kPS - 1) / kPS;
  int P = 0;
  if (Np > 0) {
    if (keep_abs > 0) P = min(Np, keep_abs);
    else P = min(Np, max(1, (int)(((long long)keep_num * Np + keep_den - 1) / keep_den)));
  }
  const int tid = threadIdx.x;
  int32_t* out = kept + (size_t)bg * p_max;
  for (int i = P + tid; i < p_max; i += kSelThreads) out[i] = -1;
  if (tid == 0) kept_count[bg] = P;
  if (P == 0) return;

  const int items = (Np + kSelThreads - 1) / kSelThreads;
  const int i0 = tid * items;
  const float* sc = scores + (size_t)bg * NpCap;
  uint32_t key[kTopPItems];
#pragma unroll
  for (int i = 0; i < kTopPItems; ++i)
    key[i] = (i < items && i0 + i < Np) ? orderable_key(sc[i0 + i]) : 0u;
  top_largest_ordered<kSelThreads, kTopPItems>(key, items, P, sh,
                                               [&](int pos, int c) { out[pos] = c; });
}

// ------------------------------------------------------------------ S5+S6
// Candidates are the rows of the kept pages in kept order, which is ascending
// position order: candidate c = (kept slot c/16, row c%16).  Candidate
// c = i*1024 + tid is held by thread tid in register slot i.
//   pass 1: H for every candidate (coalesced 16-byte code loads), LDS histogram;
//   threshold: the smallest H value T whose cumulative count reaches top_k;
//   pass 2: ordered selection -- H < T, or H == T among the first `need` --
//           with positions from wave ballots plus a scan over (slot, wave).
constexpr int kHamItems = kMaxCand / kSelThreads;  // 32
constexpr int kHamBins = 128 * kMaxG + 1;           // 2049

__global__ __launch_bounds__(kSelThreads) void k_hamming_topk(
    const uint32_t* __restrict__ q_codes, const uint32_t* __restrict__ codes,
    const int32_t* __restrict__ seq_len, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ kept_count, int p_max, int top_k, int Hq, int Hkv, int Lcap,
    int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_count, uint16_t* __restrict__ dist,
    uint32_t* __restrict__ status) {
  __shared__ int hist[kHamBins];
  __shared__ uint32_t sq[kMaxG * kNW];
  __shared__ int cnt_lt[kHamItems * 16], cnt_eq[kHamItems * 16];
  __shared__ int s_T, s_need;
  __shared__ int scan_lds[kSelThreads / kWave + 1];

  const int bg = blockIdx.x;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int L = checked_len(seq_len, b, Lcap, g == 0 ? status : nullptr);
  const int P = L > 0 ? min(kept_count[bg], p_max) : 0;
  const int ncand = P * kPS;
  const int nbins = 128 * G + 1;

  if (tid < G * kNW) sq[tid] = q_codes[((size_t)b * Hq + (size_t)g * G) * kNW + tid];
  for (int i = tid; i < nbins; i += kSelThreads) hist[i] = 0;
  __syncthreads();

  const int32_t* kp = kept + (size_t)bg * p_max;
  const uint32_t* cb = codes + (size_t)bg * Lcap * kNW;
  const int items = (ncand + kSelThreads - 1) / kSelThreads;
  // distances (<= 2048, or 0xFFFF for absent candidates) packed two per register
  uint32_t Hp[kHamItems / 2];
#pragma unroll
  for (int i = 0; i < kHamItems / 2; ++i) Hp[i] = 0xFFFFFFFFu;
#define HHR_H(i) ((int)((Hp[(i) >> 1] >> (16 * ((i) & 1))) & 0xFFFFu))
#pragma unroll
  for (int i = 0; i < kHamItems; ++i) {
    const int c = i * kSelThreads + tid;
    if (i < items && c < ncand) {
      const int page = kp[c >> 4];
      const int t = page * kPS + (c & 15);
      if (page >= 0 && t < L) {
        const u32x4 code = *(const u32x4*)(cb + (size_t)t * kNW);
        int h = 0;
        for (int qh = 0; qh < G; ++qh) {
          h += __popc(code[0] ^ sq[qh * kNW + 0]) + __popc(code[1] ^ sq[qh * kNW + 1]) +
               __popc(code[2] ^ sq[qh * kNW + 2]) + __popc(code[3] ^ sq[qh * kNW + 3]);
        }
        Hp[i >> 1] = (Hp[i >> 1] & ~(0xFFFFu << (16 * (i & 1)))) | ((uint32_t)h << (16 * (i & 1)));
        atomicAdd(&hist[h], 1);
      }
      if (dist) dist[(size_t)bg * p_max * kPS + c] = (uint16_t)HHR_H(i);
    }
  }
  __syncthreads();

  // threshold over bins in ascending H
  __shared__ int s_valid;
  {
    const int per = (nbins + kSelThreads - 1) / kSelThreads;  // <= 3
    const int b0 = tid * per;
    int local = 0;
    for (int i = 0; i < per; ++i)
      if (b0 + i < nbins) local += hist[b0 + i];
    int total;
    const int ex = block_exclusive_scan<kSelThreads, int>(local, scan_lds, &total);
    if (tid == 0) {
      s_T = nbins;  // every valid H is < nbins: take all valid candidates
      s_need = 0;
      s_valid = total;
    }
    __syncthreads();
    if (total > top_k) {
      int run = ex;
      for (int i = 0; i < per; ++i) {
        if (b0 + i < nbins) {
          const int c = hist[b0 + i];
          if (run < top_k && run + c >= top_k) {
            s_T = b0 + i;
            s_need = top_k - run;
          }
          run += c;
        }
      }
    }
    __syncthreads();
  }
  const int T = s_T;
  const int need = s_need;
  const int count = min(top_k, s_valid);

  // pass 2: per (slot i, wave w) counts of H < T and H == T
#pragma unroll
  for (int i = 0; i < kHamItems; ++i) {
    if (i < items) {
      const uint64_t blt = __ballot(HHR_H(i) < T);
      const uint64_t beq = __ballot(HHR_H(i) == T);
      if (l == 0) {
        cnt_lt[i * 16 + w] = popc64(blt);
        cnt_eq[i * 16 + w] = popc64(beq);
      }
    }
  }
  __syncthreads();
  if (w == 0) {
    // exclusive scan over the (slot i, wave w) sequence, 16 waves per slot
    const int n = items * 16;
    const int per = (n + kWave - 1) / kWave;
    int a = 0, e2 = 0;
    for (int k = 0; k < per; ++k) {
      const int j = l * per + k;
      if (j < n) {
        a += cnt_lt[j];
        e2 += cnt_eq[j];
      }
    }
    int ra = wave_inclusive_scan(a) - a;
    int re = wave_inclusive_scan(e2) - e2;
    for (int k = 0; k < per; ++k) {
      const int j = l * per + k;
      if (j < n) {
        const int ta = cnt_lt[j], te = cnt_eq[j];
        cnt_lt[j] = ra;
        cnt_eq[j] = re;
        ra += ta;
        re += te;
      }
    }
  }
  __syncthreads();

  int32_t* out = sel_idx + (size_t)bg * top_k;
  const uint64_t mlt = lanemask_lt();
#pragma unroll
  for (int i = 0; i < kHamItems; ++i) {
    if (i < items) {
      const int Hi = HHR_H(i);
      const uint64_t blt = __ballot(Hi < T);
      const uint64_t beq = __ballot(Hi == T);
      const int c = i * kSelThreads + tid;
      const int lt_before = cnt_lt[i * 16 + w] + popc64(blt & mlt);
      const int eq_before = cnt_eq[i * 16 + w] + popc64(beq & mlt);
      const bool take = Hi < T || (Hi == T && eq_before < need);
      if (take) out[lt_before + min(eq_before, need)] = kp[c >> 4] * kPS + (c & 15);
    }
  }
  for (int i = count + tid; i < top_k; i += kSelThreads) out[i] = -1;
  if (tid == 0) sel_count[bg] = count;
#undef HHR_H
}

}  // namespace

hipError_t launch_page_scores(const hhr_shape& s, const float* q_rot, const int32_t* seq_len,
                              const float* meta, float* scores, uint32_t* status,
                              hipStream_t stream) {
  const int NpCap = s.max_ctx / kPS;
  const int pages_per_wg = 128;
  dim3 grid((NpCap + pages_per_wg - 1) / pages_per_wg, s.batch * s.n_kv_heads);
  hipLaunchKernelGGL(k_page_scores, grid, dim3(256), 0, stream, q_rot, seq_len, meta, scores,
                     status, s.n_q_heads, s.n_kv_heads, s.max_ctx, pages_per_wg);
  return hipGetLastError();
}

hipError_t launch_top_pages(const hhr_shape& s, const float* scores, const int32_t* seq_len,
                            int32_t keep_num, int32_t keep_den, int32_t keep_abs, int32_t p_max,
                            int32_t* kept, int32_t* kept_count, uint32_t* status,
                            hipStream_t stream) {
  hipLaunchKernelGGL(k_top_pages, dim3(s.batch * s.n_kv_heads), dim3(kSelThreads), 0, stream,
                     scores, seq_len, keep_num, keep_den, keep_abs, p_max, s.n_kv_heads,
                     s.max_ctx, kept, kept_count, status);
  return hipGetLastError();
}

hipError_t launch_hamming_topk(const hhr_shape& s, const uint32_t* q_codes, const uint32_t* codes,
                               const int32_t* seq_len, const int32_t* kept,
                               const int32_t* kept_count, int32_t p_max, int32_t top_k,
                               int32_t* sel_idx, int32_t* sel_count, uint16_t* dist,
                               uint32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(k_hamming_topk, dim3(s.batch * s.n_kv_heads), dim3(kSelThreads), 0, stream,
                     q_codes, codes, seq_len, kept, kept_count, p_max, top_k, s.n_q_heads,
                     s.n_kv_heads, s.max_ctx, sel_idx, sel_count, dist, status);
  return hipGetLastError();
}

}  // namespace hhr
