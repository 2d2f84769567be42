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
// A wave takes a batch of 16 consecutive pages.  Lane (row r = l/16,
// sub = l%16) handles pages pb + 4j + r (j = 0..3) and, in each, the 16-byte
// pieces k = 0..3 at byte 256k + 16 sub (dims 2(sub + 16k) and +1), so every
// load instruction reads four whole 256-byte runs.  All 16 loads are issued
// before anything that depends on the query (addresses are clamped, not
// branched on, so nothing serialises them); a 4-value reduce-scatter over the
// 16 lanes of a row then leaves page pb + 4j + r in lanes with j = 2 b3 + b2.
constexpr int kScoreWaves = 4;
constexpr int kScorePagesPerWave = 16;
constexpr int kScorePagesPerWg = kScoreWaves * kScorePagesPerWave;  // 64

__global__ __launch_bounds__(256) void k_page_scores(const float* __restrict__ q_rot,
                                                     const int32_t* __restrict__ seq_len,
                                                     const float* __restrict__ meta,
                                                     float* __restrict__ scores,
                                                     uint32_t* __restrict__ status, int Hq,
                                                     int Hkv, int Lcap) {
  const int bg = blockIdx.y;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  const int G = Hq / Hkv;
  const int NpCap = Lcap / kPS;
  const int L = checked_len(seq_len, b, Lcap, blockIdx.x == 0 && g == 0 ? status : nullptr);
  const int Np = (L + kPS - 1) / kPS;
  const int w = threadIdx.x >> 6;
  const int l = threadIdx.x & 63;
  const int pb = blockIdx.x * kScorePagesPerWg + w * kScorePagesPerWave;
  if (pb >= Np) return;
  const int r = l >> 4;
  const int sub = l & 15;

  const float* mbase = meta + (size_t)bg * NpCap * kD * 2 + 4 * sub;
  floatx4 m[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = min(pb + 4 * j + r, Np - 1);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      m[j][k] = __builtin_nontemporal_load((const floatx4*)(mbase + (size_t)p * kD * 2 + 64 * k));
  }
  float A[4][2], B[4][2];
#pragma unroll
  for (int k = 0; k < 4; ++k) A[k][0] = A[k][1] = B[k][0] = B[k][1] = 0.f;
  const float* qr = q_rot + ((size_t)b * Hq + (size_t)g * G) * kD + 2 * sub;
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float2 v = *(const float2*)(qr + (size_t)h * kD + 32 * k);
      A[k][0] += fmaxf(v.x, 0.f);
      B[k][0] += fminf(v.x, 0.f);
      A[k][1] += fmaxf(v.y, 0.f);
      B[k][1] += fminf(v.y, 0.f);
    }
  }
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float x = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)  // m = {mn[d0], mx[d0], mn[d1], mx[d1]}
      x += A[k][0] * m[j][k][1] + B[k][0] * m[j][k][0] + A[k][1] * m[j][k][3] +
           B[k][1] * m[j][k][2];
    v[j] = x;
  }
  const bool b3 = l & 8, b2 = l & 4;
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
  const int p = pb + 4 * ((b3 ? 2 : 0) + (b2 ? 1 : 0)) + r;
  if ((l & 3) == 0 && p < Np) scores[(size_t)bg * NpCap + p] = v[0];
}

// ------------------------------------------------------------------ S4
// Exact top-P of the page scores of one (b, g) in one workgroup: page
// p = i*512 + tid sits in slot i of thread tid (coalesced loads); the cut-off
// comes from a value-linear histogram, and the kept pages are written
// ascending by an ordered compaction.
constexpr int kTopPThreads = 512;
constexpr int kTopPItems = kMaxCtx / kPS / kTopPThreads;  // 32: NpCap <= 16384
constexpr int kSelThreads = 1024;

__global__ __launch_bounds__(kTopPThreads) void k_top_pages(
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
  for (int i = P + tid; i < p_max; i += kTopPThreads) out[i] = -1;
  if (tid == 0) kept_count[bg] = P;
  if (P == 0) return;

  const float* sc = scores + (size_t)bg * NpCap;
  float x[kTopPItems];
  bool pr[kTopPItems];
#pragma unroll
  for (int i = 0; i < kTopPItems; ++i) {
    const int c = i * kTopPThreads + tid;
    x[i] = sc[min(c, Np - 1)];  // clamped, not branched: the loads overlap
    pr[i] = c < Np;
  }
  top_largest_strided<kTopPThreads, kTopPItems>(x, pr, P, sh,
                                                [&](int pos, int c) { out[pos] = c; });
}

// ------------------------------------------------------------------ S5+S6
// Candidates are the rows of the kept pages in kept order, which is ascending
// position order: candidate c = (kept slot c/16, row c%16), held by thread
// c % 1024 in register slot c / 1024.
//   pass 1: H for every candidate -- the kept list is staged in LDS and the
//           16-byte code loads are issued 16 at a time (clamped rows, no
//           branches) -- into an LDS histogram (4 copies spread same-bin atomics);
//   threshold: the smallest H value T whose cumulative count reaches top_k,
//           and how many candidates with H == T are taken (need);
//   pass 2: ordered compaction on key = 4096 - H (larger key = smaller H).
constexpr int kHamItems = kMaxCand / kSelThreads;  // 32
constexpr int kHamBins = 128 * kMaxG + 1;           // 2049
constexpr int kHistCopies = 4;
constexpr int kHamBatch = 16;

__global__ __launch_bounds__(kSelThreads) void k_hamming_topk(
    const uint32_t* __restrict__ q_codes, const uint32_t* __restrict__ codes,
    const int32_t* __restrict__ seq_len, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ kept_count, int p_max, int top_k, int Hq, int Hkv, int Lcap,
    int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_count, uint16_t* __restrict__ dist,
    uint32_t* __restrict__ status) {
  __shared__ int hist[kHistCopies][kHamBins];
  __shared__ int skept[kMaxCand / kPS];
  __shared__ uint32_t sq[kMaxG * kNW];
  __shared__ int s_T, s_need, s_valid;
  __shared__ int scan_lds[kSelThreads / kWave + 1];
  __shared__ TopScratch sh;

  const int bg = blockIdx.x;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int L = checked_len(seq_len, b, Lcap, g == 0 ? status : nullptr);
  const int P = L > 0 ? min(kept_count[bg], p_max) : 0;
  const int ncand = P * kPS;
  const int nbins = 128 * G + 1;

  if (tid < G * kNW) sq[tid] = q_codes[((size_t)b * Hq + (size_t)g * G) * kNW + tid];
  for (int i = tid; i < P; i += kSelThreads) skept[i] = kept[(size_t)bg * p_max + i];
  for (int i = tid; i < kHistCopies * kHamBins; i += kSelThreads) (&hist[0][0])[i] = 0;
  __syncthreads();

  const uint32_t* cb = codes + (size_t)bg * Lcap * kNW;
  const int items = (ncand + kSelThreads - 1) / kSelThreads;
  int* my_hist = hist[w & (kHistCopies - 1)];
  int H[kHamItems];
#pragma unroll
  for (int i = 0; i < kHamItems; ++i) H[i] = -1;  // absent
#pragma unroll
  for (int i0 = 0; i0 < kHamItems; i0 += kHamBatch) {
    if (i0 < items) {
      u32x4 code[kHamBatch];
      bool ok[kHamBatch];
#pragma unroll
      for (int j = 0; j < kHamBatch; ++j) {
        const int c = (i0 + j) * kSelThreads + tid;
        const int page = skept[min(c, ncand - 1) >> 4];
        const int t = page * kPS + (c & 15);
        ok[j] = c < ncand && page >= 0 && t < L;
        code[j] = *(const u32x4*)(cb + (size_t)(ok[j] ? t : 0) * kNW);
      }
#pragma unroll
      for (int j = 0; j < kHamBatch; ++j) {
        if (ok[j]) {
          int h = 0;
          for (int qh = 0; qh < G; ++qh) {
            h += __popc(code[j][0] ^ sq[qh * kNW + 0]) + __popc(code[j][1] ^ sq[qh * kNW + 1]) +
                 __popc(code[j][2] ^ sq[qh * kNW + 2]) + __popc(code[j][3] ^ sq[qh * kNW + 3]);
          }
          H[i0 + j] = h;
          atomicAdd(&my_hist[h], 1);
        }
      }
    }
  }
  if (dist) {
#pragma unroll
    for (int i = 0; i < kHamItems; ++i) {
      const int c = i * kSelThreads + tid;
      if (c < ncand) dist[(size_t)bg * p_max * kPS + c] = H[i] < 0 ? (uint16_t)0xFFFF : (uint16_t)H[i];
    }
  }
  __syncthreads();

  // threshold over bins in ascending H
  {
    const int per = (nbins + kSelThreads - 1) / kSelThreads;  // <= 3
    const int b0 = tid * per;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      if (b0 + i < nbins) {
        int c = 0;
#pragma unroll
        for (int k = 0; k < kHistCopies; ++k) c += hist[k][b0 + i];
        hist[0][b0 + i] = c;
        local += c;
      }
    }
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
          const int c = hist[0][b0 + i];
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
  const int count = min(top_k, s_valid);
  uint32_t key[kHamItems];
#pragma unroll
  for (int i = 0; i < kHamItems; ++i) key[i] = H[i] < 0 ? 0u : (uint32_t)(4096 - H[i]);
  const uint32_t T = s_T == nbins ? 0u : (uint32_t)(4096 - s_T);
  int32_t* out = sel_idx + (size_t)bg * top_k;
  compact_strided<kSelThreads, kHamItems>(key, T, s_need, sh, [&](int pos, int c) {
    out[pos] = skept[c >> 4] * kPS + (c & 15);
  });
  for (int i = count + tid; i < top_k; i += kSelThreads) out[i] = -1;
  if (tid == 0) sel_count[bg] = count;
}

}  // namespace

hipError_t launch_page_scores(const hhr_shape& s, const float* q_rot, const int32_t* seq_len,
                              const float* meta, float* scores, uint32_t* status,
                              hipStream_t stream) {
  const int NpCap = s.max_ctx / kPS;
  dim3 grid((NpCap + kScorePagesPerWg - 1) / kScorePagesPerWg, s.batch * s.n_kv_heads);
  hipLaunchKernelGGL(k_page_scores, grid, dim3(256), 0, stream, q_rot, seq_len, meta, scores,
                     status, s.n_q_heads, s.n_kv_heads, s.max_ctx);
  return hipGetLastError();
}

hipError_t launch_top_pages(const hhr_shape& s, const float* scores, const int32_t* seq_len,
                            int32_t keep_num, int32_t keep_den, int32_t keep_abs, int32_t p_max,
                            int32_t* kept, int32_t* kept_count, uint32_t* status,
                            hipStream_t stream) {
  hipLaunchKernelGGL(k_top_pages, dim3(s.batch * s.n_kv_heads), dim3(kTopPThreads), 0, stream,
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
