// S3 page-bound scorer, S4 top-P page pruning, S5 Hamming scan + S6 exact top-k.
//
// [HHR abstract] GKR derives page-level logit bounds from the rotated keys and
// prunes low-bound pages; LHP then ranks the keys of the surviving pages by
// the Hamming distance of their codes to the query's code.  [HATA abstract]
// only the relative order matters, so the fine stage is an exact top-k on the
// integer distance with a lowest-position tie-break.

#include "hhr_device.h"
#include "hhr_internal.h"
#include "stages.h"

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
// Four waves per workgroup, 16 pages per wave (score_batch).
constexpr int kScoreWaves = 4;
constexpr int kScorePagesPerWg = kScoreWaves * kScorePagesPerWave;  // 64

template <bool MBF>
__global__ __launch_bounds__(256) void k_page_scores(const float* __restrict__ q_rot,
                                                     const int32_t* __restrict__ seq_len,
                                                     const void* __restrict__ meta,
                                                     float* __restrict__ scores,
                                                     uint32_t* __restrict__ status, int Hq,
                                                     int Hkv, int Lcap) {
  const int bg = blockIdx.y;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  const int L = checked_len(seq_len, b, Lcap, blockIdx.x == 0 && g == 0 ? status : nullptr);
  const int Np = (L + kPS - 1) / kPS;
  const int pb = blockIdx.x * kScorePagesPerWg + (threadIdx.x >> 6) * kScorePagesPerWave;
  if (pb >= Np) return;
  score_batch<MBF, false>(b, g, Hq, Hkv, Lcap / kPS, Np, pb, q_rot, meta, scores);
}

// ------------------------------------------------------------------ S4
// Exact top-P of the page scores of one (b, g); kept pages written ascending.
constexpr int kTopPThreads = 1024;

__global__ __launch_bounds__(kTopPThreads) void k_top_pages(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_len, int keep_num,
    int keep_den, int keep_abs, int p_max, int Hkv, int Lcap, int32_t* __restrict__ kept,
    int32_t* __restrict__ kept_count, uint32_t* __restrict__ status) {
  __shared__ TopScratch sh;
  __shared__ __attribute__((aligned(16))) float sbuf[kMaxCtx / kPS];
  const int bg = blockIdx.x;
  const int b = bg / Hkv;
  const int L = checked_len(seq_len, b, Lcap, (bg % Hkv) == 0 ? status : nullptr);
  const int Np = (L + kPS - 1) / kPS;
  const int P = keep_count_dev(Np, keep_num, keep_den, keep_abs);
  const int tid = threadIdx.x;
  int32_t* out = kept + (size_t)bg * p_max;
  for (int i = P + tid; i < p_max; i += kTopPThreads) out[i] = -1;
  if (tid == 0) kept_count[bg] = P;
  if (P == 0) return;
  top_pages_strided<kTopPThreads, false>(scores + (size_t)bg * (Lcap / kPS), Np, P,
                                         __builtin_huge_valf(), -__builtin_huge_valf(), sbuf, sh,
                                         [&](int pos, int c) { out[pos] = c; });
}

// ------------------------------------------------------------------ S5+S6
constexpr int kHamDistThreads = 256;
constexpr int kHamSelThreads = 1024;

__device__ __forceinline__ int kept_pages(const int32_t* kept_count, int bg, int L, int p_max) {
  return L > 0 ? max(0, min(kept_count[bg], p_max)) : 0;
}

// Distances of one 64-page chunk of one (b, g) for NW-word codes: grid
// (chunks, B*Hkv).
template <int NW>
__global__ __launch_bounds__(kHamDistThreads) void k_ham_dist(
    const uint32_t* __restrict__ q_codes, const uint32_t* __restrict__ codes,
    const int32_t* __restrict__ seq_len, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ kept_count, int p_max, int Hq, int Hkv, int Lcap,
    uint16_t* __restrict__ dist, int* __restrict__ hist, uint16_t* __restrict__ cum) {
  __shared__ HamDistSmem<NW> sm;
  const int bg = blockIdx.y;
  ham_dist_chunk<kHamDistThreads, false, NW>(bg / Hkv, bg % Hkv, Hq, Hkv, Lcap, blockIdx.x, p_max,
                                         seq_len, kept_count, q_codes, codes, kept, dist, hist,
                                         cum, sm);
}

// Exact top-k of one (b, g) from its distances and chunk histograms.
__global__ __launch_bounds__(kHamSelThreads) void k_ham_select(
    const int32_t* __restrict__ seq_len, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ kept_count, int p_max, int top_k, int Hq, int Hkv, int Lcap,
    const uint16_t* __restrict__ dist, int* __restrict__ hist, int32_t* __restrict__ sel_idx,
    int32_t* __restrict__ sel_count, uint32_t* __restrict__ status, int code_bits) {
  __shared__ HamSmem sm;
  const int bg = blockIdx.x;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  const int L = checked_len(seq_len, b, Lcap, g == 0 ? status : nullptr);
  const int P = kept_pages(kept_count, bg, L, p_max);
  ham_select<kHamSelThreads, false>(b, g, Hq, Hkv, P, top_k, p_max, kept, false, dist, hist,
                                    sel_idx, sel_count, sm, code_bits);
}

}  // namespace

hipError_t launch_page_scores(const hhr_shape& s, const float* q_rot, const int32_t* seq_len,
                              const void* meta, float* scores, uint32_t* status,
                              hipStream_t stream) {
  const int NpCap = s.max_ctx / kPS;
  dim3 grid((NpCap + kScorePagesPerWg - 1) / kScorePagesPerWg, s.batch * s.n_kv_heads);
  if (s.meta_dtype == HHR_BF16)
    hipLaunchKernelGGL(k_page_scores<true>, grid, dim3(256), 0, stream, q_rot, seq_len, meta,
                       scores, status, s.n_q_heads, s.n_kv_heads, s.max_ctx);
  else
    hipLaunchKernelGGL(k_page_scores<false>, grid, dim3(256), 0, stream, q_rot, seq_len, meta,
                       scores, status, s.n_q_heads, s.n_kv_heads, s.max_ctx);
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

hipError_t launch_ham_dist(const hhr_shape& s, const uint32_t* q_codes, const uint32_t* codes,
                           const int32_t* seq_len, const int32_t* kept,
                           const int32_t* kept_count, int32_t p_max, uint16_t* dist, int* hist,
                           uint16_t* cum, hipStream_t stream) {
  const dim3 grid(ham_chunks(p_max), s.batch * s.n_kv_heads);
#define HHR_HAM_DIST(NW)                                                                      \
  hipLaunchKernelGGL(k_ham_dist<NW>, grid, dim3(kHamDistThreads), 0, stream, q_codes, codes, \
                     seq_len, kept, kept_count, p_max, s.n_q_heads, s.n_kv_heads, s.max_ctx, \
                     dist, hist, cum)
  switch (s.code_bits) {
    case 64: HHR_HAM_DIST(2); break;
    case 256: HHR_HAM_DIST(8); break;
    default: HHR_HAM_DIST(4); break;
  }
#undef HHR_HAM_DIST
  return hipGetLastError();
}

hipError_t launch_hamming_topk(const hhr_shape& s, const uint32_t* q_codes, const uint32_t* codes,
                               const int32_t* seq_len, const int32_t* kept,
                               const int32_t* kept_count, int32_t p_max, int32_t top_k,
                               int32_t* sel_idx, int32_t* sel_count, uint16_t* dist, int* hist,
                               uint32_t* status, hipStream_t stream) {
  hipError_t e =
      launch_ham_dist(s, q_codes, codes, seq_len, kept, kept_count, p_max, dist, hist, nullptr,
                      stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_ham_select, dim3(s.batch * s.n_kv_heads), dim3(kHamSelThreads), 0, stream,
                     seq_len, kept, kept_count, p_max, top_k, s.n_q_heads, s.n_kv_heads,
                     s.max_ctx, dist, hist, sel_idx, sel_count, status, s.code_bits);
  return hipGetLastError();
}

}  // namespace hhr
