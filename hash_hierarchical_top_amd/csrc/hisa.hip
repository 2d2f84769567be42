// HISA hierarchical indexer on gfx950.
//
// [HISA abstract] a DSA-style lightweight indexer scores past tokens for the
// query and keeps a token-level top-k; HISA first scores pooled block
// representatives to drop whole blocks, then runs the original indexer only
// on the tokens of the kept blocks and keeps an exact top-k among them.
// Indexer score: s(x) = sum_h w_h ReLU(qhat_h . x), fp8 e4m3fn operands with
// one positive f32 scale per row.

#include "hhr_device.h"
#include "hhr_internal.h"
#include "topk_device.h"

namespace hhr {

namespace {

constexpr int kMaxIndexHeads = 64;
constexpr int kHisaThreads = 1024;
constexpr int kHisaItems = 16;  // candidates per thread: <= 16384 per query
constexpr int kHisaMaxCand = kHisaThreads * kHisaItems;

// OCP fp8 e4m3fn -> f32: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits
// 2..0; exponent 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN; no infinities.
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t v) {
  const uint32_t sign = (v & 0x80u) << 24;
  const uint32_t e = (v >> 3) & 0xFu;
  const uint32_t m = v & 0x7u;
  float mag;
  if (e == 0) mag = (float)m * 0.001953125f;  // m * 2^-9, exact
  else if (e == 15 && m == 7) mag = __builtin_nanf("");
  else mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return __uint_as_float(__float_as_uint(mag) | sign);
}

__device__ __forceinline__ int checked_len(const int32_t* seq_len, int b, int Lcap,
                                           uint32_t* status) {
  const int L = seq_len[b];
  if (L < 0 || L > Lcap) {
    if (status && threadIdx.x == 0) atomicOr(status, HHR_DEV_BAD_SEQ_LEN);
    return 0;
  }
  return L;
}

// H1: one workgroup (128 threads = dims) per touched block.
__global__ __launch_bounds__(kD) void k_hisa_pool(const uint8_t* __restrict__ k8,
                                                  const float* __restrict__ k_scale,
                                                  const int32_t* __restrict__ start,
                                                  const int32_t* __restrict__ n_new,
                                                  float* __restrict__ reps,
                                                  uint32_t* __restrict__ status, int Lcap,
                                                  int block) {
  const int b = blockIdx.y;
  const int s = start[b];
  const int n = n_new[b];
  if (s < 0 || n < 0 || (long long)s + n > Lcap) {
    if (status && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(status, HHR_DEV_BAD_SEQ_LEN);
    return;
  }
  if (n == 0) return;
  const int e = s + n;
  const int blk = s / block + blockIdx.x;
  if (blk > (e - 1) / block) return;
  const int r0 = blk * block;
  const int r1 = min(r0 + block, e);
  const int d = threadIdx.x;
  const uint8_t* kb = k8 + (size_t)b * Lcap * kD;
  const float* sb = k_scale + (size_t)b * Lcap;
  float acc = 0.f;
  for (int t = r0; t < r1; ++t) acc = fmaf(sb[t], e4m3fn_to_f32(kb[(size_t)t * kD + d]), acc);
  reps[((size_t)b * (Lcap / block) + blk) * kD + d] = acc / (float)(r1 - r0);
}

// H2: 16 blocks per workgroup; thread (bl = tid/16, hg = tid%16) takes heads
// hg, hg+16, hg+32, hg+48 of block bl, and the 16 threads of a block reduce.
// shared: every query row b reads the one cache (row 0) of reps, as in prefill.
__global__ __launch_bounds__(256) void k_hisa_block_scores(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const float* __restrict__ w, const float* __restrict__ reps,
    const int32_t* __restrict__ seq_len, float* __restrict__ block_scores,
    uint32_t* __restrict__ status, int Hi, int Lcap, int block, int shared) {
  __shared__ float sq[kMaxIndexHeads][kD + 1];
  __shared__ float srep[16][kD];
  const int b = blockIdx.y;
  const int L = checked_len(seq_len, b, Lcap, blockIdx.x == 0 ? status : nullptr);
  const int Nb = (L + block - 1) / block;
  const int NbCap = Lcap / block;
  const int blk0 = blockIdx.x * 16;
  if (blk0 >= Nb) return;
  const int tid = threadIdx.x;
  for (int i = tid; i < Hi * kD; i += 256) {
    const int h = i / kD, d = i % kD;
    sq[h][d] = q_scale[(size_t)b * Hi + h] * e4m3fn_to_f32(q8[((size_t)b * Hi + h) * kD + d]);
  }
  for (int i = tid; i < 16 * kD; i += 256) {
    const int bl = i / kD, d = i % kD;
    srep[bl][d] =
        (blk0 + bl < Nb) ? reps[((size_t)(shared ? 0 : b) * NbCap + blk0 + bl) * kD + d] : 0.f;
  }
  __syncthreads();
  const int bl = tid >> 4;
  const int hg = tid & 15;
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = hg + 16 * i;
    if (h < Hi) {
      float dot = 0.f;
#pragma unroll 8
      for (int d = 0; d < kD; ++d) dot = fmaf(sq[h][d], srep[bl][d], dot);
      part = fmaf(w[(size_t)b * Hi + h], fmaxf(dot, 0.f), part);
    }
  }
  part = row_sum16(part);
  if (hg == 0 && blk0 + bl < Nb) block_scores[(size_t)b * NbCap + blk0 + bl] = part;
}

// H3: exact top keep_blocks blocks of one query (thread tid takes a run of consecutive blocks).
__global__ __launch_bounds__(kHisaThreads) void k_hisa_top_blocks(
    const float* __restrict__ block_scores, const int32_t* __restrict__ seq_len,
    int keep_blocks, int32_t* __restrict__ kept, int32_t* __restrict__ kept_count,
    uint32_t* __restrict__ status, int Lcap, int block) {
  __shared__ TopScratch sh;
  const int b = blockIdx.x;
  const int L = checked_len(seq_len, b, Lcap, status);
  const int Nb = (L + block - 1) / block;
  const int NbCap = Lcap / block;
  const int tid = threadIdx.x;
  int32_t* out = kept + (size_t)b * keep_blocks;
  const float* sc = block_scores + (size_t)b * NbCap;
  __shared__ __attribute__((aligned(16))) float sbuf[kHisaMaxCand];
#pragma unroll
  for (int i = 0; i < kHisaItems; ++i) {
    const int c = i * kHisaThreads + tid;
    sbuf[c] = sc[min(c, max(Nb - 1, 0))];
  }
  __syncthreads();
  const int cnt = top_largest_lds<kHisaThreads, kHisaMaxCand / (4 * kHisaThreads)>(
      sbuf, Nb, [](int) { return true; }, keep_blocks, sh,
      [&](int pos, int c) { out[pos] = c; });
  for (int i = cnt + tid; i < keep_blocks; i += kHisaThreads) out[i] = -1;
  if (tid == 0) kept_count[b] = cnt;
}

// H4: token scores of one kept block on fp8 MFMA.  D[token][head] =
// sum_d e4m3(k8[token][d]) e4m3(q8[head][d]) (exact products, f32 sums), then
// s_t = sum_h w_h ReLU(D * (q_scale_h * k_scale_t)).  Wave w takes the
// 16-token tiles w, w+4, ... of the block; 4 head tiles x 4 K-steps per tile.
typedef long fp8x8;

__global__ __launch_bounds__(256) void k_hisa_token_scores(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k8,
    const float* __restrict__ k_scale, const int32_t* __restrict__ seq_len,
    const int32_t* __restrict__ kept, const int32_t* __restrict__ kept_count, int keep_blocks,
    float* __restrict__ token_scores, int Hi, int Lcap, int block, int shared) {
  const int b = blockIdx.y;
  const int slot = blockIdx.x;
  int L = seq_len[b];
  if (L < 0 || L > Lcap) L = 0;
  const int kc = min(kept_count[b], keep_blocks);
  if (slot >= kc) return;
  const int blk = kept[(size_t)b * keep_blocks + slot];
  if (blk < 0) return;
  const int t0 = blk * block;
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int l = tid & 63;
  const int lrow = l & 15;
  const int lgrp = l >> 4;

  fp8x8 bq[4][4];
  float wq[4], sqh[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int h = 16 * nt + lrow;
    wq[nt] = h < Hi ? w[(size_t)b * Hi + h] : 0.f;
    sqh[nt] = h < Hi ? q_scale[(size_t)b * Hi + h] : 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      bq[nt][ks] = h < Hi ? *(const fp8x8*)(q8 + ((size_t)b * Hi + h) * kD + 32 * ks + 8 * lgrp) : 0;
  }
  const size_t cb = shared ? 0 : (size_t)b;  // the query row's cache
  const uint8_t* kb = k8 + cb * Lcap * kD;
  const float* ksb = k_scale + cb * Lcap;
  float* ts = token_scores + ((size_t)b * keep_blocks + slot) * block;
  const int ntile = block / 16;
  for (int mt = wv; mt < ntile; mt += 4) {
    const int ta = t0 + 16 * mt + lrow;  // A row of this lane
    fp8x8 a[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      a[ks] = ta < L ? *(const fp8x8*)(kb + (size_t)ta * kD + 32 * ks + 8 * lgrp) : 0;
    floatx4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a[ks], bq[nt][ks], acc[nt], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = t0 + 16 * mt + 4 * lgrp + j;
      const float sk = tt < L ? ksb[tt] : 0.f;
      float part = 0.f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        part = fmaf(wq[nt], fmaxf(acc[nt][j] * (sqh[nt] * sk), 0.f), part);
      part = row_sum16(part);
      if (lrow == 0) ts[16 * mt + 4 * lgrp + j] = tt < L ? part : -__builtin_huge_valf();
    }
  }
}

// H5: exact top-k over the kept blocks' valid tokens by (larger s, lower t);
// candidate c = (kept slot c / block, row c % block).  Kept blocks are
// ascending, so candidate order is position order and ties go to the lower
// position.
__global__ __launch_bounds__(kHisaThreads) void k_hisa_topk(
    const float* __restrict__ token_scores, const int32_t* __restrict__ seq_len,
    const int32_t* __restrict__ kept, const int32_t* __restrict__ kept_count, int keep_blocks,
    int top_k, int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_count, int Lcap,
    int block) {
  __shared__ TopScratch sh;
  __shared__ int skept[kHisaMaxCand / 16];
  const int b = blockIdx.x;
  int L = seq_len[b];
  if (L < 0 || L > Lcap) L = 0;
  const int kc = L > 0 ? min(kept_count[b], keep_blocks) : 0;
  const int ncand = kc * block;
  const int tid = threadIdx.x;
  for (int i = tid; i < kc; i += kHisaThreads) skept[i] = kept[(size_t)b * keep_blocks + i];
  __syncthreads();
  const float* ts = token_scores + (size_t)b * keep_blocks * block;
  __shared__ __attribute__((aligned(16))) float sbuf[kHisaMaxCand];
#pragma unroll
  for (int i = 0; i < kHisaItems; ++i) {
    const int c = i * kHisaThreads + tid;
    sbuf[c] = ts[min(c, max(ncand - 1, 0))];
  }
  __syncthreads();
  auto present = [&](int c) {
    const int blk = skept[c / block];
    return blk >= 0 && blk * block + c % block < L;
  };
  int32_t* out = sel_idx + (size_t)b * top_k;
  const int cnt = top_largest_lds<kHisaThreads, kHisaMaxCand / (4 * kHisaThreads)>(
      sbuf, ncand, present, top_k, sh,
      [&](int pos, int c) { out[pos] = skept[c / block] * block + c % block; });
  for (int i = cnt + tid; i < top_k; i += kHisaThreads) out[i] = -1;
  if (tid == 0) sel_count[b] = cnt;
}

}  // namespace

hipError_t launch_hisa_pool(const hhr_hisa_shape& s, const uint8_t* k8, const float* k_scale,
                            const int32_t* start, const int32_t* n_new, int32_t max_new,
                            float* reps, uint32_t* status, hipStream_t stream) {
  if (max_new <= 0) return hipSuccess;
  const int touched = (max_new + s.block - 1) / s.block + 1;
  hipLaunchKernelGGL(k_hisa_pool, dim3(touched, s.batch), dim3(kD), 0, stream, k8, k_scale,
                     start, n_new, reps, status, s.max_ctx, s.block);
  return hipGetLastError();
}

hipError_t launch_hisa_block_scores(const hhr_hisa_shape& s, const uint8_t* q8,
                                    const float* q_scale, const float* w, const float* reps,
                                    const int32_t* seq_len, float* block_scores,
                                    uint32_t* status, hipStream_t stream, bool shared) {
  const int NbCap = s.max_ctx / s.block;
  hipLaunchKernelGGL(k_hisa_block_scores, dim3((NbCap + 15) / 16, s.batch), dim3(256), 0, stream,
                     q8, q_scale, w, reps, seq_len, block_scores, status, s.n_index_heads,
                     s.max_ctx, s.block, shared ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_hisa_top_blocks(const hhr_hisa_shape& s, const float* block_scores,
                                  const int32_t* seq_len, int32_t keep_blocks, int32_t* kept,
                                  int32_t* kept_count, uint32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(k_hisa_top_blocks, dim3(s.batch), dim3(kHisaThreads), 0, stream,
                     block_scores, seq_len, keep_blocks, kept, kept_count, status, s.max_ctx,
                     s.block);
  return hipGetLastError();
}

hipError_t launch_hisa_token_topk(const hhr_hisa_shape& s, const uint8_t* q8,
                                  const float* q_scale, const float* w, const uint8_t* k8,
                                  const float* k_scale, const int32_t* seq_len,
                                  const int32_t* kept, const int32_t* kept_count,
                                  int32_t keep_blocks, int32_t top_k, int32_t* sel_idx,
                                  int32_t* sel_count, float* token_scores, uint32_t* status,
                                  hipStream_t stream, bool shared) {
  (void)status;
  hipLaunchKernelGGL(k_hisa_token_scores, dim3(keep_blocks, s.batch), dim3(256), 0, stream, q8,
                     q_scale, w, k8, k_scale, seq_len, kept, kept_count, keep_blocks,
                     token_scores, s.n_index_heads, s.max_ctx, s.block, shared ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_hisa_topk, dim3(s.batch), dim3(kHisaThreads), 0, stream, token_scores,
                     seq_len, kept, kept_count, keep_blocks, top_k, sel_idx, sel_count,
                     s.max_ctx, s.block);
  return hipGetLastError();
}

}  // namespace hhr
