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

// H2 on MFMA.  A wave takes groups of 16 blocks of one query:
//   D[h][blk] = sum_d e4m3(q8[h][d]) rep[blk][d]
// as 4 head tiles x 4 K-steps of 16x16x32 bf16 MFMAs: the fp8 query is exact
// in bf16, the f32 representative is split into bf16 hi + lo (two MFMAs, f32
// sums).  Then s_blk = sum_h w_h ReLU(q_scale_h D[h][blk]).  Lane (lrow,
// lgrp) holds D of block lrow for heads 16 mt + 4 lgrp + j: it sums its 16
// heads in that order, and two lane-swap adds sum the four lane groups.  The
// workgroup converts the query to bf16 once, into LDS; after that barrier the
// waves are independent, and a wave past the last block stops.
constexpr int kBsWaves = 4;

__device__ __forceinline__ float add_swap32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float add_swap16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__global__ __launch_bounds__(64 * kBsWaves) void k_hisa_block_scores(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const float* __restrict__ w, const float* __restrict__ reps,
    const int32_t* __restrict__ seq_len, float* __restrict__ block_scores,
    uint32_t* __restrict__ status, int Hi, int Lcap, int block, int shared, int gpw) {
  // the query in bf16, converted once per workgroup (rows padded against bank
  // conflicts; heads >= Hi are zero)
  __shared__ __attribute__((aligned(16))) uint16_t sq[kMaxIndexHeads][kD + 8];
  const int b = blockIdx.y;
  const int NbCap = Lcap / block;
  const int wg_blk0 = blockIdx.x * kBsWaves * gpw * 16;
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int l = tid & 63;
  const int lrow = l & 15;
  const int lgrp = l >> 4;
  // The query, its weights and scales and the first group's representatives
  // load before the row's length is known (every address stays inside its
  // buffer; rows past the end are computed and never stored), so they share
  // that round trip.
  constexpr int kQWords = kMaxIndexHeads * kD / 4 / (64 * kBsWaves);
  static_assert(kQWords * 64 * kBsWaves == kMaxIndexHeads * kD / 4, "query words per thread");
  const uint8_t* qb = q8 + (size_t)b * Hi * kD;
  uint32_t qv[kQWords];
#pragma unroll
  for (int k = 0; k < kQWords; ++k) {
    const int i = tid + k * 64 * kBsWaves;
    const int h = i / (kD / 4);
    qv[k] = h < Hi ? *(const uint32_t*)(qb + (size_t)h * kD + 4 * (i % (kD / 4))) : 0u;
  }
  // this lane's 16 heads in the epilogue: 16 mt + 4 lgrp + j
  float wh[4][4], sh[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = 16 * mt + 4 * lgrp + j;
      wh[mt][j] = h < Hi ? w[(size_t)b * Hi + h] : 0.f;
      sh[mt][j] = h < Hi ? q_scale[(size_t)b * Hi + h] : 0.f;
    }
  // B rows: the representative of block blk0 + lrow, dims 32 ks + 8 lgrp + [0, 8)
  const float* repb = reps + (size_t)(shared ? 0 : b) * NbCap * kD;
  floatx4 x0[4], x1[4];
  auto load_reps = [&](int row) {
    const float* rb = repb + (size_t)row * kD;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      x0[ks] = *(const floatx4*)(rb + 32 * ks + 8 * lgrp);
      x1[ks] = *(const floatx4*)(rb + 32 * ks + 8 * lgrp + 4);
    }
  };
  load_reps(min(wg_blk0 + wv * 16 + lrow, NbCap - 1));
  const int L = checked_len(seq_len, b, Lcap, blockIdx.x == 0 ? status : nullptr);
  const int Nb = (L + block - 1) / block;
  if (wg_blk0 >= Nb) return;  // block-uniform, before the barrier
#pragma unroll
  for (int k = 0; k < kQWords; ++k) {
    const int i = tid + k * 64 * kBsWaves;
    const int h = i / (kD / 4);
    const int d = 4 * (i % (kD / 4));
    u32x2 pk;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint32_t lo = __float_as_uint(e4m3fn_to_f32((qv[k] >> (16 * kk)) & 0xFFu)) >> 16;
      const uint32_t hi = __float_as_uint(e4m3fn_to_f32((qv[k] >> (16 * kk + 8)) & 0xFFu)) >> 16;
      pk[kk] = lo | (hi << 16);
    }
    *(u32x2*)&sq[h][d] = pk;
  }
  __syncthreads();
  // A: head 16 mt + lrow, dims 32 ks + 8 lgrp + [0, 8)
  bf16x8 aq[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      aq[mt][ks] = as_bf16x8(*(const u32x4*)&sq[16 * mt + lrow][32 * ks + 8 * lgrp]);
  const float inf = opaque_inf();
  for (int grp = 0; grp < gpw; ++grp) {
    const int blk0 = wg_blk0 + (grp * kBsWaves + wv) * 16;
    if (blk0 >= Nb) break;  // wave-uniform; no barrier follows
    if (grp > 0) load_reps(min(blk0 + lrow, Nb - 1));
    bf16x8 bhi[4], blo[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 hv, lv;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        uint32_t h0, l0, h1, l1;
        split_bf16(jj < 2 ? x0[ks][2 * jj] : x1[ks][2 * jj - 4], h0, l0);
        split_bf16(jj < 2 ? x0[ks][2 * jj + 1] : x1[ks][2 * jj - 3], h1, l1);
        hv[jj] = h0 | (h1 << 16);
        lv[jj] = l0 | (l1 << 16);
      }
      bhi[ks] = as_bf16x8(hv);
      blo[ks] = as_bf16x8(lv);
    }
    floatx4 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[mt][ks], bhi[ks], acc[mt], 0, 0, 0);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[mt][ks], blo[ks], acc[mt], 0, 0, 0);
      }
    }
    float part = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        part = fmaf(wh[mt][j], med_max(acc[mt][j] * sh[mt][j], 0.f, inf), part);
    part = add_swap16(add_swap32(part));
    if (lgrp == 0 && blk0 + lrow < Nb) block_scores[(size_t)b * NbCap + blk0 + lrow] = part;
  }
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
  __shared__ __attribute__((aligned(16))) float sbuf[kHisaMaxCand];  // radix fallback only
  const int cnt = top_strided<kHisaThreads, false>(sc, Nb, Nb, keep_blocks, AllPresent(),
                                                   __builtin_huge_valf(), -__builtin_huge_valf(),
                                                   sbuf, sh, [&](int pos, int c) { out[pos] = c; });
  for (int i = cnt + tid; i < keep_blocks; i += kHisaThreads) out[i] = -1;
  if (tid == 0) kept_count[b] = cnt;
}

// H4: token scores on fp8 MFMA.  A workgroup takes the kept-block slots
// [slot0, slot0 + nslot) of one query row; its waves take the 16-token tiles of
// those blocks in turn.  Per tile, the transposed product
//   D[h][t] = sum_d e4m3(q8[h][d]) e4m3(k8[t][d])   (exact products, f32 sums)
// runs as 4 head tiles x 4 K-steps; lane (lrow, lgrp) holds D for token lrow
// and heads 16 ht + 4 lgrp + j, so
//   s_t = k_scale_t * sum_h (w_h q_scale_h) ReLU(D[h][t])
// (the scales are positive, so they factor out of the ReLU) is 16 in-lane
// steps and two lane-swap adds.  The query's fragments and weights stay in
// registers for all its tiles; each wave keeps the key fragments of its next
// two tiles in flight.
typedef long fp8x8;
constexpr int kTsWaves = 8;

__global__ __launch_bounds__(64 * kTsWaves) void k_hisa_token_scores(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k8,
    const float* __restrict__ k_scale, const int32_t* __restrict__ seq_len,
    const int32_t* __restrict__ kept, const int32_t* __restrict__ kept_count, int keep_blocks,
    float* __restrict__ token_scores, int Hi, int Lcap, int block, int shared, int nslot,
    int nrows, int xcd_rows) {
  // xcd_rows: rows in contiguous runs per XCD (workgroups go round-robin over
  // the eight XCDs; the grid has 8 x ceil(nrows / 8) rows): neighbouring rows
  // keep mostly the same blocks and share an L2
  const int by = blockIdx.y;
  const int b = xcd_rows ? (by % 8) * (gridDim.y / 8) + by / 8 : by;
  if (b >= nrows) return;
  const int slot0 = blockIdx.x * nslot;
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int l = tid & 63;
  const int lrow = l & 15;
  const int lgrp = l >> 4;
  const int tiles_per_block = block / 16;

  // The query's fragments and weights and the block of this wave's first tile
  // load before the row's length and kept count are known (every address
  // stays inside its buffer), so they share that round trip.
  // A: head 16 ht + lrow; this lane's 16 heads for the epilogue: 16 ht + 4 lgrp + j
  fp8x8 aq[4][4];
  float wsq[4][4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const int h = 16 * ht + lrow;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      aq[ht][ks] = h < Hi ? *(const fp8x8*)(q8 + ((size_t)b * Hi + h) * kD + 32 * ks + 8 * lgrp) : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int he = 16 * ht + 4 * lgrp + j;
      wsq[ht][j] = he < Hi ? w[(size_t)b * Hi + he] * q_scale[(size_t)b * Hi + he] : 0.f;
    }
  }
  const int pslot = min(slot0 + wv / tiles_per_block, keep_blocks - 1);
  const int pblk = kept[(size_t)b * keep_blocks + pslot];
  int L = seq_len[b];
  if (L < 0 || L > Lcap) L = 0;
  const int kc = min(kept_count[b], keep_blocks);
  const int slot1 = min(slot0 + nslot, kc);
  if (slot0 >= slot1) return;

  const size_t cb = shared ? 0 : (size_t)b;  // the query row's cache
  const uint8_t* kb = k8 + cb * Lcap * kD;
  const float* ksb = k_scale + cb * Lcap;
  const int ntiles = (slot1 - slot0) * tiles_per_block;
  // key fragments of tile i (token row of this lane; rows past L read row 0)
  auto tile_token = [&](int i) {
    const int slot = slot0 + i / tiles_per_block;
    const int blk = slot == pslot ? pblk : kept[(size_t)b * keep_blocks + slot];
    return blk * block + 16 * (i % tiles_per_block) + lrow;
  };
  auto load_tile = [&](int i, fp8x8 (&kf)[4]) {
    const int t = tile_token(i);
    const size_t row = (t >= 0 && t < L) ? (size_t)t : 0;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kf[ks] = *(const fp8x8*)(kb + row * kD + 32 * ks + 8 * lgrp);
  };
  int i = wv;
  fp8x8 kf[4], k1[4];
  if (i < ntiles) load_tile(i, kf);
  if (i + kTsWaves < ntiles) load_tile(i + kTsWaves, k1);
  for (; i < ntiles; i += kTsWaves) {
    fp8x8 k2[4];
    if (i + 2 * kTsWaves < ntiles) load_tile(i + 2 * kTsWaves, k2);
    floatx4 acc[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      acc[ht] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(aq[ht][ks], kf[ks], acc[ht], 0, 0, 0);
    }
    const int t = tile_token(i);
    const bool valid = t >= 0 && t < L;
    const float sk = valid ? ksb[t] : 0.f;
    const float inf = opaque_inf();
    float part = 0.f;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int j = 0; j < 4; ++j) part = fmaf(wsq[ht][j], med_max(acc[ht][j], 0.f, inf), part);
    part = add_swap16(add_swap32(part)) * sk;
    if (lgrp == 0) {
      const int slot = slot0 + i / tiles_per_block;
      token_scores[((size_t)b * keep_blocks + slot) * block + 16 * (i % tiles_per_block) + lrow] =
          valid ? part : -__builtin_huge_valf();
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      kf[ks] = k1[ks];
      k1[ks] = k2[ks];
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
  const float* ts = token_scores + (size_t)b * keep_blocks * block;
  __shared__ __attribute__((aligned(16))) float sbuf[kHisaMaxCand];  // radix fallback only
  // the kept blocks (for the output positions) load with the scores; the
  // scores load before the kept count is known (clamped to the buffer), and
  // only the first ncand are candidates.  The token-score pass wrote -inf for
  // every slot past the sequence end and a finite score for every token of it.
  auto load_kept = [&]() {
    for (int i = tid; i < kc; i += kHisaThreads) skept[i] = kept[(size_t)b * keep_blocks + i];
  };
  auto present = [](float v) { return v != -__builtin_huge_valf(); };
  int32_t* out = sel_idx + (size_t)b * top_k;
  const int cnt = top_strided<kHisaThreads, false>(
      ts, keep_blocks * block, ncand, top_k, present, __builtin_huge_valf(),
      -__builtin_huge_valf(), sbuf, sh,
      [&](int pos, int c) { out[pos] = skept[c / block] * block + c % block; }, load_kept);
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
  // many queries: each workgroup covers 4 groups of 16 blocks per wave, so the
  // query conversion is shared; few: one group per wave for parallelism
  const int gpw = s.batch >= 64 ? 4 : 1;
  const int per_wg = 16 * kBsWaves * gpw;
  hipLaunchKernelGGL(k_hisa_block_scores, dim3((NbCap + per_wg - 1) / per_wg, s.batch),
                     dim3(64 * kBsWaves), 0, stream, q8, q_scale, w, reps, seq_len, block_scores,
                     status, s.n_index_heads, s.max_ctx, s.block, shared ? 1 : 0, gpw);
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
  // enough workgroups to fill the chip: a run of kept blocks per workgroup,
  // all of a row's blocks once there are many rows
  const int nsplit = std::max(1, std::min<int>(keep_blocks, (512 + s.batch - 1) / s.batch));
  const int nslot = (keep_blocks + nsplit - 1) / nsplit;
  // many rows: spread them over the 8 XCDs in contiguous runs
  const int xcd_rows = s.batch >= 64;
  const int rows = xcd_rows ? (s.batch + 7) / 8 * 8 : s.batch;
  hipLaunchKernelGGL(k_hisa_token_scores, dim3(nsplit, rows), dim3(64 * kTsWaves), 0, stream, q8,
                     q_scale, w, k8, k_scale, seq_len, kept, kept_count, keep_blocks,
                     token_scores, s.n_index_heads, s.max_ctx, s.block, shared ? 1 : 0, nslot,
                     s.batch, xcd_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_hisa_topk, dim3(s.batch), dim3(kHisaThreads), 0, stream, token_scores,
                     seq_len, kept, kept_count, keep_blocks, top_k, sel_idx, sel_count,
                     s.max_ctx, s.block);
  return hipGetLastError();
}

}  // namespace hhr
