// HISA hierarchical indexer on gfx950.
//
// [HISA abstract] a DSA-style lightweight indexer scores past tokens for the
// query and keeps a token-level top-k; HISA first scores pooled block
// representatives to drop whole blocks, then runs the original indexer only
// on the tokens of the kept blocks and keeps an exact top-k among them.
// Indexer score: s(x) = sum_h w_h ReLU(qhat_h . x), fp8 e4m3fn operands with
// one positive f32 scale per row.

#include <type_traits>

#include "hhr_device.h"
#include "hhr_internal.h"
#include "topk_device.h"

namespace hhr {

namespace {

constexpr int kMaxIndexHeads = 64;
constexpr int kHisaThreads = 1024;
constexpr int kHisaItems = 16;  // candidates per thread: <= 16384 per query
constexpr int kHisaMaxCand = kHisaThreads * kHisaItems;

// OCP fp8 e4m3fn -> f32 (exact): sign bit 7, exponent bits 6..3 (bias 7), mantissa
// bits 2..0; exponent 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN; no infinities.
// On gfx950 v_cvt_f32_fp8 decodes this format: one instruction for the field decode
// (the same bits for all 256 codes).  v holds the code in its low byte.
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t v) {
  return __builtin_amdgcn_cvt_f32_fp8((int)v, 0);
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

// Mean of dimension d over index-key rows [r0, r1) (r1 > r0) of one cache:
// sum_t k_scale[t] * e4m3(k8[t][d]) accumulated in row order, then divided by
// the row count.  Both the block pooling and a prefill row's partly visible
// block use it, so equal rows give bit-identical means.  The workgroup (128
// threads = dims) stages the rows in LDS, kPoolRows at a time with every
// thread's 16-byte loads in flight together; then each thread runs its chain.
// All threads call (barriers).
constexpr int kPoolRows = 128;

struct PoolSmem {
  __attribute__((aligned(16))) uint8_t k[kPoolRows][kD];
  float s[kPoolRows];
};

__device__ __forceinline__ float pool_mean(const uint8_t* __restrict__ kb,
                                           const float* __restrict__ sb, int r0, int r1,
                                           PoolSmem& sm) {
  constexpr int kChunks = kPoolRows * kD / 16 / kD;  // 16-byte loads per thread per round
  const int d = threadIdx.x;
  float acc = 0.f;
  for (int c0 = r0; c0 < r1; c0 += kPoolRows) {  // block-uniform
    const int n = min(kPoolRows, r1 - c0);
    u32x4 v[kChunks];
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int e = d + kD * i;  // 16-byte piece e of the round: row e / 8, piece e % 8
      v[i] = *(const u32x4*)(kb + (size_t)(c0 + min(e / 8, n - 1)) * kD + 16 * (e % 8));
    }
    const float sc = sb[c0 + min(d, n - 1)];
    __syncthreads();  // the previous round's LDS reads are done
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int e = d + kD * i;
      *(u32x4*)&sm.k[e / 8][16 * (e % 8)] = v[i];
    }
    sm.s[d] = sc;
    __syncthreads();
#pragma unroll 8
    for (int t = 0; t < n; ++t) acc = fmaf(sm.s[t], e4m3fn_to_f32(sm.k[t][d]), acc);
  }
  return acc / (float)(r1 - r0);
}

// H1: one workgroup (128 threads = dims) per touched block.
__global__ __launch_bounds__(kD) void k_hisa_pool(const uint8_t* __restrict__ k8,
                                                  const float* __restrict__ k_scale,
                                                  const int32_t* __restrict__ start,
                                                  const int32_t* __restrict__ n_new,
                                                  float* __restrict__ reps,
                                                  uint32_t* __restrict__ status, int Lcap,
                                                  int block) {
  __shared__ PoolSmem sm;
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
  const float m = pool_mean(k8 + (size_t)b * Lcap * kD, k_scale + (size_t)b * Lcap, r0, r1, sm);
  reps[((size_t)b * (Lcap / block) + blk) * kD + d] = m;
}

// Prefill rows against one shared cache: row r sees tokens t < q_len[r], so
// when q_len[r] is not a multiple of the block, its last block is only partly
// visible and is represented by the mean of its visible rows
// [block * floor(q_len / block), q_len) alone, never by the cache's pooled
// block (which holds later keys).  One workgroup (128 threads = dims) per row
// writes that mean to tail[r]; rows ending on a block edge write nothing.
__global__ __launch_bounds__(kD) void k_hisa_pool_tail(const uint8_t* __restrict__ k8,
                                                       const float* __restrict__ k_scale,
                                                       const int32_t* __restrict__ q_len,
                                                       float* __restrict__ tail, int Lcap,
                                                       int block) {
  __shared__ PoolSmem sm;
  const int r = blockIdx.x;
  const int L = q_len[r];
  if (L <= 0 || L > Lcap || L % block == 0) return;  // bad lengths: the scorer flags them
  const int r0 = L / block * block;
  tail[(size_t)r * kD + threadIdx.x] = pool_mean(k8, k_scale, r0, L, sm);
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

// TOP: H3 in the same launch.  Every workgroup publishes its block scores
// (agent-scope stores) and counts in on its row's counter; the last one to
// arrive takes the row's top keep_blocks blocks (as k_hisa_top_blocks does,
// with this workgroup's threads), so H3 needs no launch of its own.  Only for
// rows of at most kBsTopMax blocks.
constexpr int kBsTopWaves = 8;  // with H3 (16 would spill: 128 VGPRs at 1024 threads)
constexpr int kBsTopMax = 16 * 64 * kBsTopWaves;  // top_strided's limit at that width

struct BsTopSmem {
  __attribute__((aligned(16))) float sbuf[kBsTopMax];  // radix fallback only
  TopScratch sh;
};

template <int WAVES, bool TOP>
__global__ __launch_bounds__(64 * WAVES) void k_hisa_block_scores(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const float* __restrict__ w, const float* __restrict__ reps,
    const int32_t* __restrict__ seq_len, const float* __restrict__ tail,
    float* __restrict__ block_scores, uint32_t* __restrict__ status, int Hi, int Lcap, int block,
    int shared, int gpw, int keep_blocks, int32_t* __restrict__ kept,
    int32_t* __restrict__ kept_count, uint32_t* __restrict__ counters) {
  // the query in bf16, converted once per workgroup (rows padded against bank
  // conflicts; heads >= Hi are zero)
  __shared__ __attribute__((aligned(16))) uint16_t sq[kMaxIndexHeads][kD + 8];
  __shared__ typename std::conditional<TOP, BsTopSmem, char>::type top_sm;
  __shared__ int s_last;
  const int b = blockIdx.y;
  const int NbCap = Lcap / block;
  const int wg_blk0 = blockIdx.x * WAVES * gpw * 16;
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int l = tid & 63;
  const int lrow = l & 15;
  const int lgrp = l >> 4;
  // The query, its weights and scales and the first group's representatives
  // load before the row's length is known (every address stays inside its
  // buffer; rows past the end are computed and never stored), so they share
  // that round trip.
  constexpr int kQWords = kMaxIndexHeads * kD / 4 / (64 * WAVES);
  static_assert(kQWords * 64 * WAVES == kMaxIndexHeads * kD / 4, "query words per thread");
  const uint8_t* qb = q8 + (size_t)b * Hi * kD;
  uint32_t qv[kQWords];
#pragma unroll
  for (int k = 0; k < kQWords; ++k) {
    const int i = tid + k * 64 * WAVES;
    const int h = min(i / (kD / 4), Hi - 1);
    qv[k] = *(const uint32_t*)(qb + (size_t)h * kD + 4 * (i % (kD / 4)));
  }
  // the weights and scales once per workgroup (one load per thread, zero past
  // Hi), into LDS after the barrier below; lane (lrow, lgrp) takes those of
  // its 16 epilogue heads 16 mt + 4 lgrp + j from there
  __shared__ float sw[kMaxIndexHeads], ss[kMaxIndexHeads];
  float w_ = 0.f, s_ = 0.f;
  if (tid < Hi) {
    w_ = w[(size_t)b * Hi + tid];
    s_ = q_scale[(size_t)b * Hi + tid];
  }
  issue_loads_here();
#pragma unroll
  for (int k = 0; k < kQWords; ++k)
    if ((tid + k * 64 * WAVES) / (kD / 4) >= Hi) qv[k] = 0u;
  // B rows: the representative of block blk0 + lrow, dims 32 ks + 8 lgrp + [0, 8).
  // Shared cache (prefill rows): a row's partly visible last block is its own
  // tail mean (k_hisa_pool_tail), not the cache's pooled block.
  const float* repb = reps + (size_t)(shared ? 0 : b) * NbCap * kD;
  floatx4 x0[4], x1[4];
  auto load_rep_row = [&](const float* rb) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      x0[ks] = *(const floatx4*)(rb + 32 * ks + 8 * lgrp);
      x1[ks] = *(const floatx4*)(rb + 32 * ks + 8 * lgrp + 4);
    }
  };
  load_rep_row(repb + (size_t)min(wg_blk0 + wv * 16 + lrow, NbCap - 1) * kD);
  const int L = checked_len(seq_len, b, Lcap, blockIdx.x == 0 ? status : nullptr);
  const int Nb = (L + block - 1) / block;
  // the block (of this launch's row b) whose representative is the row's tail mean, or -1
  const int tail_blk = shared && L % block != 0 ? Nb - 1 : -1;
  auto load_reps = [&](int row) {
    load_rep_row(row == tail_blk ? tail + (size_t)b * kD : repb + (size_t)row * kD);
  };
  if (!TOP && wg_blk0 >= Nb) return;  // block-uniform, before the barrier
  if (wg_blk0 + wv * 16 + lrow == tail_blk) load_reps(tail_blk);
#pragma unroll
  for (int k = 0; k < kQWords; ++k) {
    const int i = tid + k * 64 * WAVES;
    const int h = i / (kD / 4);
    const int d = 4 * (i % (kD / 4));
    u32x2 pk;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint32_t lo = __float_as_uint(e4m3fn_to_f32(qv[k] >> (16 * kk))) >> 16;
      const uint32_t hi = __float_as_uint(e4m3fn_to_f32(qv[k] >> (16 * kk + 8))) >> 16;
      pk[kk] = lo | (hi << 16);
    }
    *(u32x2*)&sq[h][d] = pk;
  }
  if (tid < kMaxIndexHeads) {
    sw[tid] = w_;
    ss[tid] = s_;
  }
  __syncthreads();
  float wh[4][4], sh[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wh[mt][j] = sw[16 * mt + 4 * lgrp + j];
      sh[mt][j] = ss[16 * mt + 4 * lgrp + j];
    }
  // A: head 16 mt + lrow, dims 32 ks + 8 lgrp + [0, 8)
  bf16x8 aq[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      aq[mt][ks] = as_bf16x8(*(const u32x4*)&sq[16 * mt + lrow][32 * ks + 8 * lgrp]);
  const float inf = opaque_inf();
  for (int grp = 0; grp < gpw; ++grp) {
    const int blk0 = wg_blk0 + (grp * WAVES + wv) * 16;
    if (blk0 >= Nb) break;  // wave-uniform; no barrier follows
    if (grp > 0) load_reps(min(blk0 + lrow, Nb - 1));
    bf16x8 bhi[4], blo[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 hv, lv;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const u32x2 hl = split_bf16x2(jj < 2 ? x0[ks][2 * jj] : x1[ks][2 * jj - 4],
                                      jj < 2 ? x0[ks][2 * jj + 1] : x1[ks][2 * jj - 3]);
        hv[jj] = hl[0];
        lv[jj] = hl[1];
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
    if (lgrp == 0 && blk0 + lrow < Nb) Mem<TOP>::st(block_scores + (size_t)b * NbCap + blk0 + lrow, part);
  }
  if constexpr (TOP) {
    if (!arrive_last(counters + (size_t)b * kHisaCounters, gridDim.x, &s_last)) return;
    // H3 of row b from every workgroup's published scores
    int32_t* out = kept + (size_t)b * keep_blocks;
    const int cnt = top_strided<64 * WAVES, true>(
        block_scores + (size_t)b * NbCap, Nb, Nb, keep_blocks, AllPresent(),
        __builtin_huge_valf(), -__builtin_huge_valf(), top_sm.sbuf, top_sm.sh,
        [&](int pos, int c) { out[pos] = c; });
    for (int i = cnt + tid; i < keep_blocks; i += 64 * WAVES) out[i] = -1;
    if (tid == 0) kept_count[b] = cnt;
  }
}

// H3: exact top keep_blocks blocks of one query (thread tid takes a run of consecutive blocks).
template <int NVMAX>
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
  __shared__ __attribute__((aligned(16))) float sbuf[kHisaThreads * NVMAX];  // radix fallback only
  auto emit = [&](int pos, int c) { out[pos] = c; };
  const int cnt = top_strided<kHisaThreads, false, AllPresent, decltype(emit), NoMid, NVMAX>(
      sc, Nb, Nb, keep_blocks, AllPresent(), __builtin_huge_valf(), -__builtin_huge_valf(), sbuf,
      sh, emit);
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
//
// TOPK: H5 in the same launch (few rows).  Every workgroup publishes its token
// scores (agent-scope stores) and counts in on its row's counter; the last to
// arrive takes the row's exact top-k as k_hisa_topk does, with its 16 waves.
typedef long fp8x8;
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
constexpr int kTsWaves = 8;      // the plain variant
constexpr int kTsTopWaves = 16;  // with H5: k_hisa_topk's width

struct TsTopSmem {
  __attribute__((aligned(16))) float sbuf[kHisaMaxCand];  // radix fallback only
  TopScratch sh;
};

template <int WAVES, bool TOPK>
__global__ __launch_bounds__(64 * WAVES) void k_hisa_token_scores(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k8,
    const float* __restrict__ k_scale, const int32_t* __restrict__ seq_len,
    const int32_t* __restrict__ kept, const int32_t* __restrict__ kept_count, int keep_blocks,
    float* __restrict__ token_scores, int Hi, int Lcap, int block, int shared, int nslot,
    int nrows, int xcd_rows, int top_k, int32_t* __restrict__ sel_idx,
    int32_t* __restrict__ sel_count, uint32_t* __restrict__ counters) {
  static_assert(!TOPK || 64 * WAVES == kHisaThreads, "H5 runs at k_hisa_topk's width");
  constexpr int kTsWavesT = WAVES;
  __shared__ typename std::conditional<TOPK, TsTopSmem, char>::type top_sm;
  __shared__ int s_last;
  // xcd_rows: rows in contiguous runs per XCD (workgroups go round-robin over
  // the eight XCDs; the grid has 8 x ceil(nrows / 8) rows): neighbouring rows
  // keep mostly the same blocks and share an L2
  const int by = blockIdx.y;
  const int b = xcd_rows ? (by % 8) * (gridDim.y / 8) + by / 8 : by;
  if (b >= nrows) return;
  const int slot0 = blockIdx.x * nslot;
  const int tid = threadIdx.x;
  __shared__ int skb[kHisaMaxCand / 16];  // kept blocks of this workgroup's slots
  const int wv = tid >> 6;
  const int l = tid & 63;
  const int lrow = l & 15;
  const int lgrp = l >> 4;
  const int tiles_per_block = block / 16;

  // The query (fp8, Hi x 128 bytes), its weights and scales and this
  // workgroup's kept blocks load once per workgroup, coalesced and all
  // together, before the row's length and kept count are known (addresses
  // clamped into the buffers); the waves then take their fragments from LDS.
  __shared__ __attribute__((aligned(16))) uint8_t sq8[kMaxIndexHeads][kD + 16];
  __shared__ float swsq[kMaxIndexHeads];
  u32x4 qc = {0u, 0u, 0u, 0u};
  const int nq16 = Hi * kD / 16;  // 16-byte chunks of the query
  if (tid < nq16) qc = *(const u32x4*)(q8 + (size_t)b * Hi * kD + 16 * tid);
  float wv_ = 0.f, sv_ = 0.f;
  if (tid < Hi) {
    wv_ = w[(size_t)b * Hi + tid];
    sv_ = q_scale[(size_t)b * Hi + tid];
  }
  int L = seq_len[b];
  const int kc = min(kept_count[b], keep_blocks);
  // (a run longer than the workgroup, prefill only, takes further rounds)
  for (int i = tid; i < nslot; i += 64 * WAVES)
    skb[i] = kept[(size_t)b * keep_blocks + min(slot0 + i, keep_blocks - 1)];
  if (tid < nq16) *(u32x4*)&sq8[(16 * tid) / kD][(16 * tid) % kD] = qc;
  if (tid < kMaxIndexHeads) swsq[tid] = tid < Hi ? wv_ * sv_ : 0.f;
  __syncthreads();
  // A: head 16 ht + lrow (zero past Hi); this lane's 16 heads for the
  // epilogue: 16 ht + 4 lgrp + j.  The k-step ks of lane group lgrp takes dims
  // 32 lgrp + 8 ks .. + 7 (in A as in B), so that a lane's four key fragments
  // are 32 contiguous bytes of its row, two 16-byte loads.
  fp8x8 aq[4][4];
  float wsq[4][4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const bool hv = 16 * ht + lrow < Hi;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      aq[ht][ks] = hv ? *(const fp8x8*)&sq8[16 * ht + lrow][32 * lgrp + 8 * ks] : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) wsq[ht][j] = swsq[16 * ht + 4 * lgrp + j];
  }
  if (L < 0 || L > Lcap) L = 0;
  const int slot1 = min(slot0 + nslot, kc);
  if (!TOPK && slot0 >= slot1) return;
  if (slot0 < slot1) {  // block-uniform
  const size_t cb = shared ? 0 : (size_t)b;  // the query row's cache
  const uint8_t* kb = k8 + cb * Lcap * kD;
  const float* ksb = k_scale + cb * Lcap;
  const int ntiles = (slot1 - slot0) * tiles_per_block;
  auto tile_token = [&](int i) {
    return skb[i / tiles_per_block] * block + 16 * (i % tiles_per_block) + lrow;
  };
  // key fragments of tile i (token row of this lane; rows past L read row 0)
  auto load_keys = [&](int i, fp8x8 (&kf)[4]) {
    const int t = tile_token(i);
    const size_t row = (t >= 0 && t < L) ? (size_t)t : 0;
    const u64x2* src = (const u64x2*)(kb + row * kD + 32 * lgrp);
    const u64x2 lo = src[0], hi = src[1];
    kf[0] = (fp8x8)lo[0];
    kf[1] = (fp8x8)lo[1];
    kf[2] = (fp8x8)hi[0];
    kf[3] = (fp8x8)hi[1];
  };
  // The wave's tiles i, i + W, ... go in groups of four, tile j of a group in
  // key buffer j, loaded two tiles ahead.  While every load of a group is in
  // range (all but the last group or two) the group runs without guards: a
  // guarded load leaves the compiler a join after which it can only wait for
  // every load in flight.  Lane group lgrp loads the key scale of its row of
  // the group's tile lgrp and stores that tile's score (after the lane-swap
  // sums every lane holds its row's sum), so that a group costs one scale load
  // and one store instead of four each.
  constexpr int W = kTsWavesT;
  fp8x8 kf[4][4];
  // this lane's tile of the group at i, and its token (-1 past the tiles)
  auto lane_token = [&](int i) {
    const int ti = i + lgrp * W;
    return ti < ntiles ? tile_token(ti) : -1;
  };
  auto scale_at = [&](int i) {  // issued a group ahead of its use
    const int tt = lane_token(i);
    return ksb[(tt >= 0 && tt < L) ? tt : 0];
  };
  auto run_group = [&](int i, float skr, auto guarded) {
    constexpr bool kGuard = decltype(guarded)::value;
    float out = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!kGuard || i + (j + 2) * W < ntiles) load_keys(i + (j + 2) * W, kf[(j + 2) % 4]);
      if (!kGuard || i + j * W < ntiles) {  // wave-uniform
        floatx4 acc[4];
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
          acc[ht] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(aq[ht][ks], kf[j][ks], acc[ht],
                                                                 0, 0, 0);
        }
        const float inf = opaque_inf();
        float part = 0.f;
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            part = fmaf(wsq[ht][jj], med_max(acc[ht][jj], 0.f, inf), part);
        part = add_swap16(add_swap32(part));
        if (lgrp == j) out = part;
      }
    }
    const int ti = i + lgrp * W;
    if (ti < ntiles) {
      const int tt = tile_token(ti);
      const int slot = slot0 + ti / tiles_per_block;
      Mem<TOPK>::st(
          token_scores + ((size_t)b * keep_blocks + slot) * block + 16 * (ti % tiles_per_block) +
              lrow,
          tt >= 0 && tt < L ? out * skr : -__builtin_huge_valf());
    }
  };
  int i = wv;
  if constexpr (TOPK) {
    // a decode row: a tile or two per wave, each tile's keys and scale loaded
    // together two tiles ahead
    auto load_tile = [&](int i, fp8x8 (&k)[4], float& sc) {
      load_keys(i, k);
      const int t = tile_token(i);
      sc = ksb[(t >= 0 && t < L) ? t : 0];
    };
    fp8x8 k0[4], k1[4];
    float s0 = 0.f, s1 = 0.f;
    if (i < ntiles) load_tile(i, k0, s0);
    if (i + W < ntiles) load_tile(i + W, k1, s1);
    for (; i < ntiles; i += W) {
      fp8x8 k2[4];
      float s2 = 0.f;
      if (i + 2 * W < ntiles) load_tile(i + 2 * W, k2, s2);
      floatx4 acc[4];
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        acc[ht] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc[ht] =
              __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(aq[ht][ks], k0[ks], acc[ht], 0, 0, 0);
      }
      const int t = tile_token(i);
      const bool valid = t >= 0 && t < L;
      const float inf = opaque_inf();
      float part = 0.f;
#pragma unroll
      for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          part = fmaf(wsq[ht][jj], med_max(acc[ht][jj], 0.f, inf), part);
      part = add_swap16(add_swap32(part)) * (valid ? s0 : 0.f);
      if (lgrp == 0)
        Mem<TOPK>::st(token_scores + ((size_t)b * keep_blocks + slot0 + i / tiles_per_block) *
                                         block +
                          16 * (i % tiles_per_block) + lrow,
                      valid ? part : -__builtin_huge_valf());
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        k0[ks] = k1[ks];
        k1[ks] = k2[ks];
      }
      s0 = s1;
      s1 = s2;
    }
  } else {
    if (i < ntiles) load_keys(i, kf[0]);
    if (i + W < ntiles) load_keys(i + W, kf[1]);
    float skr = scale_at(i);
    for (; i + 5 * W < ntiles; i += 4 * W) {
      const float next = scale_at(i + 4 * W);
      run_group(i, skr, std::false_type{});
      skr = next;
    }
    for (; i < ntiles; i += 4 * W) {
      const float next = scale_at(i + 4 * W);
      run_group(i, skr, std::true_type{});
      skr = next;
    }
  }
  }
  if constexpr (TOPK) {
    if (!arrive_last(counters + (size_t)b * kHisaCounters + 1, gridDim.x, &s_last)) return;
    // H5 of row b from every workgroup's published scores (k_hisa_topk's steps)
    const int kcv = L > 0 ? kc : 0;
    const int ncand = kcv * block;
    const float* ts = token_scores + (size_t)b * keep_blocks * block;
    auto load_kept = [&]() {  // skb is free now: all of the row's kept blocks
      for (int i = tid; i < kcv; i += 64 * WAVES) skb[i] = kept[(size_t)b * keep_blocks + i];
    };
    auto present = [](float v) { return v != -__builtin_huge_valf(); };
    int32_t* out = sel_idx + (size_t)b * top_k;
    __syncthreads();  // every wave is done with skb
    const int cnt = top_strided<64 * WAVES, true>(
        ts, keep_blocks * block, ncand, top_k, present, __builtin_huge_valf(),
        -__builtin_huge_valf(), top_sm.sbuf, top_sm.sh,
        [&](int pos, int c) { out[pos] = skb[c / block] * block + c % block; }, load_kept);
    for (int i = cnt + tid; i < top_k; i += 64 * WAVES) out[i] = -1;
    if (tid == 0) sel_count[b] = cnt;
  }
}

// H5: exact top-k over the kept blocks' valid tokens by (larger s, lower t);
// candidate c = (kept slot c / block, row c % block).  Kept blocks are
// ascending, so candidate order is position order and ties go to the lower
// position.
template <int NVMAX>
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
  __shared__ __attribute__((aligned(16))) float sbuf[kHisaThreads * NVMAX];  // radix fallback only
  // the kept blocks (for the output positions) load with the scores; the
  // scores load before the kept count is known (clamped to the buffer), and
  // only the first ncand are candidates.  The token-score pass wrote -inf for
  // every slot past the sequence end and a finite score for every token of it.
  auto load_kept = [&]() {
    for (int i = tid; i < kc; i += kHisaThreads) skept[i] = kept[(size_t)b * keep_blocks + i];
  };
  auto present = [](float v) { return v != -__builtin_huge_valf(); };
  int32_t* out = sel_idx + (size_t)b * top_k;
  auto emit = [&](int pos, int c) { out[pos] = skept[c / block] * block + c % block; };
  const int cnt =
      top_strided<kHisaThreads, false, decltype(present), decltype(emit), decltype(load_kept),
                  NVMAX>(ts, keep_blocks * block, ncand, top_k, present, __builtin_huge_valf(),
                         -__builtin_huge_valf(), sbuf, sh, emit, load_kept);
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

bool hisa_fused_top_blocks(const hhr_hisa_shape& s) {
  return s.batch <= kHisaFusedMaxRows && s.max_ctx / s.block <= kBsTopMax;
}

hipError_t launch_hisa_block_scores(const hhr_hisa_shape& s, const uint8_t* q8,
                                    const float* q_scale, const float* w, const float* reps,
                                    const int32_t* seq_len, float* block_scores,
                                    uint32_t* status, hipStream_t stream, const uint8_t* k8,
                                    const float* k_scale, float* tail, int32_t keep_blocks,
                                    int32_t* kept, int32_t* kept_count, uint32_t* counters) {
  const bool shared = tail != nullptr;
  if (shared) {
    hipLaunchKernelGGL(k_hisa_pool_tail, dim3(s.batch), dim3(kD), 0, stream, k8, k_scale,
                       seq_len, tail, s.max_ctx, s.block);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int NbCap = s.max_ctx / s.block;
  // many queries: each workgroup covers 4 groups of 16 blocks per wave, so the
  // query conversion is shared; few: one group per wave for parallelism
  const int gpw = s.batch >= 64 ? 4 : 1;
  const int waves = kept != nullptr ? kBsTopWaves : kBsWaves;
  const int per_wg = 16 * waves * gpw;
  const dim3 grid((NbCap + per_wg - 1) / per_wg, s.batch);
  if (kept != nullptr)  // H3 in this launch (hisa_fused_top_blocks)
    hipLaunchKernelGGL((k_hisa_block_scores<kBsTopWaves, true>), grid, dim3(64 * kBsTopWaves), 0,
                       stream, q8,
                       q_scale, w, reps, seq_len, tail, block_scores, status, s.n_index_heads,
                       s.max_ctx, s.block, shared ? 1 : 0, gpw, keep_blocks, kept, kept_count,
                       counters);
  else
    hipLaunchKernelGGL((k_hisa_block_scores<kBsWaves, false>), grid, dim3(64 * kBsWaves), 0,
                       stream, q8,
                       q_scale, w, reps, seq_len, tail, block_scores, status, s.n_index_heads,
                       s.max_ctx, s.block, shared ? 1 : 0, gpw, 0, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_hisa_top_blocks(const hhr_hisa_shape& s, const float* block_scores,
                                  const int32_t* seq_len, int32_t keep_blocks, int32_t* kept,
                                  int32_t* kept_count, uint32_t* status, hipStream_t stream) {
  // register-resident blocks per thread: 1 up to 1024 blocks (two workgroups
  // then fit on a CU), else up to 16
  auto kern = s.max_ctx / s.block <= kHisaThreads ? k_hisa_top_blocks<1> : k_hisa_top_blocks<16>;
  hipLaunchKernelGGL(kern, dim3(s.batch), dim3(kHisaThreads), 0, stream,
                     block_scores, seq_len, keep_blocks, kept, kept_count, status, s.max_ctx,
                     s.block);
  return hipGetLastError();
}

bool hisa_fused_topk(const hhr_hisa_shape& s) { return s.batch <= kHisaFusedMaxRows; }

hipError_t launch_hisa_token_topk(const hhr_hisa_shape& s, const uint8_t* q8,
                                  const float* q_scale, const float* w, const uint8_t* k8,
                                  const float* k_scale, const int32_t* seq_len,
                                  const int32_t* kept, const int32_t* kept_count,
                                  int32_t keep_blocks, int32_t top_k, int32_t* sel_idx,
                                  int32_t* sel_count, float* token_scores, uint32_t* status,
                                  hipStream_t stream, bool shared, uint32_t* counters) {
  (void)status;
  if (counters != nullptr) {  // H5 in the token-score launch (hisa_fused_topk)
    // a workgroup's 16 waves take one tile each: enough kept blocks to fill them
    const int nslot = std::max(1, kTsTopWaves / (s.block / 16));
    const int nsplit = (keep_blocks + nslot - 1) / nslot;
    hipLaunchKernelGGL((k_hisa_token_scores<kTsTopWaves, true>), dim3(nsplit, s.batch),
                       dim3(64 * kTsTopWaves), 0, stream, q8, q_scale, w, k8, k_scale, seq_len,
                       kept, kept_count, keep_blocks, token_scores, s.n_index_heads, s.max_ctx,
                       s.block, shared ? 1 : 0, nslot, s.batch, 0, top_k, sel_idx, sel_count,
                       counters);
    return hipGetLastError();
  }
  // enough workgroups to fill the chip: a run of kept blocks per workgroup,
  // all of a row's blocks once there are many rows
  const int nsplit = std::max(1, std::min<int>(keep_blocks, (512 + s.batch - 1) / s.batch));
  const int nslot = (keep_blocks + nsplit - 1) / nsplit;
  // many rows: spread them over the 8 XCDs in contiguous runs
  const int xcd_rows = s.batch >= 64;
  const int rows = xcd_rows ? (s.batch + 7) / 8 * 8 : s.batch;
  hipLaunchKernelGGL((k_hisa_token_scores<kTsWaves, false>), dim3(nsplit, rows),
                     dim3(64 * kTsWaves), 0, stream, q8, q_scale, w, k8, k_scale, seq_len, kept,
                     kept_count, keep_blocks, token_scores, s.n_index_heads, s.max_ctx, s.block,
                     shared ? 1 : 0, nslot, s.batch, xcd_rows, 0, nullptr, nullptr, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // register-resident candidates per thread: up to 8 (two workgroups then fit
  // on a CU), else up to 16
  auto topk = keep_blocks * s.block <= 8 * kHisaThreads ? k_hisa_topk<8> : k_hisa_topk<16>;
  hipLaunchKernelGGL(topk, dim3(s.batch), dim3(kHisaThreads), 0, stream, token_scores,
                     seq_len, kept, kept_count, keep_blocks, top_k, sel_idx, sel_count,
                     s.max_ctx, s.block);
  return hipGetLastError();
}

}  // namespace hhr
