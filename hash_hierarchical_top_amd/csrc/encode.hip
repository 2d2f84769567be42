// S1 key encoder and S2 query encoder for gfx950.
//
// [HHR abstract] keys are rotated by a head-wise orthogonal R_h (GKR) and
// hashed by the signs of a head-wise projection W_h (LHP; Figure 2 caption:
// a projection followed by sign).  The encoder computes X = K R and Y = K W
// for a tile of keys as one dense contraction on MFMA, then, in the same
// kernel, packs the sign bits of Y into 128-bit codes (Table 4: 128-bit hash
// codes) and reduces X to per-page, per-dimension [min, max] metadata.

#include "hhr_device.h"
#include "hhr_internal.h"
#include "stages.h"

namespace hhr {

namespace {

constexpr int kTilePages = 4;                 // pages per tile
constexpr int kTileRows = kTilePages * kPS;   // 64 key rows per tile
constexpr int kLdsStride = kD + 8;            // bf16 elements per staged row (bank spread)

// Column split: [R | W] (W is [128][32 NW]) has 128 + 32 NW output columns,
// in tiles of 16.  A wave owns NTW consecutive tiles: the first 8 / NTW waves
// produce X (the rotated keys), the next 2 NW / NTW produce Y (the hash
// projection).  The wave's B operand (16 NTW columns x 128 rows, bf16 hi + lo)
// stays in registers for every tile of keys the workgroup processes; key
// tiles are staged through LDS.
template <int NTW>
constexpr int enc_x_waves() { return 8 / NTW; }
template <int NW, int NTW>
constexpr int enc_threads() { return 64 * (8 / NTW + 2 * NW / NTW); }

// The wave's B operand: element (k, n) of its 16 NTW columns of [R | W], k =
// 32 ks + 8 lgrp + j, split into bf16 hi + lo (hi + lo carries 16 of f32's 24
// significant bits; the products are summed in f32).
template <int NW, int NTW>
__device__ __forceinline__ void enc_load_b(const float* R, const float* W, int g, int w, int l,
                                           bf16x8 (&bhi)[NTW][4], bf16x8 (&blo)[NTW][4]) {
  const int lrow = l & 15;
  const int lgrp = l >> 4;
  const bool xw = w < enc_x_waves<NTW>();
  const int mstride = xw ? kD : 32 * NW;  // row length of R or W
  const float* M = xw ? R + (size_t)g * kD * kD : W + (size_t)g * kD * (32 * NW);
  const int col0 = 16 * NTW * (xw ? w : w - enc_x_waves<NTW>());
  // per column tile: its 32 loads first (independent, one round trip), then the split
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    float raw[4][8];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        raw[ks][i] = M[(size_t)(32 * ks + 8 * lgrp + i) * mstride + col0 + 16 * nt + lrow];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 hv, lv;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const u32x2 hl = split_bf16x2(raw[ks][2 * jj], raw[ks][2 * jj + 1]);
        hv[jj] = hl[0];
        lv[jj] = hl[1];
      }
      bhi[nt][ks] = as_bf16x8(hv);
      blo[nt][ks] = as_bf16x8(lv);
    }
  }
}

// Epilogue of one page (rows prow0 .. prow0 + 15; valid rows < e, new rows >=
// s).  X waves: acc[nt][j] is (row 4 lgrp + j, column 16 nt + lrow) of the
// wave's 16 NTW columns of X, reduced to the page's per-dimension {min, max}
// over its valid rows.  Y waves: the transposed tile (see below), reduced to
// the sign bits of the new rows, NTW / 2 code words each.
template <int NW, int NTW, bool XW>
__device__ __forceinline__ void enc_page_epilogue(const floatx4 (&acc)[NTW], int w, int l,
                                                  int bg, int page, int s, int e, int NpCap,
                                                  int Lcap, uint32_t* codes, void* meta,
                                                  int meta_bf16) {
  static_assert(NTW == 2 || NTW == 4, "column tiles per wave");
  const int lgrp = l >> 4;
  const int prow0 = page * kPS;
  if constexpr (XW) {
    // min / max over the page's valid rows: 4 rows in-lane, then across the
    // four lane groups by two lane swaps (lane l ^ 32, then l ^ 16)
    const float inf = opaque_inf();
    float mn[NTW], mx[NTW];
    if (prow0 + kPS <= e) {  // uniform: a full page
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const floatx4 v = acc[nt];
        mn[nt] = med_min(med_min(v[0], v[1], inf), med_min(v[2], v[3], inf), inf);
        mx[nt] = med_max(med_max(v[0], v[1], inf), med_max(v[2], v[3], inf), inf);
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        mn[nt] = inf;
        mx[nt] = -inf;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool ok = prow0 + 4 * lgrp + j < e;
          mn[nt] = med_min(mn[nt], ok ? acc[nt][j] : inf, inf);
          mx[nt] = med_max(mx[nt], ok ? acc[nt][j] : -inf, inf);
        }
      }
    }
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      mn[nt] = fmin_swap32(mn[nt], inf);
      mx[nt] = fmax_swap32(mx[nt], inf);
    }
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      mn[nt] = fmin_swap16(mn[nt], inf);
      mx[nt] = fmax_swap16(mx[nt], inf);
    }
    // every lane group now holds all the wave's column tiles: group q stores
    // tile q, so the wave writes its 16 NTW dimensions in one contiguous store
    float smn, smx;
    if constexpr (NTW == 4) {
      smn = lgrp == 0 ? mn[0] : lgrp == 1 ? mn[1] : lgrp == 2 ? mn[2] : mn[3];
      smx = lgrp == 0 ? mx[0] : lgrp == 1 ? mx[1] : lgrp == 2 ? mx[2] : mx[3];
    } else {
      smn = lgrp == 0 ? mn[0] : mn[1];
      smx = lgrp == 0 ? mx[0] : mx[1];
    }
    if (NTW == 4 || lgrp < NTW) {
      const size_t at = ((size_t)bg * NpCap + page) * kD + 16 * NTW * w + l;
      if (meta_bf16)  // {min down, max up} as bf16 in one word
        ((uint32_t*)meta)[at] = f32_to_bf16_down(smn) | (f32_to_bf16_up(smx) << 16);
      else
        ((float2*)meta)[at] = make_float2(smn, smx);
    }
  } else {
    // Y waves run the transposed product: acc[nt][j] = Y(row lrow of the page,
    // code bit 16 nt + 4 lgrp + j).  Each lane sets its 4 bits of each tile in
    // the row's code word, the two lane swaps OR in the other lane groups'
    // bits, and lane group 0 stores the page's 16 rows.
    uint32_t word[NTW / 2];
#pragma unroll
    for (int wi = 0; wi < NTW / 2; ++wi) {
      uint32_t v = 0u;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          v |= acc[2 * wi + h][j] >= 0.0f ? 1u << (16 * h + 4 * lgrp + j) : 0u;
      word[wi] = or_swap16(or_swap32(v));
    }
    const int row = prow0 + (l & 15);
    if (lgrp == 0 && row >= s && row < e) {
      uint32_t* dst = codes + ((size_t)bg * Lcap + row) * NW + (NTW / 2) * (w - enc_x_waves<NTW>());
      if constexpr (NTW == 4)
        *(u32x2*)dst = u32x2{word[0], word[1]};
      else
        *dst = word[0];
    }
  }
}

// The rows to encode for (b, g): [s, e), from the n_new / last-row modes.
// Returns false (and flags bad input) when there is nothing to do.
__device__ __forceinline__ bool enc_range(const int32_t* start, const int32_t* n_new, int b, int g,
                                          int Lcap, uint32_t* status, int& s, int& e) {
  // n_new NULL: start holds seq_len and the one row seq_len - 1 is new
  s = n_new ? start[b] : start[b] - 1;
  const int n = n_new ? n_new[b] : (start[b] > 0 ? 1 : 0);
  if (n_new == nullptr && start[b] == 0) return false;
  if (s < 0 || n < 0 || (long long)s + n > Lcap) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && g == 0 && status)
      atomicOr(status, HHR_DEV_BAD_SEQ_LEN);
    return false;
  }
  e = s + n;
  return n > 0;
}

// f32 keys: each tile is loaded into registers, split into bf16 hi + lo and
// stored to LDS (the A operand takes three products: hi*hi, hi*lo, lo*hi).
template <int NW>
__global__ __launch_bounds__((enc_threads<NW, 4>())) void k_append_encode_f32(
    const float* __restrict__ kcache, const int32_t* __restrict__ start,
    const int32_t* __restrict__ n_new, const float* __restrict__ R, const float* __restrict__ W,
    uint32_t* __restrict__ codes, void* __restrict__ meta, int meta_bf16,
    uint32_t* __restrict__ status, int Hkv, int Lcap, int tiles_per_wg) {
  __shared__ __attribute__((aligned(16))) uint16_t a_hi[kTileRows * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t a_lo[kTileRows * kLdsStride];

  const int bg = blockIdx.y;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  int s, e;
  if (!enc_range(start, n_new, b, g, Lcap, status, s, e)) return;
  const int first_page = s / kPS;
  const int last_page = (e - 1) / kPS;
  const int ntiles = (last_page - first_page + kTilePages) / kTilePages;
  const int t0 = blockIdx.x * tiles_per_wg;
  if (t0 >= ntiles) return;
  const int t1 = min(ntiles, t0 + tiles_per_wg);
  const int NpCap = Lcap / kPS;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int lrow = l & 15;
  const int lgrp = l >> 4;
  constexpr int kNT = enc_threads<NW, 4>();
  const bool xw = w < enc_x_waves<4>();  // wave-uniform
  bf16x8 bhi[4][4], blo[4][4];
  enc_load_b<NW, 4>(R, W, g, w, l, bhi, blo);

  for (int t = t0; t < t1; ++t) {
    const int page0 = first_page + t * kTilePages;
    const int row0 = page0 * kPS;
    __syncthreads();  // previous tile's LDS reads are done
    const float* Kf = kcache + (size_t)bg * Lcap * kD;
#pragma unroll
    for (int i = 0; i < (kTileRows * 32 + kNT - 1) / kNT; ++i) {
      const int c = tid + kNT * i;  // 16-byte chunk of 4 floats: 64 rows x 32 chunks
      if (c < kTileRows * 32) {
        const int r = c >> 5;
        const int cc = c & 31;
        const int grow = row0 + r;
        floatx4 v = {0.f, 0.f, 0.f, 0.f};
        if (grow < e) v = *(const floatx4*)(Kf + (size_t)grow * kD + cc * 4);
        const u32x2 a = split_bf16x2(v[0], v[1]), c = split_bf16x2(v[2], v[3]);
        const u32x2 hv = {a[0], c[0]}, lv = {a[1], c[1]};
        *(u32x2*)(a_hi + r * kLdsStride + cc * 4) = hv;
        *(u32x2*)(a_lo + r * kLdsStride + cc * 4) = lv;
      }
    }
    __syncthreads();

#pragma unroll
    for (int mt = 0; mt < kTilePages; ++mt) {
      if (row0 + 16 * mt >= e) break;  // uniform
      floatx4 acc[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int off = (16 * mt + lrow) * kLdsStride + 32 * ks + 8 * lgrp;
        const bf16x8 a = as_bf16x8(*(const u32x4*)(a_hi + off));
        const bf16x8 alo = as_bf16x8(*(const u32x4*)(a_lo + off));
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          if (xw) {  // X tile: rows = keys
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bhi[nt][ks], acc[nt], 0, 0, 0);
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, blo[nt][ks], acc[nt], 0, 0, 0);
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bhi[nt][ks], acc[nt], 0, 0, 0);
          } else {  // Y tile transposed: rows = code bits
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bhi[nt][ks], a, acc[nt], 0, 0, 0);
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(blo[nt][ks], a, acc[nt], 0, 0, 0);
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bhi[nt][ks], alo, acc[nt], 0, 0, 0);
          }
        }
      }
      if (xw)
        enc_page_epilogue<NW, 4, true>(acc, w, l, bg, page0 + mt, s, e, NpCap, Lcap, codes,
                                       meta, meta_bf16);
      else
        enc_page_epilogue<NW, 4, false>(acc, w, l, bg, page0 + mt, s, e, NpCap, Lcap, codes,
                                        meta, meta_bf16);
    }
  }
}

// bf16 keys (exact in bf16: the A operand is the key itself).  Key tiles move
// HBM -> LDS by the waves' direct LDS loads (global_load_lds_dwordx4), in a
// ring of three tiles: while the MFMAs and the epilogue of tile t run, tiles
// t + 1 and t + 2 are in flight, with no registers held for them.  A tile is
// 64 rows x 256 bytes with no padding; the 16-byte chunk (r, c) of the tile
// sits at LDS chunk (r, c ^ (r & 15)), so the 16 rows an A-fragment read
// touches fall in 16 different chunk columns.  Each wave owns two column tiles
// (32 columns), so its B operand takes 64 registers and four waves share a
// SIMD: one wave's epilogue overlaps the others' MFMAs.
//
// Waits: vector-memory loads complete in issue order, so once at most the
// newest tile's loads (n per wave) are outstanding, every older tile of this
// wave has landed; the barrier that follows makes all waves' loads visible.
// Stores in between do not break this: they only add to the count.
constexpr int kEncRing = 3;
constexpr int kEncTileBytes = kTileRows * kD * 2;     // 16 KiB
constexpr int kEncWaveLoads = kEncTileBytes / 1024;  // 16 wave loads of 1 KiB per tile
constexpr int kEncNTW = 2;                           // column tiles per wave (bf16 keys)

typedef __attribute__((address_space(3))) void lds_void_t;

template <int N>
__device__ __forceinline__ void wait_vm_le() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);  // vmcnt(N), expcnt and lgkmcnt not waited
}

template <int NW>
__global__ __launch_bounds__((enc_threads<NW, kEncNTW>()), NW == 8 ? 1 : 2) void
k_append_encode_bf16(const uint16_t* __restrict__ kcache, const int32_t* __restrict__ start,
                     const int32_t* __restrict__ n_new, const float* __restrict__ R,
                     const float* __restrict__ W, uint32_t* __restrict__ codes,
                     void* __restrict__ meta, int meta_bf16, uint32_t* __restrict__ status,
                     int Hkv, int Lcap, int tiles_per_wg) {
  constexpr int NTW = kEncNTW;
  __shared__ __attribute__((aligned(1024))) uint16_t ring[kEncRing][kTileRows * kD];

  const int bg = blockIdx.y;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  int s, e;
  if (!enc_range(start, n_new, b, g, Lcap, status, s, e)) return;
  const int first_page = s / kPS;
  const int last_page = (e - 1) / kPS;
  const int ntiles = (last_page - first_page + kTilePages) / kTilePages;
  const int t0 = blockIdx.x * tiles_per_wg;
  if (t0 >= ntiles) return;
  const int t1 = min(ntiles, t0 + tiles_per_wg);
  const int NpCap = Lcap / kPS;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int lrow = l & 15;
  const int lgrp = l >> 4;
  constexpr int kWaves = enc_threads<NW, NTW>() / 64;
  // every wave issues at least this many of a tile's 16 wave loads
  constexpr int kMinLoads = kEncWaveLoads / kWaves;
  static_assert(kMinLoads >= 1, "every wave loads part of each tile");
  const uint16_t* Kb = kcache + (size_t)bg * Lcap * kD;

  // wave load i of tile t fills LDS rows [4i, 4i + 4): lane l writes chunk
  // (4i + l / 16, l % 16), which holds key chunk (l % 16) ^ (row & 15); rows
  // past the cache end read its last row (their results are never used)
  auto issue = [&](int t) {
    const int row0 = (first_page + t * kTilePages) * kPS;
    uint16_t* dst = ring[(t - t0) % kEncRing];
    for (int i = w; i < kEncWaveLoads; i += kWaves) {
      const int r = 4 * i + (l >> 4);
      const int c = (l & 15) ^ (r & 15);
      const int grow = min(row0 + r, Lcap - 1);
      __builtin_amdgcn_global_load_lds((const void*)(Kb + (size_t)grow * kD + c * 8),
                                       (lds_void_t*)(dst + 512 * i), 16, 0, 0);
    }
  };
  issue(t0);
  if (t0 + 1 < t1) issue(t0 + 1);

  bf16x8 bhi[NTW][4], blo[NTW][4];
  enc_load_b<NW, NTW>(R, W, g, w, l, bhi, blo);

  // X waves and Y waves run the same loop (same barriers) with their own
  // epilogue, so the loop body has no role branch
  auto run = [&](auto xw) {
    constexpr bool XW = decltype(xw)::value;
    for (int t = t0; t < t1; ++t) {
      if (t + 1 < t1)
        wait_vm_le<kMinLoads>();
      else
        wait_vm_le<0>();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_barrier();  // tile t is in LDS; tile t - 1's slot is free
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (t + 2 < t1) issue(t + 2);
      const uint16_t* A = ring[(t - t0) % kEncRing];
      const int page0 = first_page + t * kTilePages;
      const int row0 = page0 * kPS;
#pragma unroll
      for (int mt = 0; mt < kTilePages; ++mt) {
        if (row0 + 16 * mt >= e) break;  // uniform
        floatx4 acc[NTW];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int kc = 4 * ks + lgrp;  // 16-byte chunk of the row
          const bf16x8 a =
              as_bf16x8(*(const u32x4*)(A + (16 * mt + lrow) * kD + 8 * (kc ^ lrow)));
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) {
            if constexpr (XW) {  // X tile: rows = keys
              acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bhi[nt][ks], acc[nt], 0, 0, 0);
              acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, blo[nt][ks], acc[nt], 0, 0, 0);
            } else {  // Y tile transposed: rows = code bits
              acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bhi[nt][ks], a, acc[nt], 0, 0, 0);
              acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(blo[nt][ks], a, acc[nt], 0, 0, 0);
            }
          }
        }
        enc_page_epilogue<NW, NTW, XW>(acc, w, l, bg, page0 + mt, s, e, NpCap, Lcap, codes,
                                       meta, meta_bf16);
      }
    }
  };
  if (w < enc_x_waves<NTW>())
    run(std::true_type{});
  else
    run(std::false_type{});
}

// S2: one workgroup (kQeThreads) per (b, KV head) encodes the G queries of the group.
template <int NW>
__global__ __launch_bounds__(kQeThreads) void k_encode_queries(
    const float* __restrict__ q, const float* __restrict__ R, const float* __restrict__ W,
    float* __restrict__ q_rot, uint32_t* __restrict__ q_codes, int Hq, int Hkv) {
  __shared__ QencSmem sm;
  const int bg = blockIdx.x;
  qenc_group<false, NW>(bg / Hkv, bg % Hkv, Hq, Hkv, q, R, W, q_rot, q_codes, sm);
}

}  // namespace

hipError_t launch_append_keys(const hhr_shape& s, const void* k_cache, const int32_t* start,
                              const int32_t* n_new, int32_t max_new, const float* R,
                              const float* W, uint32_t* codes, void* meta, uint32_t* status,
                              hipStream_t stream) {
  if (max_new <= 0) return hipSuccess;
  const int touched_pages = (max_new + kPS - 1) / kPS + 1;
  const int max_tiles = (touched_pages + kTilePages - 1) / kTilePages;
  const int bgs = s.batch * s.n_kv_heads;
  const bool kf32 = s.kv_dtype == HHR_F32;
  // bf16: two workgroups per CU (one at 256-bit codes), each over a long run
  // of tiles (the B operand loads once per workgroup).  f32: more, shorter
  // workgroups.
  const long long target_wgs = kf32 ? 2048 : (s.code_bits == 256 ? 256 : 2 * 256);
  int tpw = (int)(((long long)max_tiles * bgs + target_wgs - 1) / target_wgs);
  if (tpw < 1) tpw = 1;
  dim3 grid((max_tiles + tpw - 1) / tpw, bgs);
  const int mbf = s.meta_dtype == HHR_BF16;
#define HHR_ENC(NW)                                                                             \
  if (kf32)                                                                                     \
    hipLaunchKernelGGL((k_append_encode_f32<NW>), grid, dim3(enc_threads<NW, 4>()), 0, stream,  \
                       (const float*)k_cache, start, n_new, R, W, codes, meta, mbf, status,     \
                       s.n_kv_heads, s.max_ctx, tpw);                                           \
  else                                                                                          \
    hipLaunchKernelGGL((k_append_encode_bf16<NW>), grid, dim3(enc_threads<NW, kEncNTW>()), 0,   \
                       stream,                                                                  \
                       (const uint16_t*)k_cache, start, n_new, R, W, codes, meta, mbf, status,  \
                       s.n_kv_heads, s.max_ctx, tpw)
  switch (s.code_bits) {
    case 64: HHR_ENC(2); break;
    case 256: HHR_ENC(8); break;
    default: HHR_ENC(4); break;
  }
#undef HHR_ENC
  return hipGetLastError();
}

hipError_t launch_append_last_row(const hhr_shape& s, const void* k_cache,
                                  const int32_t* seq_len, const float* R, const float* W,
                                  uint32_t* codes, void* meta, uint32_t* status,
                                  hipStream_t stream) {
  return launch_append_keys(s, k_cache, seq_len, nullptr, 1, R, W, codes, meta, status, stream);
}

hipError_t launch_encode_queries(const hhr_shape& s, const float* q, const float* R,
                                 const float* W, float* q_rot, uint32_t* q_codes,
                                 hipStream_t stream) {
  const dim3 grid(s.batch * s.n_kv_heads);
  if (s.code_bits == 64)
    hipLaunchKernelGGL(k_encode_queries<2>, grid, dim3(kQeThreads), 0, stream, q, R, W, q_rot,
                       q_codes, s.n_q_heads, s.n_kv_heads);
  else if (s.code_bits == 256)
    hipLaunchKernelGGL(k_encode_queries<8>, grid, dim3(kQeThreads), 0, stream, q, R, W, q_rot,
                       q_codes, s.n_q_heads, s.n_kv_heads);
  else
    hipLaunchKernelGGL(k_encode_queries<4>, grid, dim3(kQeThreads), 0, stream, q, R, W, q_rot,
                       q_codes, s.n_q_heads, s.n_kv_heads);
  return hipGetLastError();
}

}  // namespace hhr
