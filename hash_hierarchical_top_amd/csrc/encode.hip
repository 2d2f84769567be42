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

// One workgroup = 2 + NW/2 waves; wave w owns output columns [64w, 64w+64) of
// [R | W] (W is [128][32 NW]): waves 0-1 produce X (rotated keys), waves 2..
// produce Y (hash projection), two code words each.  The B operand (64
// columns x 128 rows, bf16 hi + lo) stays in registers for every tile the
// workgroup processes; key tiles are staged through LDS.
template <int NW>
constexpr int enc_threads() { return 64 * (2 + NW / 2); }

template <bool KF32, int NW>
__global__ __launch_bounds__(enc_threads<NW>()) void k_append_encode(
    const void* __restrict__ kcache, const int32_t* __restrict__ start,
    const int32_t* __restrict__ n_new, const float* __restrict__ R, const float* __restrict__ W,
    uint32_t* __restrict__ codes, void* __restrict__ meta, int meta_bf16,
    uint32_t* __restrict__ status, int Hkv, int Lcap, int tiles_per_wg) {
  __shared__ __attribute__((aligned(16))) uint16_t a_hi[kTileRows * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t a_lo[KF32 ? kTileRows * kLdsStride : 8];

  const int bg = blockIdx.y;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  // n_new NULL: start holds seq_len and the one row seq_len - 1 is new
  const int s = n_new ? start[b] : start[b] - 1;
  const int n = n_new ? n_new[b] : (start[b] > 0 ? 1 : 0);
  if (n_new == nullptr && start[b] == 0) return;
  if (s < 0 || n < 0 || (long long)s + n > Lcap) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && g == 0 && status)
      atomicOr(status, HHR_DEV_BAD_SEQ_LEN);
    return;
  }
  if (n == 0) return;
  const int e = s + n;
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
  const int lrow = l & 15;     // MFMA row/col within a 16x16 tile
  const int lgrp = l >> 4;     // lane group: K slots [8*lgrp, 8*lgrp+8)

  // B operand: element (k, n) of the wave's 64 columns, k = 32*ks + 8*lgrp + j.
  constexpr int kNT = enc_threads<NW>();
  const int mstride = w < 2 ? kD : 32 * NW;  // row length of R or W
  const float* M = w < 2 ? R + (size_t)g * kD * kD : W + (size_t)g * kD * (32 * NW);
  const int col0 = w < 2 ? 64 * w : 64 * (w - 2);
  bf16x8 bhi[4][4], blo[4][4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 hv, lv;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int k = 32 * ks + 8 * lgrp + 2 * jj;
        const int col = col0 + 16 * nt + lrow;
        uint32_t h0, l0, h1, l1;
        split_bf16(M[(size_t)k * mstride + col], h0, l0);
        split_bf16(M[(size_t)(k + 1) * mstride + col], h1, l1);
        hv[jj] = h0 | (h1 << 16);
        lv[jj] = l0 | (l1 << 16);
      }
      bhi[nt][ks] = as_bf16x8(hv);
      blo[nt][ks] = as_bf16x8(lv);
    }
  }

  for (int t = t0; t < t1; ++t) {
    const int page0 = first_page + t * kTilePages;
    const int row0 = page0 * kPS;
    __syncthreads();  // previous tile's LDS reads are done
    if constexpr (!KF32) {
      const uint16_t* Kb = (const uint16_t*)kcache + (size_t)bg * Lcap * kD;
#pragma unroll
      for (int i = 0; i < (kTileRows * 16 + kNT - 1) / kNT; ++i) {
        const int c = tid + kNT * i;  // 16-byte chunk: 64 rows x 16 chunks
        if (c < kTileRows * 16) {
          const int r = c >> 4;
          const int cc = c & 15;
          const int grow = row0 + r;
          u32x4 v = {0u, 0u, 0u, 0u};
          if (grow < e) v = *(const u32x4*)(Kb + (size_t)grow * kD + cc * 8);
          *(u32x4*)(a_hi + r * kLdsStride + cc * 8) = v;
        }
      }
    } else {
      const float* Kf = (const float*)kcache + (size_t)bg * Lcap * kD;
#pragma unroll
      for (int i = 0; i < (kTileRows * 32 + kNT - 1) / kNT; ++i) {
        const int c = tid + kNT * i;  // 16-byte chunk of 4 floats: 64 rows x 32 chunks
        if (c < kTileRows * 32) {
          const int r = c >> 5;
          const int cc = c & 31;
          const int grow = row0 + r;
          floatx4 v = {0.f, 0.f, 0.f, 0.f};
          if (grow < e) v = *(const floatx4*)(Kf + (size_t)grow * kD + cc * 4);
          uint32_t h[4], lo[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) split_bf16(v[j], h[j], lo[j]);
          u32x2 hv = {h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
          u32x2 lv = {lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
          *(u32x2*)(a_hi + r * kLdsStride + cc * 4) = hv;
          *(u32x2*)(a_lo + r * kLdsStride + cc * 4) = lv;
        }
      }
    }
    __syncthreads();

    floatx4 acc[kTilePages][4];
#pragma unroll
    for (int mt = 0; mt < kTilePages; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int mt = 0; mt < kTilePages; ++mt) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int off = (16 * mt + lrow) * kLdsStride + 32 * ks + 8 * lgrp;
        const bf16x8 a = as_bf16x8(*(const u32x4*)(a_hi + off));
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bhi[nt][ks], acc[mt][nt], 0, 0, 0);
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, blo[nt][ks], acc[mt][nt], 0, 0, 0);
        }
        if constexpr (KF32) {
          const bf16x8 alo = as_bf16x8(*(const u32x4*)(a_lo + off));
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bhi[nt][ks], acc[mt][nt], 0, 0, 0);
        }
      }
    }

    // Epilogue.  acc[mt][nt][j] is (row 4*lgrp + j of page page0+mt,
    // column col0 + 16*nt + lrow) of this wave's half of [X | Y].
#pragma unroll
    for (int mt = 0; mt < kTilePages; ++mt) {
      const int page = page0 + mt;
      const int prow0 = page * kPS;
      if (prow0 >= e) break;  // uniform
      if (w < 2) {
        // page min/max of X over the valid rows (rows < e)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (prow0 + 4 * lgrp + j < e) {
              mn = fminf(mn, acc[mt][nt][j]);
              mx = fmaxf(mx, acc[mt][nt][j]);
            }
          }
          mn = fminf(mn, __shfl_xor(mn, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mn = fminf(mn, __shfl_xor(mn, 32));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          if (lgrp == 0) {
            const size_t at = ((size_t)bg * NpCap + page) * kD + col0 + 16 * nt + lrow;
            if (meta_bf16)  // {min down, max up} as bf16 in one word
              ((uint32_t*)meta)[at] = f32_to_bf16_down(mn) | (f32_to_bf16_up(mx) << 16);
            else
              ((float2*)meta)[at] = make_float2(mn, mx);
          }
        }
      } else {
        // sign bits of Y: ballot[nt][j] bit (16*grp + c) = [Y(row 4*grp + j, col 16*nt + c) >= 0]
        uint64_t bal[4][4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int j = 0; j < 4; ++j) bal[nt][j] = __ballot(acc[mt][nt][j] >= 0.0f);
        if (l < 16) {
          const int r = l;            // row within the page
          const int j = r & 3;
          const int sh = 16 * (r >> 2);
          uint32_t half[4];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            const uint64_t v = j == 0 ? bal[nt][0] : j == 1 ? bal[nt][1] : j == 2 ? bal[nt][2] : bal[nt][3];
            half[nt] = (uint32_t)(v >> sh) & 0xFFFFu;
          }
          const int row = prow0 + r;
          if (row >= s && row < e) {
            u32x2 wv = {half[0] | (half[1] << 16), half[2] | (half[3] << 16)};
            *(u32x2*)(codes + ((size_t)bg * Lcap + row) * NW + 2 * (w - 2)) = wv;
          }
        }
      }
    }
  }
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
  // Enough workgroups to fill 256 CUs several times over, few enough that the
  // per-workgroup register load of [R | W] stays small next to the key traffic.
  const long long target_wgs = 2048;
  int tpw = (int)(((long long)max_tiles * bgs + target_wgs - 1) / target_wgs);
  if (tpw < 1) tpw = 1;
  dim3 grid((max_tiles + tpw - 1) / tpw, bgs);
  const int mbf = s.meta_dtype == HHR_BF16;
#define HHR_ENC(KF32, NW)                                                                      \
  hipLaunchKernelGGL((k_append_encode<KF32, NW>), grid, dim3(enc_threads<NW>()), 0, stream,    \
                     k_cache, start, n_new, R, W, codes, meta, mbf, status, s.n_kv_heads,       \
                     s.max_ctx, tpw)
  const bool kf32 = s.kv_dtype == HHR_F32;
  switch (s.code_bits) {
    case 64: if (kf32) HHR_ENC(true, 2); else HHR_ENC(false, 2); break;
    case 256: if (kf32) HHR_ENC(true, 8); else HHR_ENC(false, 8); break;
    default: if (kf32) HHR_ENC(true, 4); else HHR_ENC(false, 4); break;
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
