// Device functions of the decode steps S2..S7, shared by the kernels behind
// the entry points, so every composition computes bit-identical results.
// Internal header.
//
// COH selects agent-scope (sc1) accesses, for kernels in which one workgroup
// consumes data that another workgroup of the same launch produced (see Mem<>
// in hhr_device.h); COH = false is the plain path between launches.
#pragma once

#include <type_traits>

#include "hhr_device.h"
#include "hhr_internal.h"
#include "topk_device.h"

namespace hhr {

// ============================================================== S2: query
// Columns 0..127 of [R | W] give q' = q R, columns 128 .. 128 + 32 NW - 1
// give the sign bits of q W (W is [128][32 NW]).  Every output (head h,
// column c) is computed the same way: 8 partial sums over the input dims
// 16 k .. 16 k + 15 (sequential FMAs), then the partials added in LDS in
// order k = 0..7.  NT threads share the (column, k) work items, CPT adjacent
// columns each (the fewest of 1, 2, 4 that cover the columns; threads past
// them idle), so a thread holds 16 CPT matrix values in registers and the
// result does not depend on NT or on the column range [COL0, COL0 + NCOL)
// (0 and 128 + 32 NW: rotation and codes; 0 and 128: rotation only; 128 and
// 32 NW: codes only).
// rot(h, col, v) receives q'; code(h, word, bits) receives 32 code bits.
// With extra_row (a KF32/bf16 key row of length 128, or NULL) it is encoded
// the same way as row h = G after the G queries.  Every thread of the
// workgroup must call (barriers).
constexpr int kQeThreads = 1024;
constexpr int kQeChunk = 4;  // rows (query heads, then the extra key) per reduction round

struct QencSmem {
  float sq[kMaxG + 1][kD];
  float red[8][kQeChunk][kD + 32 * kMaxNW];
};

template <int NCOL, int NT>
constexpr int qenc_cpt() {
  return 8 * NCOL <= NT ? 1 : 8 * NCOL <= 2 * NT ? 2 : 4;
}

template <int NCOL, int NT, typename Rot, typename Code, int NW = kNW, int COL0 = 0>
__device__ __forceinline__ void qenc_core(int b, int g, int Hq, int Hkv, const float* __restrict__ q,
                          const float* __restrict__ R, const float* __restrict__ W,
                          QencSmem& sm, Rot rot, Code code, const void* extra_row = nullptr,
                          bool extra_f32 = false) {
  static_assert((COL0 == 0 && (NCOL == kD || NCOL == kD + 32 * NW)) ||
                    (COL0 == kD && NCOL == 32 * NW),
                "rotation, rotation and codes, or codes");
  static_assert(NCOL % 64 == 0, "a wave's outputs stay in one row");
  constexpr int CPT = qenc_cpt<NCOL, NT>();  // columns per thread
  static_assert(8 * NCOL <= CPT * NT, "too many columns for the workgroup");
  constexpr int kGroupsC = NCOL / CPT;
  constexpr int kCB = 32 * NW;  // W's row length
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const size_t qbase = ((size_t)b * Hq + (size_t)g * G) * kD;
  const bool active = tid < 8 * kGroupsC;  // threads past the work items only reduce
  const int cg = active ? tid % kGroupsC : 0;
  const int dg = active ? tid / kGroupsC : 0;  // 0..7
  const int c0 = COL0 + CPT * cg;              // first column in [COL0, COL0 + NCOL)
  const float* M = c0 < kD ? R + (size_t)g * kD * kD + c0 : W + (size_t)g * kD * kCB + (c0 - kD);
  const int mstride = c0 < kD ? kD : kCB;
  float m[16][CPT];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float* row = M + (size_t)(16 * dg + j) * mstride;
    if constexpr (CPT == 4) {
      const floatx4 v = *(const floatx4*)row;
#pragma unroll
      for (int k = 0; k < 4; ++k) m[j][k] = v[k];
    } else if constexpr (CPT == 2) {
      const float2 v = *(const float2*)row;
      m[j][0] = v.x;
      m[j][1] = v.y;
    } else {
      m[j][0] = *row;
    }
  }
  for (int i = tid; i < G * kD; i += NT) sm.sq[i / kD][i % kD] = q[qbase + i];
  const int rows = G + (extra_row != nullptr ? 1 : 0);  // block-uniform
  if (extra_row != nullptr && tid < kD)
    sm.sq[G][tid] = extra_f32 ? ((const float*)extra_row)[tid]
                              : bf16_to_f32(((const uint16_t*)extra_row)[tid]);
  __syncthreads();
  constexpr int kOut = kQeChunk * NCOL;  // outputs per round
  for (int hc = 0; hc < rows; hc += kQeChunk) {
#pragma unroll
    for (int hh = 0; hh < kQeChunk; ++hh) {
      float acc[CPT];
#pragma unroll
      for (int k = 0; k < CPT; ++k) acc[k] = 0.f;
      if (hc + hh < rows) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float x = sm.sq[hc + hh][16 * dg + j];
#pragma unroll
          for (int k = 0; k < CPT; ++k) acc[k] = fmaf(x, m[j][k], acc[k]);
        }
      }
      if (active) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) sm.red[dg][hh][c0 + k] = acc[k];
      }
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < (kOut + NT - 1) / NT; ++pass) {
      const int o = tid + NT * pass;  // (row hh, column col) of this round
      if (o >= kOut) break;           // wave-uniform: kOut is a multiple of 64
      const int hh = o / NCOL;
      const int col = COL0 + o % NCOL;
      float v = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) v += sm.red[k][hh][col];
      const int h = hc + hh;
      if (col < kD) {
        if (h < rows) rot(h, col, v);
      } else {
        const uint64_t bits = __ballot(v >= 0.0f);
        if ((tid & 63) == 0 && h < rows) {
          const int word = (col - kD) >> 5;  // col is the wave's first column here
          code(h, word, (uint32_t)bits);
          code(h, word + 1, (uint32_t)(bits >> 32));
        }
      }
    }
    __syncthreads();
  }
}

// q' and the codes (NW words each) of one (b, g) to global memory.
template <bool COH, int NW = kNW>
__device__ void qenc_group(int b, int g, int Hq, int Hkv, const float* __restrict__ q,
                           const float* __restrict__ R, const float* __restrict__ W,
                           float* q_rot, uint32_t* q_codes, QencSmem& sm) {
  const int G = Hq / Hkv;
  const size_t qbase = ((size_t)b * Hq + (size_t)g * G) * kD;
  auto rot = [&](int h, int col, float v) { Mem<COH>::st(q_rot + qbase + (size_t)h * kD + col, v); };
  auto code = [&](int h, int word, uint32_t bits) {
    Mem<COH>::st(q_codes + ((size_t)b * Hq + (size_t)g * G + h) * NW + word, bits);
  };
  qenc_core<kD + 32 * NW, kQeThreads, decltype(rot), decltype(code), NW>(b, g, Hq, Hkv, q, R, W,
                                                                         sm, rot, code);
}

// ============================================================== S3: bound
// s(p) = sum_h sum_d max(q'_hd mn_pd, q'_hd mx_pd).  Because mn <= mx,
// max(q mn, q mx) = max(q,0) mx + min(q,0) mn, so per dimension the group
// reduces to A_d = sum_h max(q'_hd, 0) and B_d = sum_h min(q'_hd, 0), and
// s(p) = sum_d (A_d mx_pd + B_d mn_pd).
//
// One wave scores pages pb .. pb+15 (those < Np).  Lane (row r = l/16,
// sub = l%16) handles pages pb + 4j + r (j = 0..3) and, in each, the 16-byte
// pieces k at byte 256k + 16 sub of the page's metadata, so every load
// instruction reads four whole 256-byte runs.  f32 metadata (1 KiB a page):
// k = 0..3, each piece {mn, mx} of dims 2(sub + 16k) and +1.  bf16 metadata
// (512 B a page): k = 0..1, each piece one {mn | mx << 16} word for dims
// 4(sub + 16k) + 0..3.  Either way a lane owns 8 dims (slots 0..7, dim_of).
// All loads are issued first (addresses clamped, not branched on); a 4-value
// reduce-scatter over the 16 lanes of a row then leaves page pb + 4j + r in
// lanes with j = 2 b3 + b2.  The whole wave must be active (cross-lane DPP
// exchanges).
constexpr int kScorePagesPerWave = 16;

// Dimension of this lane's slot (0..7) for the metadata format MBF.
template <bool MBF>
__device__ __forceinline__ int score_dim(int sub, int slot) {
  return MBF ? 4 * sub + 64 * (slot >> 2) + (slot & 3) : 2 * sub + 32 * (slot >> 1) + (slot & 1);
}

// Metadata of NB consecutive 16-page batches pb, pb + 16, ... of one (b, g),
// loaded by one wave (lane layout above; bf16 words are kept as raw bits in
// pieces 0..1).  Pages past Np are clamped to the last page; their results
// are never stored.
template <int NB>
struct PageLoads {
  floatx4 m[NB][4][4];
};

template <bool MBF, int NB>
__device__ __forceinline__ void score_load(int bg, int NpCap, int Np, int pb,
                                           const void* __restrict__ meta, PageLoads<NB>& pl) {
  constexpr int kPageFloats = MBF ? kD : 2 * kD;  // 4-byte words per page
  constexpr int kPieces = MBF ? 2 : 4;
  const int l = threadIdx.x & 63;
  const int r = l >> 4;
  const int sub = l & 15;
  const float* mbase = (const float*)meta + (size_t)bg * NpCap * kPageFloats + 4 * sub;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = min(pb + kScorePagesPerWave * nb + 4 * j + r, Np - 1);
#pragma unroll
      for (int k = 0; k < kPieces; ++k)
        pl.m[nb][j][k] = __builtin_nontemporal_load(
            (const floatx4*)(mbase + (size_t)p * kPageFloats + 64 * k));
    }
}

// A/B of this lane's 8 dims (slot order of score_dim), summed over the G heads
// in order: rot_of(h, d) returns q'_hd.
template <bool MBF, typename RotOf>
__device__ __forceinline__ void score_ab(int G, RotOf rot_of, float A[8], float B[8]) {
  const int sub = threadIdx.x & 15;
#pragma unroll
  for (int i = 0; i < 8; ++i) A[i] = B[i] = 0.f;
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = rot_of(h, score_dim<MBF>(sub, i));
      A[i] += fmaxf(v, 0.f);
      B[i] += fminf(v, 0.f);
    }
  }
}

// Bounds of the loaded pages; each page's bound is stored by one lane, and
// emit(p, v) sees it too.
template <bool MBF, bool COH, int NB, typename Emit>
__device__ __forceinline__ void score_finish(int bg, int NpCap, int Np, int pb,
                                             const PageLoads<NB>& pl, const float A[8],
                                             const float B[8], float* scores, Emit emit) {
  const int l = threadIdx.x & 63;
  const int r = l >> 4;
  const bool b3 = l & 8, b2 = l & 4;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x = 0.f;
      if constexpr (MBF) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t w = __float_as_uint(pl.m[nb][j][k][i]);
            x += A[4 * k + i] * __uint_as_float(w & 0xFFFF0000u) +
                 B[4 * k + i] * __uint_as_float(w << 16);
          }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)  // m = {mn[d0], mx[d0], mn[d1], mx[d1]}
          x += A[2 * k] * pl.m[nb][j][k][1] + B[2 * k] * pl.m[nb][j][k][0] +
               A[2 * k + 1] * pl.m[nb][j][k][3] + B[2 * k + 1] * pl.m[nb][j][k][2];
      }
      v[j] = x;
    }
    // partner lanes: 15 - sub (other 8-lane half), then 7 - (sub % 8) (other
    // quad of the half), then the quad's own butterfly
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float send = b3 ? v[i] : v[i + 2];
      const float keep = b3 ? v[i + 2] : v[i];
      v[i] = keep + dpp_f<dpp::kRowMirror>(send);
    }
    {
      const float send = b2 ? v[0] : v[1];
      const float keep = b2 ? v[1] : v[0];
      v[0] = keep + dpp_f<dpp::kRowHalfMirror>(send);
    }
    v[0] += dpp_f<dpp::kQuadXor2>(v[0]);
    v[0] += dpp_f<dpp::kQuadXor1>(v[0]);
    const int p = pb + kScorePagesPerWave * nb + 4 * ((b3 ? 2 : 0) + (b2 ? 1 : 0)) + r;
    if ((l & 3) == 0 && p < Np) {
      Mem<COH>::st(scores + (size_t)bg * NpCap + p, v[0]);
      emit(p, v[0]);
    }
  }
}

// One wave: load, read q' from q_rot, finish.
template <bool MBF, bool COH, int NB = 1>
__device__ void score_batch(int b, int g, int Hq, int Hkv, int NpCap, int Np, int pb,
                            const float* q_rot, const void* __restrict__ meta, float* scores) {
  const int G = Hq / Hkv;
  const int bg = b * Hkv + g;
  PageLoads<NB> pl;
  score_load<MBF, NB>(bg, NpCap, Np, pb, meta, pl);
  float A[8], B[8];
  const float* qr = q_rot + ((size_t)b * Hq + (size_t)g * G) * kD;
  score_ab<MBF>(G, [&](int h, int d) { return Mem<COH>::ld(qr + (size_t)h * kD + d); }, A, B);
  score_finish<MBF, COH, NB>(bg, NpCap, Np, pb, pl, A, B, scores, [](int, float) {});
}

// ============================================================== S4: prune
// Exact top-P of Np page scores in one workgroup of NT threads
// (top_largest_strided): thread t loads pages j NT + t, so the loads coalesce
// and the scores stay in registers.  The range is the given pieces (lo, hi)
// together with this thread's own scores (pass +inf, -inf to take it from the
// scores alone).  mid() runs once, after the loads are issued and before their
// values are used, so that work of the caller's with loads of its own shares
// their round trip.  sbuf (kMaxCtx / kPS floats, LDS) serves only the radix
// fallback.  emit(pos, page) with pos ascending in page.
template <int NT, bool COH, typename Emit, typename Mid = NoMid>
__device__ __forceinline__ int top_pages_strided(const float* sc, int Np, int P, float lo, float hi, float* sbuf,
                                 TopScratch& sh, Emit emit, Mid mid = Mid()) {
  static_assert(16 * NT >= kMaxCtx / kPS, "16 pages per thread cover the largest context");
  return top_strided<NT, COH>(sc, Np, Np, P, AllPresent(), lo, hi, sbuf, sh, emit, mid);
}

__device__ __forceinline__ int keep_count_dev(int Np, int keep_num, int keep_den, int keep_abs) {
  if (Np <= 0) return 0;
  if (keep_abs > 0) return min(Np, keep_abs);
  return min(Np, max(1, (int)(((long long)keep_num * Np + keep_den - 1) / keep_den)));
}

// ====================================================== S5 + S6: fine top-k
// Candidates are the rows of the kept pages in kept order, which is ascending
// position order: candidate c = (kept slot c/16, row c%16).  Two stages:
//   distances (many workgroups): chunk k holds the candidates of kept slots
//     [64k, 64k + 64); each workgroup computes H for its chunk, writes it
//     (0xFFFF for a row past the sequence end) and adds its chunk's
//     histogram over H = 0 .. 128 G into the (b, g)'s histogram with integer
//     atomics (order-free, so exact).  Spreading this over many CUs matters:
//     per candidate it costs a 16-byte gather and ~50 vector ops;
//   selection (one workgroup per (b, g)): reads the histogram (and zeroes it
//     for the next call), finds the smallest H value T whose cumulative count
//     reaches top_k and how many candidates with H == T are taken, then
//     compacts in candidate order.
// For hhr_decode the selection stage is replaced by the attention workgroups:
// each finds its own output ranks from the distances and the histogram
// (pick_window).
// H = 0 .. 32 NW G: 32 NW G + 1 bins for NW-word codes and G heads.
template <int NW>
constexpr int ham_bins_max() { return 32 * NW * kMaxG + 1; }
constexpr int kHamBins = ham_bins_max<kNW>();         // 2049: the 128-bit composite path
constexpr int kHamBinsMax = ham_bins_max<kMaxNW>();   // 4097
constexpr int kHistCopies = 4;
constexpr int kHamChunk = kHamChunkPages * kPS;  // 1024 candidates

template <int NW>
struct HamDistSmem {
  int hist[kHistCopies][ham_bins_max<NW>()];
  int skept[kHamChunkPages];
  __attribute__((aligned(16))) uint32_t sq[kMaxG * NW];
};

// 16-byte load; the coherent form is four agent-scope dword loads.
template <bool COH>
__device__ __forceinline__ u32x4 ld_u32x4(const uint32_t* p) {
  if constexpr (COH) {
    return u32x4{Mem<true>::ld(p), Mem<true>::ld(p + 1), Mem<true>::ld(p + 2),
                 Mem<true>::ld(p + 3)};
  } else {
    return *(const u32x4*)p;
  }
}

// Distances of chunk k of (b, g): candidates c in [1024k, 1024k + 1024) with
// c < 16 P, P = the (b, g)'s kept count (nothing to do past it).  dist
// [B][Hkv][p_max*16] u16; hist [B][Hkv][128 G + 1] (counts added
// atomically); cum (or NULL) [B][Hkv][ham_cum_blocks(p_max)][128 G + 1] u16.
// Item j of every thread lies in block 4k + j of 256 candidates, whose
// histogram is LDS copy j (fewer conflicting adds); the copies are summed
// before the global adds.  Codes are NW 32-bit words.  All threads call.
template <int NT, bool COH, int NW = kNW>
__device__ void ham_dist_chunk(int b, int g, int Hq, int Hkv, int Lcap, int k, int p_max,
                               const int32_t* seq_len, const int32_t* kept_count,
                               const uint32_t* q_codes, const uint32_t* __restrict__ codes,
                               const int32_t* kept, uint16_t* dist, int* hist, uint16_t* cum,
                               HamDistSmem<NW>& sm) {
  constexpr int kItems = kHamChunk / NT;
  static_assert(NT == kCumBlock && kItems == kHistCopies, "item j = block j = LDS copy j");
  static_assert(NW == 2 || NW == 4 || NW == 8, "64-, 128- or 256-bit codes");
  const int G = Hq / Hkv;
  const int bg = b * Hkv + g;
  const int tid = threadIdx.x;
  const int nbins = 32 * NW * G + 1;
  const int page0 = k * kHamChunkPages;
  // kept pages and query codes are loaded before the kept count is known
  // (addresses clamped into the buffers), so they share its round trip
  int kp = 0;
  uint32_t qw = 0u;
  if (tid < kHamChunkPages)
    kp = Mem<COH>::ld(kept + (size_t)bg * p_max + min(page0 + tid, p_max - 1));
  if (tid < G * NW) qw = Mem<COH>::ld(q_codes + ((size_t)b * Hq + (size_t)g * G) * NW + tid);
  const int L0 = seq_len[b];
  const int L = (L0 < 0 || L0 > Lcap) ? 0 : L0;
  const int P = L > 0 ? max(0, min(kept_count[bg], p_max)) : 0;
  if (page0 >= P) return;  // block-uniform
  const int Np = (L + kPS - 1) / kPS;
  const int npg = min(kHamChunkPages, P - page0);
  const int ncl = npg * kPS;  // candidates in this chunk
  if (tid < npg) sm.skept[tid] = kp;
  if (tid < G * NW) sm.sq[tid] = qw;
  for (int i = tid; i < kHistCopies * nbins; i += NT) sm.hist[i / nbins][i % nbins] = 0;
  __syncthreads();

  const uint32_t* cb = codes + (size_t)bg * Lcap * NW;
  const int lastc = max(ncl - 1, 0);
  uint32_t code[kItems][NW];
  bool ok[kItems];
  uint32_t h[kItems];
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int c = j * NT + tid;
    const int page = sm.skept[min(c, lastc) >> 4];
    const int t = page * kPS + (c & 15);
    ok[j] = c < ncl && (unsigned)page < (unsigned)Np && t < L;
    const uint32_t* src = cb + (size_t)(ok[j] ? t : 0) * NW;
    if constexpr (NW == 2) {
      const u32x2 v = *(const u32x2*)src;
      code[j][0] = v[0];
      code[j][1] = v[1];
    } else {
#pragma unroll
      for (int v4 = 0; v4 < NW / 4; ++v4) {
        const u32x4 v = *(const u32x4*)(src + 4 * v4);
#pragma unroll
        for (int i = 0; i < 4; ++i) code[j][4 * v4 + i] = v[i];
      }
    }
    h[j] = 0u;
  }
  for (int qh = 0; qh < G; ++qh) {
    uint32_t q[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) q[i] = sm.sq[qh * NW + i];
#pragma unroll
    for (int j = 0; j < kItems; ++j)
#pragma unroll
      for (int i = 0; i < NW; ++i) h[j] += __popc(code[j][i] ^ q[i]);
  }
  uint16_t* dc = dist + (size_t)bg * p_max * kPS + (size_t)page0 * kPS;
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int c = j * NT + tid;
    if (ok[j]) atomicAdd(&sm.hist[j][h[j]], 1);
    if (c < ncl) Mem<COH>::st(dc + c, (uint16_t)(ok[j] ? h[j] : 0xFFFFu));
  }
  __syncthreads();
  int* hb = hist + (size_t)bg * nbins;
  for (int i = tid; i < nbins; i += NT) {
    int c = 0;
#pragma unroll
    for (int r = 0; r < kHistCopies; ++r) c += sm.hist[r][i];
    if (c != 0) atomicAdd(hb + i, c);  // device-scope: chunks run on every XCD
  }
  // cumulative histogram of block 4k + w by wave w, 64 bins per wave scan, so
  // each store instruction writes 128 contiguous bytes
  const int w = tid >> 6;
  const int l = tid & 63;
  if (cum == nullptr || w * kCumBlock >= ncl) return;  // wave-uniform; no barrier follows
  uint16_t* row = cum + ((size_t)bg * ham_cum_blocks(p_max) + (size_t)k * kHistCopies + w) * nbins;
  int carry = 0;
  for (int i0 = 0; i0 < nbins; i0 += kWave) {
    const int i = i0 + l;
    const int incl = wave_inclusive_scan(i < nbins ? sm.hist[w][i] : 0) + carry;
    if (i < nbins) row[i] = (uint16_t)incl;
    carry = __builtin_amdgcn_readlane(incl, kWave - 1);
  }
}

// The fine stage's spread histogram needs (nbins + 1) x (sub-bins) words: 16
// sub-bins for 128-bit codes and 4-head groups.
constexpr int kHamHistCap = 16 * (32 * kNW * 4 + 2);

struct HamSmem {
  int hist[kHamHistCap > kHamBinsMax ? kHamHistCap : kHamBinsMax];
  union {
    __attribute__((aligned(16))) uint16_t hval[kMaxCand];      // H of candidate c
    __attribute__((aligned(16))) float scores[kMaxCtx / kPS];  // page scores (S4)
  };
  int skept[kMaxCand / kPS];
  int s_T, s_need, s_valid;
  int scan[17];
  TopScratch top;
};

template <int NT, bool COH>
__device__ void ham_select_core(int bg, int P, int top_k, int nbins, int32_t* sel_idx,
                                int32_t* sel_count, HamSmem& sm);

// Selection of (b, g) from the distances and histogram its distance chunks
// wrote; leaves the histogram zero.  If skept_ready, sm.skept already holds
// the kept pages; otherwise they are read from kept.  All threads call.
template <int NT, bool COH>
__device__ void ham_select(int b, int g, int Hq, int Hkv, int P, int top_k, int p_max,
                           const int32_t* kept, bool skept_ready, const uint16_t* dist,
                           int* hist, int32_t* sel_idx, int32_t* sel_count, HamSmem& sm,
                           int code_bits = 32 * kNW) {
  const int G = Hq / Hkv;
  const int bg = b * Hkv + g;
  const int tid = threadIdx.x;
  const int ncand = P * kPS;
  const int nbins = code_bits * G + 1;

  // gather: kept pages, distances (8 per 16-byte load), summed histograms
  if (!skept_ready)
    for (int i = tid; i < P; i += NT) sm.skept[i] = Mem<COH>::ld(kept + (size_t)bg * p_max + i);
  {
    const uint32_t* d32 = reinterpret_cast<const uint32_t*>(dist + (size_t)bg * p_max * kPS);
    const int nv8 = (ncand + 7) / 8;
#pragma unroll 4
    for (int i = tid; i < nv8; i += NT)
      reinterpret_cast<u32x4*>(sm.hval)[i] = ld_u32x4<COH>(d32 + 4 * i);
  }
  int* hb = hist + (size_t)bg * nbins;
  for (int i = tid; i < nbins; i += NT) {
    sm.hist[i] = Mem<COH>::ld(hb + i);
    Mem<COH>::st(hb + i, 0);
  }
  __syncthreads();
  ham_select_core<NT, COH>(bg, P, top_k, nbins, sel_idx, sel_count, sm);
}

// The cut and the ordered compaction of ham_select, once sm.hist holds the
// histogram of the valid candidates over H = 0 .. nbins - 1, sm.hval their
// distances (0xFFFF for an invalid row) and sm.skept the P kept pages, all
// behind a barrier.  Writes sel_idx[bg][0 .. top_k) and sel_count[bg].
template <int NT, bool COH>
__device__ void ham_select_core(int bg, int P, int top_k, int nbins, int32_t* sel_idx,
                                int32_t* sel_count, HamSmem& sm) {
  const int tid = threadIdx.x;
  const int ncand = P * kPS;

  // threshold over bins in ascending H
  {
    const int per = (nbins + NT - 1) / NT;  // <= 5
    const int b0 = tid * per;
    int local = 0;
    for (int i = 0; i < per; ++i)
      if (b0 + i < nbins) local += sm.hist[b0 + i];
    int total;
    const int ex = block_exclusive_scan<NT, int>(local, sm.scan, &total);
    if (tid == 0) {
      sm.s_T = nbins;  // every valid H is < nbins: take all valid candidates
      sm.s_need = 0;
      sm.s_valid = total;
    }
    __syncthreads();
    if (total > top_k) {
      int run = ex;
      for (int i = 0; i < per; ++i) {
        if (b0 + i < nbins) {
          const int c = sm.hist[b0 + i];
          if (run < top_k && run + c >= top_k) {
            sm.s_T = b0 + i;
            sm.s_need = top_k - run;
          }
          run += c;
        }
      }
    }
    __syncthreads();
  }
  const int count = min(top_k, sm.s_valid);
  const uint32_t Th = (uint32_t)sm.s_T;
  const int need_eq = sm.s_need;

  // ordered compaction over each thread's run of candidates, read as 8
  // distances per 16-byte LDS load in rolled loops
  const int nv8 = (ncand + 8 * NT - 1) / (8 * NT);
  const int c0 = 8 * nv8 * tid;
  const u32x4* run8 = reinterpret_cast<const u32x4*>(sm.hval) + nv8 * tid;
  auto cls_of = [&](const u32x4& hw, int e, int c) -> int {
    const uint32_t word = hw[e >> 1];
    uint32_t h = (e & 1) ? (word >> 16) : (word & 0xFFFFu);
    if (c >= ncand) h = 0xFFFFu;
    return h < Th ? 1 : (h == Th ? 2 : 0);
  };
  int gt = 0, eq = 0;
#pragma unroll 1
  for (int j = 0; j < nv8; ++j) {
    const u32x4 hw = run8[j];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = cls_of(hw, e, c0 + 8 * j + e);
      gt += k == 1;
      eq += k == 2;
    }
  }
  int gb, eb;
  run_offsets<NT>(gt, eq, sm.top, gb, eb);
  int32_t* out = sel_idx + (size_t)bg * top_k;
#pragma unroll 1
  for (int j = 0; j < nv8; ++j) {
    const u32x4 hw = run8[j];
    const int cj = c0 + 8 * j;  // 8 candidates of one kept page
    const int base = sm.skept[min(cj, max(ncand - 1, 0)) >> 4] * kPS - (cj & ~15);
    auto emit = [&](int pos, int c) { Mem<COH>::st(out + pos, base + c); };
#pragma unroll
    for (int e = 0; e < 8; ++e) emit_ordered(cls_of(hw, e, cj + e), cj + e, need_eq, gb, eb, emit);
  }
  for (int i = count + tid; i < top_k; i += NT) Mem<COH>::st(out + i, -1);
  if (tid == 0) Mem<COH>::st(sel_count + bg, count);
}

// 16 bytes at byte offset off of buf (whose size is bytes), loaded with the
// sc1 cache policy: coherent with agent-scope stores of other workgroups of
// the same launch, like an agent-scope atomic load, but as one dwordx4.
__device__ __forceinline__ u32x4 ld_sc1_x4(const void* buf, uint32_t bytes, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(buf), (short)0, (int)bytes, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 16 /* sc1 */);
}

// seq_len[b], or 0 (and HHR_DEV_BAD_SEQ_LEN in *status, if given) when it is
// outside [0, Lcap].
__device__ __forceinline__ int clamped_len(const int32_t* seq_len, int b, int Lcap,
                                           uint32_t* status) {
  const int L = seq_len[b];
  if (L < 0 || L > Lcap) {
    if (status && threadIdx.x == 0) atomicOr(status, HHR_DEV_BAD_SEQ_LEN);
    return 0;
  }
  return L;
}

// The selected positions of output ranks [k0, k0 + 64) of (b, g), found
// without the compacted selection, from what k_ham_dist wrote: the distances
// (candidate c = kept slot c / 16, row c % 16, in position order), their H
// histogram and, per block of 256 candidates, the cumulative histogram.
// Candidate c is taken iff H < T, or H == T and fewer than `need` candidates
// with H == T precede it, T and need being the cut of the whole histogram.
//   pick_load (at kernel start, with the caller's other loads): the sequence
//     length and kept count, the histogram (wave 0, kPickMaxPer bins per lane
//     when 64 lanes hold them all), and -- guessed from the window's place
//     among the output ranks, as if the taken candidates were spread evenly
//     -- kPickPre blocks of distances and kept pages around the window, so
//     that usually no later load is needed.
//   pick_window: wave 0 alone finds the cut (lane-local runs of bins and one
//     wave scan) and, per block, from two entries of its cumulative
//     histogram, the counts below and at the cut and so its first output
//     rank; after one barrier every block that reaches into the window places
//     its taken candidates, ranked within the block by wave ballots
//     (prefetched blocks all at once; others loaded here).
// The result is sidx[i] = the position of output rank k0 + i (-1 past the
// selection); pick_window returns the selection size min(top_k, #valid).
// All NT = 256 threads call both.
constexpr int kPickPre = 8;  // blocks prefetched
constexpr int kPickMaxPer = 9;  // histogram bins per lane of wave 0: 576 >= 128 G + 1 for G <= 4

struct PickRegs {
  int P;
  int cnt_bin[kPickMaxPer];
  int pb0;  // first prefetched block
  uint32_t h[kPickPre];
  int pg[kPickPre];
};

struct PickSmem {
  int s_T, s_need, s_count, s_blo, s_bhi;
  int blk_first[2 * kWave];  // first output rank of each block
  int blk_eq[2 * kWave];     // candidates with H == T in earlier blocks
  int wcnt[kPickPre][4];     // per block and wave: (H < T) | (H == T) << 16
};

template <int NT>
__device__ __forceinline__ void pick_load(int b, int bg, int p_max, int Lcap, int nbins,
                                          int top_k, int k0, const int32_t* seq_len,
                                          const int32_t* kept, const int32_t* kept_count,
                                          const uint16_t* dist, const int* hist,
                                          uint32_t* status, PickRegs& pr) {
  static_assert(NT == kCumBlock, "one candidate of a block per thread");
  const int tid = threadIdx.x;
  const int L = clamped_len(seq_len, b, Lcap, status);
  const int kc = kept_count[bg];
  const int* hb = hist + (size_t)bg * nbins;
  // wave 0 takes the histogram, kPickMaxPer consecutive bins per lane (when
  // they fit; else pick_window loads them itself)
  const int perw = (nbins + kWave - 1) / kWave;
  if (tid < kWave && perw <= kPickMaxPer) {
#pragma unroll
    for (int i = 0; i < kPickMaxPer; ++i)
      pr.cnt_bin[i] = hb[min(tid * kPickMaxPer + i, nbins - 1)];
    issue_loads_here();
#pragma unroll
    for (int i = 0; i < kPickMaxPer; ++i)
      if (tid * kPickMaxPer + i >= nbins) pr.cnt_bin[i] = 0;
  }
  const int P = L > 0 ? max(0, min(kc, p_max)) : 0;
  pr.P = P;
  const int ncand = P * kPS;
  const int nblk = (ncand + kCumBlock - 1) / kCumBlock;
  const int est = max(min(top_k, ncand), 1);
  const int guess = (int)((int64_t)k0 * ncand / est) / kCumBlock;
  pr.pb0 = max(0, min(guess - kPickPre / 2 + 1, nblk - kPickPre));
  const uint16_t* db = dist + (size_t)bg * p_max * kPS;
  const int32_t* kb = kept + (size_t)bg * p_max;
  const int lastc = max(ncand - 1, 0);
#pragma unroll
  for (int u = 0; u < kPickPre; ++u) {
    const int c = min((pr.pb0 + u) * kCumBlock + tid, lastc);
    pr.h[u] = db[c];
    pr.pg[u] = kb[c >> 4];
  }
}

__device__ __forceinline__ int pick_window(int p_max, int nbins, int top_k, int k0,
                                           const int32_t* kept, const uint16_t* dist,
                                           const int* hist, const uint16_t* cum, int bg,
                                           const PickRegs& pr, int* sidx, PickSmem& ps) {
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int P = pr.P;
  const int ncand = P * kPS;
  const int nblk = (ncand + kCumBlock - 1) / kCumBlock;  // <= 2 * kWave
  if (tid < kAttnChunk) sidx[tid] = -1;

  // wave 0 alone: the cut -- the smallest T with #(H <= T) >= top_k and how
  // many H == T are taken -- from lane-local runs of bins and one wave scan;
  // then, per block, #(H < T) and #(H == T) from its cumulative histogram and
  // so its first output rank; the window's blocks are [s_blo, s_bhi]
  if (w == 0) {
    // lane l holds bins [l * perw, l * perw + perw): pick_load's kPickMaxPer
    // when they fit, else loaded here
    const int perw = (nbins + kWave - 1) / kWave <= kPickMaxPer ? kPickMaxPer
                                                                : (nbins + kWave - 1) / kWave;
    const int* hb = hist + (size_t)bg * nbins;
    auto bin = [&](int i) -> int {  // lane l's bin l * perw + i, when not in pr.cnt_bin
      const int bi = l * perw + i;
      return bi < nbins ? hb[bi] : 0;
    };
    int local = 0;
    if (perw == kPickMaxPer) {
#pragma unroll
      for (int i = 0; i < kPickMaxPer; ++i) local += pr.cnt_bin[i];
    } else {
      for (int i = 0; i < perw; ++i) local += bin(i);
    }
    const int incl = wave_inclusive_scan(local);
    const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
    int Tl = nbins, needl = 0;
    const bool mine = total > top_k && incl - local < top_k && incl >= top_k;
    if (mine) {  // the one lane whose bins cross top_k
      int run = incl - local;
      auto step = [&](int i, int c) {
        if (run < top_k && run + c >= top_k && c > 0) {
          Tl = l * perw + i;
          needl = top_k - run;
        }
        run += c;
      };
      if (perw == kPickMaxPer) {
#pragma unroll
        for (int i = 0; i < kPickMaxPer; ++i) step(i, pr.cnt_bin[i]);
      } else {
        for (int i = 0; i < perw; ++i) step(i, bin(i));
      }
    }
    const uint64_t who = __ballot(mine);
    const int src = who ? (int)__builtin_ctzll(who) : 0;
    // no crossing lane: every valid H is < nbins, take all valid candidates
    const int Th = who ? __builtin_amdgcn_readlane(Tl, src) : nbins;
    const int need = who ? __builtin_amdgcn_readlane(needl, src) : 0;
    const int count = min(top_k, total);
    int lo = 2 * kWave, hi = -1;
    if (k0 < count) {  // wave-uniform
      const uint16_t* cb = cum + (size_t)bg * ham_cum_blocks(p_max) * nbins;
      int lt[2], eq[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int blk = r * kWave + l;
        const uint16_t* row = cb + (size_t)min(blk, max(nblk - 1, 0)) * nbins;
        lt[r] = row[max(min(Th, nbins) - 1, 0)];
        eq[r] = row[min(Th, nbins - 1)];
      }
      issue_loads_here();
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int blk = r * kWave + l;
        const int below = Th == 0 ? 0 : lt[r];
        const int upto = Th >= nbins ? below : eq[r];
        lt[r] = blk < nblk ? below : 0;
        eq[r] = blk < nblk ? upto - below : 0;
      }
      int lt_carry = 0, eq_carry = 0;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int blk = r * kWave + l;
        const int lt_in = wave_inclusive_scan(lt[r]);
        const int eq_in = wave_inclusive_scan(eq[r]);
        const int lt_before = lt_carry + lt_in - lt[r];
        const int eq_before = eq_carry + eq_in - eq[r];
        const int first = lt_before + min(eq_before, need);
        const int taken = lt[r] + min(max(need - eq_before, 0), eq[r]);
        ps.blk_first[blk] = first;
        ps.blk_eq[blk] = eq_before;
        if (blk < nblk && taken > 0 && first < k0 + kAttnChunk && first + taken > k0) {
          lo = min(lo, blk);
          hi = max(hi, blk);
        }
        lt_carry += __builtin_amdgcn_readlane(lt_in, kWave - 1);
        eq_carry += __builtin_amdgcn_readlane(eq_in, kWave - 1);
      }
      lo = (int)wave_min_u((uint32_t)lo);
      hi = (int)wave_max_u((uint32_t)(hi + 1)) - 1;
    }
    if (l == 0) {
      ps.s_T = Th;
      ps.s_need = need;
      ps.s_count = count;
      ps.s_blo = lo;
      ps.s_bhi = hi;
    }
  }
  __syncthreads();
  const int count = ps.s_count;
  if (k0 >= count) return count;  // block-uniform: nothing in the window
  const int Th = ps.s_T;
  const int need = ps.s_need;
  const int blo = ps.s_blo, bhi = ps.s_bhi;
  // rank of this thread's candidate of block blk (distance hv) within the
  // block from the wave ballots and the earlier waves' counts in ps.wcnt[u]
  auto place = [&](int u, int blk, uint32_t hv, int page, uint32_t in_wave) {
    uint32_t before = in_wave;
    for (int v = 0; v < w; ++v) before += (uint32_t)ps.wcnt[u][v];
    const int lt_b = (int)(before & 0xFFFFu), eq_b = (int)(before >> 16);
    const int r = max(need - ps.blk_eq[blk], 0);  // ties still to take at the block start
    const bool tk = hv < (uint32_t)Th || (hv == (uint32_t)Th && eq_b < r);
    const int pos = ps.blk_first[blk] + lt_b + min(eq_b, r) - k0;
    const int c = blk * kCumBlock + tid;
    if (tk && pos >= 0 && pos < kAttnChunk) sidx[pos] = page * kPS + (c & 15);
  };
  auto ballots = [&](int u, uint32_t hv) -> uint32_t {
    const uint64_t blt = __ballot(hv < (uint32_t)Th);
    const uint64_t beq = __ballot(hv == (uint32_t)Th);
    if (l == 0) ps.wcnt[u][w] = (int)((uint32_t)popc64(blt) | ((uint32_t)popc64(beq) << 16));
    return mbcnt64(blt) | (mbcnt64(beq) << 16);
  };
  // the prefetched blocks that reach into the window, all at once
  uint32_t inw[kPickPre];
#pragma unroll
  for (int u = 0; u < kPickPre; ++u) {
    const int blk = pr.pb0 + u;
    inw[u] = 0u;
    if (blk >= blo && blk <= bhi) {  // block-uniform
      const uint32_t hv = blk * kCumBlock + tid < ncand ? pr.h[u] : 0xFFFFu;
      inw[u] = ballots(u, hv);
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kPickPre; ++u) {
    const int blk = pr.pb0 + u;
    if (blk >= blo && blk <= bhi) {  // block-uniform
      const uint32_t hv = blk * kCumBlock + tid < ncand ? pr.h[u] : 0xFFFFu;
      place(u, blk, hv, pr.pg[u], inw[u]);
    }
  }
  // the window's blocks that were not prefetched (a guess that missed)
  const uint16_t* db = dist + (size_t)bg * p_max * kPS;
  const int32_t* kb = kept + (size_t)bg * p_max;
#pragma unroll 1
  for (int blk = blo; blk <= bhi; ++blk) {  // block-uniform
    if (blk >= pr.pb0 && blk < pr.pb0 + kPickPre) continue;
    const int c = blk * kCumBlock + tid;
    const int cc = min(c, max(ncand - 1, 0));
    const uint32_t hv = c < ncand ? (uint32_t)db[cc] : 0xFFFFu;
    const int page = kb[cc >> 4];
    __syncthreads();  // ps.wcnt[0] is free
    const uint32_t iw = ballots(0, hv);
    __syncthreads();
    place(0, blk, hv, page, iw);
  }
  __syncthreads();
  return count;
}

// ============================================================== S7: attend
// One 256-thread group takes a chunk of up to 64 selected keys of one (b, g)
// for all G query heads (their positions from sel_idx, or, with sel_idx
// NULL, already in sm.sidx: 64 entries, -1 past nk).  It gathers the chunk's
// K and V rows with every load in flight at once (row indices clamped, data
// masked), stages K in LDS for the logits, then reuses the buffer for V;
// writes the unnormalised partial
// (o~, m, l): o~_h = sum_i e^(x_hi - m_h) V_i, m_h = max_i x_hi,
// l_h = sum_i e^(x_hi - m_h), x_hi = q_h . K_i * scale.
// The group's queries come from q, or, with q_ready, are already in sm
// (attn_put_q).
// All threads of the workgroup must call (barriers); each 256-thread group
// passes its own chunk (nk = 0 for an idle group).  Only query heads
// [h_lo, h_hi) of the group are attended and their partials written, so that
// several workgroups can share one chunk's heads when the group is large.
constexpr int kCh = kAttnChunk;      // 64 selected keys per chunk
constexpr int kRowPad = 8;           // LDS row padding (bank spread), in elements

template <bool KF32>
struct AttnSmem {
  typedef typename std::conditional<KF32, float, uint16_t>::type ET;
  static constexpr int kQRows = KF32 ? kMaxG : 1;   // f32 queries (f32 caches only)
  static constexpr int kBRows = KF32 ? 1 : kMaxG;   // bf16 hi + lo operands (bf16 caches)
  __attribute__((aligned(16))) ET rows[kCh * (kD + kRowPad)];
  float sq[kQRows][kD];
  float sp[kMaxG][kCh];
  // bf16 hi + lo of the queries (until the logits are done), then of the
  // softmax numerators: the MFMA A operands, rows padded by 16 bytes since an
  // operand read walks down 16 rows
  union {
    struct {
      __attribute__((aligned(16))) uint16_t h[kBRows][kD + 8], l[kBRows][kD + 8];
    } q;
    struct {
      __attribute__((aligned(16))) uint16_t h[kBRows][kCh + 8], l[kBRows][kCh + 8];
    } p;
  } ab;
  int sidx[kCh];
  float sm[kMaxG], sl[kMaxG];
};

// Puts the group's queries into sm: element e = tq + 256 i of the G x 128
// query block is qv[i] (e past the block: ignored).  f32 caches keep them as
// f32, bf16 caches as the bf16 hi + lo MFMA operands.  All 256 threads call
// (no barrier).
template <bool KF32, int NQ>
__device__ __forceinline__ void attn_put_q(AttnSmem<KF32>& sm, const float (&qv)[NQ], int G) {
  const int tq = threadIdx.x & 255;
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int e = tq + 256 * i;
    if (e < G * kD) {
      if constexpr (KF32) {
        sm.sq[e / kD][e % kD] = qv[i];
      } else {
        uint32_t hi, lo;
        split_bf16(qv[i], hi, lo);
        sm.ab.q.h[e / kD][e % kD] = (uint16_t)hi;
        sm.ab.q.l[e / kD][e % kD] = (uint16_t)lo;
      }
    }
  }
}

template <bool KF32, bool COH>
__device__ void attn_chunk(int b, int g, int Hq, int Hkv, int Lcap, int top_k, int k0, int nk,
                           float scale, const float* __restrict__ q,
                           const void* __restrict__ kcache, const void* __restrict__ vcache,
                           const int32_t* sel_idx, float* pout, uint32_t* status,
                           AttnSmem<KF32>& sm, int h_lo = 0, int h_hi = kMaxG,
                           bool q_ready = false) {
  typedef typename AttnSmem<KF32>::ET ET;
  constexpr int kStride = kD + kRowPad;
  constexpr int kVec = 16 / sizeof(ET);              // elements per 16-byte load
  constexpr int kChunksPerRow = kD / kVec;           // 16 (bf16) or 32 (f32)
  constexpr int kLoads = kCh * kChunksPerRow / 256;  // per thread, per matrix: 4 or 8
  const int G = Hq / Hkv;
  const int bg = b * Hkv + g;
  const int tq = threadIdx.x & 255;
  const int w = tq >> 6;
  const int l = tq & 63;

  // the chunk's positions and the group's queries, loaded together (addresses
  // clamped into the buffers, values past them dropped afterwards)
  constexpr int kQPer = kMaxG * kD / 256;
  float qv[kQPer];
  int idx = -1;
  if (!q_ready) {  // else the caller filled sm.sq
    const float* qg = q + ((size_t)b * Hq + (size_t)g * G) * kD;
#pragma unroll
    for (int i = 0; i < kQPer; ++i) qv[i] = qg[min(tq + 256 * i, G * kD - 1)];
  }
  if (sel_idx != nullptr && tq < kCh)  // else the caller filled sm.sidx (valid or -1)
    idx = Mem<COH>::ld(sel_idx + (size_t)bg * top_k + k0 + min(tq, max(nk - 1, 0)));
  issue_loads_here();
  if (sel_idx != nullptr && tq < kCh) {
    if (tq >= nk) {
      idx = -1;
    } else if (idx < 0 || idx >= Lcap) {
      if (status) atomicOr(status, HHR_DEV_BAD_INDEX);
      idx = -1;
    }
    sm.sidx[tq] = idx;
  }
  const int h_end = min(h_hi, G);  // this workgroup's query heads [h_lo, h_end)
  if (!q_ready) attn_put_q(sm, qv, G);
  __syncthreads();

  // gather: every thread issues all of its K and V loads before storing any
  const ET* kb = (const ET*)kcache + (size_t)bg * Lcap * kD;
  const ET* vb = (const ET*)vcache + (size_t)bg * Lcap * kD;
  u32x4 kreg[kLoads], vreg[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int c = tq + 256 * i;
    const int r = c / kChunksPerRow;
    const int cc = c % kChunksPerRow;
    const int idx = max(sm.sidx[r], 0);
    kreg[i] = *(const u32x4*)(kb + (size_t)idx * kD + cc * kVec);
    vreg[i] = *(const u32x4*)(vb + (size_t)idx * kD + cc * kVec);
  }
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int c = tq + 256 * i;
    const int r = c / kChunksPerRow;
    const int cc = c % kChunksPerRow;
    if (sm.sidx[r] < 0) {
      kreg[i] = u32x4{0u, 0u, 0u, 0u};
      vreg[i] = u32x4{0u, 0u, 0u, 0u};
    }
    *(u32x4*)(sm.rows + r * kStride + cc * kVec) = kreg[i];
  }
  __syncthreads();

  if constexpr (!KF32) {
    // logits on MFMA (bf16 keys): S[h][key] for 16 query-head rows (those
    // outside [h_lo, h_end) are zero) and wave w's 16 keys 16 w .. 16 w + 15,
    // K = 128 dims in 4 steps of 32.  A = the queries as bf16 hi + lo (lane:
    // head lrow, dims 32 ks + 8 lgrp ..), B = the key rows as stored
    // (lane: key 16 w + lrow, the same dims); D: lane holds S[4 lgrp + i][key].
    const int lrow = l & 15;
    const int lgrp = l >> 4;
    const bool hrow = lrow >= h_lo && lrow < h_end;
    const u32x4 z = {0u, 0u, 0u, 0u};
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) {
      const u32x4 qh = *(const u32x4*)&sm.ab.q.h[lrow][32 * ks + 8 * lgrp];
      const u32x4 ql = *(const u32x4*)&sm.ab.q.l[lrow][32 * ks + 8 * lgrp];
      const bf16x8 ahi = as_bf16x8(hrow ? qh : z);
      const bf16x8 alo = as_bf16x8(hrow ? ql : z);
      const bf16x8 bk =
          as_bf16x8(*(const u32x4*)(sm.rows + (16 * w + lrow) * kStride + 32 * ks + 8 * lgrp));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bk, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bk, acc, 0, 0, 0);
    }
    const int key = 16 * w + lrow;
    const bool kval = key < nk && sm.sidx[key] >= 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * lgrp + i;
      if (h >= h_lo && h < h_end) sm.sp[h][key] = kval ? acc[i] * scale : -__builtin_huge_valf();
    }
  } else {
  // logits: thread (key = l, head group w) -> heads w, w+4, ...
  for (int h = h_lo + w; h < h_end; h += 4) {
    const ET* row = sm.rows + l * kStride;
    float dot = 0.f;
#pragma unroll 4
    for (int c = 0; c < kD / kVec; ++c) {
      const u32x4 v = *(const u32x4*)(row + c * kVec);
      if constexpr (KF32) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dot = fmaf(sm.sq[h][4 * c + j], __uint_as_float(v[j]), dot);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dot = fmaf(sm.sq[h][8 * c + 2 * j], bf16_to_f32(v[j] & 0xFFFFu), dot);
          dot = fmaf(sm.sq[h][8 * c + 2 * j + 1], bf16_to_f32(v[j] >> 16), dot);
        }
      }
    }
    sm.sp[h][l] = (l < nk && sm.sidx[l] >= 0) ? dot * scale : -__builtin_huge_valf();
  }
  }
  __syncthreads();

  // V rows replace K rows; chunk softmax numerators
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int c = tq + 256 * i;
    *(u32x4*)(sm.rows + (c / kChunksPerRow) * kStride + (c % kChunksPerRow) * kVec) = vreg[i];
  }
  if constexpr (!KF32) {
    // all query heads at once: thread (head tq / 16, keys 4 (tq % 16) ..), the
    // max and sum over the head's 16 lanes; the numerators go out as the bf16
    // hi + lo MFMA operands
    const int h = tq >> 4;
    const int k4 = 4 * (tq & 15);
    if (h >= h_lo && h < h_end) {
      const floatx4 x = *(const floatx4*)&sm.sp[h][k4];
      float m = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
      float p[4], s = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = (x[i] == -__builtin_huge_valf()) ? 0.f : expf(x[i] - m);
        s += p[i];
      }
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) s += __shfl_xor(s, o, 16);
      const u32x2 a = split_bf16x2(p[0], p[1]), c = split_bf16x2(p[2], p[3]);
      *(u32x2*)&sm.ab.p.h[h][k4] = u32x2{a[0], c[0]};
      *(u32x2*)&sm.ab.p.l[h][k4] = u32x2{a[1], c[1]};
      if ((tq & 15) == 0) {
        sm.sm[h] = m;
        sm.sl[h] = s;
      }
    }
  } else {
  for (int h = h_lo + w; h < h_end; h += 4) {
    const float x = sm.sp[h][l];
    const float m = wave_max(x);
    const float p = (x == -__builtin_huge_valf()) ? 0.f : expf(x - m);
    const float s = wave_sum(p);
    sm.sp[h][l] = p;
    if (l == 0) {
      sm.sm[h] = m;
      sm.sl[h] = s;
    }
  }
  }
  __syncthreads();

  if constexpr (!KF32) {
    // partial o~_h[d] = sum_k p_h[k] V[k][d] on MFMA (bf16 values): 16
    // query-head rows (outside [h_lo, h_end) zero), wave w's dims 32 w ..
    // 32 w + 31 as two column tiles, K = the 64 keys in 2 steps of 32.  A = the
    // numerators as bf16 hi + lo (lane: head lrow, keys 32 ks + 8 lgrp ..),
    // B = V (lane: dim 16 nt + lrow, the same keys, read down the rows);
    // D: lane holds o~[4 lgrp + i][16 nt + lrow].
    if (nk > 0) {
      const int lrow = l & 15;
      const int lgrp = l >> 4;
      const bool hrow = lrow >= h_lo && lrow < h_end;
      bf16x8 phi[2], plo[2];
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int ks = 0; ks < kCh / 32; ++ks) {
        const u32x4 a = *(const u32x4*)&sm.ab.p.h[lrow][32 * ks + 8 * lgrp];
        const u32x4 b = *(const u32x4*)&sm.ab.p.l[lrow][32 * ks + 8 * lgrp];
        phi[ks] = as_bf16x8(hrow ? a : z);
        plo[ks] = as_bf16x8(hrow ? b : z);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int d = 32 * w + 16 * t + lrow;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kCh / 32; ++ks) {
          const ET* col = sm.rows + (32 * ks + 8 * lgrp) * kStride + d;
          uint32_t v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = col[j * kStride];
          const bf16x8 bv = as_bf16x8(u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16),
                                            v[4] | (v[5] << 16), v[6] | (v[7] << 16)});
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi[ks], bv, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo[ks], bv, acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int h = 4 * lgrp + i;
          if (h >= h_lo && h < h_end) Mem<COH>::st(pout + h * kPartStride + d, acc[i]);
        }
      }
      if (tq >= h_lo && tq < h_end) {
        Mem<COH>::st(pout + tq * kPartStride + kD, sm.sm[tq]);
        Mem<COH>::st(pout + tq * kPartStride + kD + 1, sm.sl[tq]);
      }
    }
  } else {
  // partial o~_h[d] = sum_k p_h[k] V[k][d]: lane owns dims {2l, 2l+1}, wave w heads w, w+4, ...
  if (nk > 0) {
    for (int h = h_lo + w; h < h_end; h += 4) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll 8
      for (int k = 0; k < kCh; ++k) {
        const float p = sm.sp[h][k];
        const ET* row = sm.rows + k * kStride;
        float v0, v1;
        if constexpr (KF32) {
          v0 = row[2 * l];
          v1 = row[2 * l + 1];
        } else {
          const uint32_t pair = *(const uint32_t*)(row + 2 * l);
          v0 = bf16_to_f32(pair & 0xFFFFu);
          v1 = bf16_to_f32(pair >> 16);
        }
        a0 = fmaf(p, v0, a0);
        a1 = fmaf(p, v1, a1);
      }
      Mem<COH>::st(pout + h * kPartStride + 2 * l, a0);
      Mem<COH>::st(pout + h * kPartStride + 2 * l + 1, a1);
      if (l == 0) {
        Mem<COH>::st(pout + h * kPartStride + kD, sm.sm[h]);
        Mem<COH>::st(pout + h * kPartStride + kD + 1, sm.sl[h]);
      }
    }
  }
  }
}

// Merge the ns chunk partials of query head h of one (b, g) into o_h
// (kCombThreads threads, one workgroup per (b, g, h)):
//   M = max_s m_s, f_s = e^(m_s - M), L = sum_s f_s l_s,
//   o_h = sum_s f_s o~_s / L  (o = 0 when nothing was selected).
// Thread (dim quad, s-group) sums chunks s = sgrp, sgrp + 4, ... in ascending
// order; the four s-groups are then added in order in LDS.  The first 16 of
// each thread's partials are loaded together with every (m, l) before the
// weights are known, so up to 64 chunks cost one round trip.
constexpr int kCombThreads = 128;
constexpr int kCombGroups = kCombThreads / (kD / 4);  // 4 chunk groups
constexpr int kCombMaxChunks = kMaxCand / kCh;  // 512

struct CombSmem {
  float f[kCombMaxChunks];
  float lsum;
  floatx4 red[kCombThreads];
};

template <bool COH>
__device__ __forceinline__ floatx4 ld_f32x4(const float* p) {
  if constexpr (COH) {
    return floatx4{Mem<true>::ld(p), Mem<true>::ld(p + 1), Mem<true>::ld(p + 2),
                   Mem<true>::ld(p + 3)};
  } else {
    return *(const floatx4*)p;
  }
}

// kCombThreads threads (every caller uses this count, so all sum in the same
// order).
template <bool COH>
__device__ void attn_combine(int b, int g, int h, int Hq, int Hkv, int ns, int n_split,
                             const float* part, float* __restrict__ out, CombSmem& sm) {
  constexpr int kB = 16;  // partials per thread per round trip
  const int G = Hq / Hkv;
  const int bg = b * Hkv + g;
  const int tid = threadIdx.x;
  const int l = tid & 63;
  const size_t sstride = (size_t)kMaxG * kPartStride;
  const float* pb = part + (size_t)bg * n_split * sstride + (size_t)h * kPartStride;
  const int d4 = tid % (kD / 4);
  const int sgrp = tid / (kD / 4);
  floatx4 v[kB];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int sc = min(s0 + j * kCombGroups, max(ns - 1, 0));  // clamped; weight 0 past ns
      v[j] = ld_f32x4<COH>(pb + sc * sstride + 4 * d4);
    }
  };
  // chunk weights (chunks s = l, l + 64, ...; every wave computes them, wave
  // 0 stores them).  The (m, l) of chunk l load first, then the first
  // partials, all without branches, so that waiting for the weights does not
  // wait for the partials.
  const float* ph = pb + kD;
  const int sc0 = min(l, max(ns - 1, 0));
  const float m0 = Mem<COH>::ld(ph + sc0 * sstride);
  const float l0 = Mem<COH>::ld(ph + sc0 * sstride + 1);
  load_batch(sgrp);
  {
    float M = l < ns ? m0 : -__builtin_huge_valf();
    for (int s = l + kWave; s < ns; s += kWave) M = fmaxf(M, Mem<COH>::ld(ph + s * sstride));
    M = wave_max(M);
    float ls = 0.f;
    if (l < ns) {
      const float f = (m0 == -__builtin_huge_valf()) ? 0.f : expf(m0 - M);
      if (tid < kWave) sm.f[l] = f;
      ls = fmaf(f, l0, 0.f);
    }
    for (int s = l + kWave; s < ns; s += kWave) {
      const float ms = Mem<COH>::ld(ph + s * sstride);
      const float f = (ms == -__builtin_huge_valf()) ? 0.f : expf(ms - M);
      if (tid < kWave) sm.f[s] = f;
      ls = fmaf(f, Mem<COH>::ld(ph + s * sstride + 1), ls);
    }
    ls = wave_sum(ls);
    if (tid == 0) sm.lsum = ls;
  }
  __syncthreads();
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int s0 = sgrp; s0 < ns; s0 += kB * kCombGroups) {
    if (s0 != sgrp) load_batch(s0);
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int s = s0 + j * kCombGroups;
      const float f = s < ns ? sm.f[min(s, ns - 1)] : 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = fmaf(f, v[j][k], acc[k]);
    }
  }
  sm.red[tid] = acc;
  __syncthreads();
  if (tid < kD / 4) {
    floatx4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kCombGroups; ++k) {
      const floatx4 r = sm.red[k * (kD / 4) + tid];
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] += r[j];
    }
    const float L = sm.lsum;
    floatx4 res;
#pragma unroll
    for (int j = 0; j < 4; ++j) res[j] = (ns > 0 && L > 0.f) ? o[j] / L : 0.f;
    *(floatx4*)(out + ((size_t)b * Hq + (size_t)g * G + h) * kD + 4 * tid) = res;
  }
}

}  // namespace hhr
