// The composite paths.  hhr_select: k_score_topp (S2 + S3 + S4), k_ham_dist,
// k_ham_select.  hhr_decode: k_score_topp, k_ham_dist, k_attn_pick (S6 + S7:
// every attention workgroup finds its own 64 selected keys), k_attn_merge.
//
// k_score_topp ends the page stage with the workgroup that finishes last:
// every workgroup writes its bounds, and each wave the smallest and largest of
// its 16, with agent-scope stores, waits for them (s_waitcnt), and bumps a
// per-(b, g) counter with an agent-scope atomic; the workgroup that brings the
// counter to the grid size resets it and runs top-P on everyone's bounds
// (read with agent-scope loads), binning them over the range the waves
// published, so it needs no pass of its own to find it.  (One atomic max per
// wave on a shared word instead costs ~25 us at 128K: they serialise.)  Nobody waits for anybody, so there
// is no scheduling hazard.  Each workgroup rotates its group's queries itself,
// so no separate query-encoding launch precedes it.
// (Measured: such a hand-off costs about as much as a kernel boundary, ~2 us;
// the gain here is the query encoding off the critical path.)
//
// Every step calls the same device functions as the one-step kernels, with
// the same thread counts where the order of floating-point sums depends on it,
// so both compositions give bit-identical results.

#include "hhr_device.h"
#include "hhr_internal.h"
#include "stages.h"

namespace hhr {

namespace {

constexpr int kScoreThreads = 1024;
// k_score_topp runs one 1024-thread workgroup per CU; past two rounds of them
// the coarse stage runs staged instead (query encode, bounds, top-P).
constexpr int kScoreToppMaxWgs = 2 * 256;
constexpr int kScorePagesPerWg = (kScoreThreads / kWave) * kScorePagesPerWave;  // 256
// With few pages (short contexts, small batches) a workgroup scores only 128
// or 64 pages (its first 8 or 4 waves), so that the scoring grid still covers
// the chip's 256 CUs; the top-P workgroup always has all 1024 threads.
constexpr int kScoreMinPagesPerWg = 4 * kScorePagesPerWave;  // 64
constexpr int kScoreTargetWgs = 256;
// Polls (about a microsecond each) before the top-P workgroup of the
// one-launch selection gives up waiting for the other workgroups' distances.
constexpr int kFineSpinMax = 1 << 20;

__device__ __forceinline__ int clamped_len(const int32_t* seq_len, int b, int Lcap,
                                           uint32_t* status) {
  const int L = seq_len[b];
  if (L < 0 || L > Lcap) {
    if (status && threadIdx.x == 0) atomicOr(status, HHR_DEV_BAD_SEQ_LEN);
    return 0;
  }
  return L;
}

// Publishes this workgroup's stores and counts it in; true in the workgroup
// that arrives last (which also re-zeroes the counter).  All threads call.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t n_wg, int* s_last) {
  wait_all_mem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = add_agent_u32(counter, 1u);
    *s_last = prev == n_wg - 1u;
    if (*s_last) st_agent_u32(counter, 0u);
  }
  __syncthreads();
  return *s_last != 0;
}

// Thread 0 polls *p (agent scope) until it reaches want, giving up after
// kFineSpinMax polls (HHR_DEV_TIMEOUT); the workgroup then meets at a
// barrier.  Used only to wait for workgroups that are already running.
__device__ __forceinline__ void wait_count(const uint32_t* p, uint32_t want, uint32_t* status);

struct ScoreRotSmem {
  QencSmem qe;
  float qrot[kMaxG][kD];
  float xnew[kD];  // the appended key's rotation (APPEND)
};

__device__ __forceinline__ void wait_count(const uint32_t* p, uint32_t want, uint32_t* status) {
  if (threadIdx.x == 0) {
    uint32_t n = ld_agent_u32(p);
    for (int spin = 0; n < want && spin < kFineSpinMax; ++spin) {
      __builtin_amdgcn_s_sleep(2);
      n = ld_agent_u32(p);
    }
    if (n < want) atomicOr(status, HHR_DEV_TIMEOUT);
  }
  __syncthreads();
}

struct ScoreTopSmem {
  union {
    ScoreRotSmem rot;
    struct {
      __attribute__((aligned(16))) float sbuf[kMaxCtx / kPS];
      TopScratch top;
    } sel;
  };
};

// With the fine stage: the top-P stages the bounds in fine.scores and emits
// the kept pages into fine.skept, then the distances of their keys replace
// the bounds (fine.hval).  The query codes stay outside the union.
struct ScoreFineSmem {
  union {
    ScoreRotSmem rot;
    HamSmem fine;
  };
  __attribute__((aligned(16))) uint32_t qc[kMaxG * kNW];
  // the top-P workgroup's own pages' distances (ham_wave_dist's packing)
  __attribute__((aligned(16))) uint16_t own_h[kScorePagesPerWg * kPS];
};

// Folds the appended key's rotation x (LDS, 128 dims) into page pn's metadata
// held by this wave (score_load's lane layout), or makes it the page's only row
// when it opens the page, and stores the page back.  f32: {min, max} per dim;
// bf16: min rounded down, max rounded up, merged as bf16 values (the rounding
// is monotone, so this equals rounding the merged f32 values).
template <bool MBF>
__device__ __forceinline__ void merge_appended_row(int bg, int NpCap, int pn, int pb, bool opens,
                                                   const float* x, void* meta,
                                                   PageLoads<1>& pl) {
  const int l = threadIdx.x & 63;
  const int r = l >> 4;
  const int sub = l & 15;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (pb + 4 * j + r != pn) continue;
    if constexpr (MBF) {
      uint32_t* dst = (uint32_t*)meta + ((size_t)bg * NpCap + pn) * kD + 4 * sub;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        floatx4 piece = pl.m[0][j][k];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = x[4 * sub + 64 * k + i];
          uint32_t lo = f32_to_bf16_down(v), hi = f32_to_bf16_up(v);
          if (!opens) {
            const uint32_t w = __float_as_uint(piece[i]);
            if (bf16_to_f32(w & 0xFFFFu) < bf16_to_f32(lo)) lo = w & 0xFFFFu;
            if (bf16_to_f32(w >> 16) > bf16_to_f32(hi)) hi = w >> 16;
          }
          piece[i] = __uint_as_float(lo | (hi << 16));
        }
        pl.m[0][j][k] = piece;
        *(floatx4*)(dst + 64 * k) = piece;
      }
    } else {
      float* dst = (float*)meta + ((size_t)bg * NpCap + pn) * kD * 2 + 4 * sub;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        floatx4 piece = pl.m[0][j][k];  // {mn[d0], mx[d0], mn[d1], mx[d1]}
        const float x0 = x[2 * sub + 32 * k], x1 = x[2 * sub + 32 * k + 1];
        piece[0] = opens ? x0 : fminf(piece[0], x0);
        piece[1] = opens ? x0 : fmaxf(piece[1], x0);
        piece[2] = opens ? x1 : fminf(piece[2], x1);
        piece[3] = opens ? x1 : fmaxf(piece[3], x1);
        pl.m[0][j][k] = piece;
        *(floatx4*)(dst + 64 * k) = piece;
      }
    }
  }
}

// S2 + S3 + S4.  grid (ceil(NpCap / ppw), B*Hkv), 1024 threads: the first
// ppw / 16 of the 16 waves score 16 pages each (ppw = 256, or 128 or 64 when
// the grid would not cover the chip).  Each workgroup rotates its group's queries itself (64 KiB of R from
// L2, issued after its metadata loads so both are in flight together);
// workgroup 0 of each (b, g) also writes the query codes.
//
// APPEND: row L - 1 of every sequence is a key appended since the last encode
// (its K row is in kcache).  The workgroup that holds the last page encodes
// it with its queries (rotation and code bits, the same per-column sums),
// writes its code, and the wave that holds the page folds it into the page's
// {min, max} (or starts the page with it) in registers before the bound, and
// stores the page's metadata back.  Nothing else touches that page, so no
// other workgroup can see it half-updated.
//
// FINE (S5 + S6 as well): every workgroup also encodes the query codes.
// After the first hand-off every other workgroup computes H for every key of
// its own pages (ham_page_wave) while the top-P runs, and counts itself in on
// a second counter.  The top-P workgroup then waits for that count, gathers
// the kept pages' distances (computing those of its own pages on the spot),
// takes the exact top-k by (H, position) and writes sel_idx and sel_count.
// So the fine stage costs one gather after the top-P instead of two further
// launches.
template <bool MBF, bool APPEND, bool FINE>
__global__ __launch_bounds__(kScoreThreads) void k_score_topp(
    const float* __restrict__ q, const int32_t* __restrict__ seq_len,
    const float* __restrict__ R, const float* __restrict__ W, void* __restrict__ meta,
    const void* __restrict__ kcache, int kv_f32, uint32_t* __restrict__ codes,
    int keep_num, int keep_den, int keep_abs, int p_max, int Hq, int Hkv, int Lcap,
    float* __restrict__ scores, float2* __restrict__ wave_range,
    uint32_t* __restrict__ q_codes, int32_t* __restrict__ kept,
    int32_t* __restrict__ kept_count, uint32_t* __restrict__ counters,
    uint32_t* __restrict__ status, const uint32_t* __restrict__ ham_codes,
    uint16_t* __restrict__ hall, int top_k, int32_t* __restrict__ sel_idx,
    int32_t* __restrict__ sel_count, int ppw) {
  using Smem = std::conditional_t<FINE, ScoreFineSmem, ScoreTopSmem>;
  __shared__ Smem sm;
  __shared__ int s_last;
  const int bg = blockIdx.y;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int NpCap = Lcap / kPS;
  const int pb = blockIdx.x * ppw + (tid >> 6) * kScorePagesPerWave;
  // a wave loads its pages' metadata only once the sequence length says they
  // exist (clamped to the last one), so a short sequence in a long cache reads
  // only its own pages
  const bool wave_in = (tid >> 6) * kScorePagesPerWave < ppw && pb < NpCap;  // wave-uniform
  const int L = clamped_len(seq_len, b, Lcap, blockIdx.x == 0 && g == 0 ? status : nullptr);
  const int Np = (L + kPS - 1) / kPS;
  const bool wave_has = wave_in && pb < Np;          // wave-uniform
  PageLoads<1> pl;
  if (wave_has) score_load<MBF, 1>(bg, NpCap, Np, pb, meta, pl);
  const bool wg_has = (int)blockIdx.x * ppw < Np;  // block-uniform
  auto to_lds = [&](int h, int col, float v) { sm.rot.qrot[h][col] = v; };
  // the workgroup holding the last page, when a key was appended (block-uniform)
  const bool owner = APPEND && L > 0 && (int)blockIdx.x == (Np - 1) / ppw;
  if (owner) {
    const size_t krow = ((size_t)bg * Lcap + (size_t)(L - 1)) * kD;
    const void* key = kv_f32 ? (const void*)((const float*)kcache + krow)
                             : (const void*)((const uint16_t*)kcache + krow);
    const size_t cbase = ((size_t)b * Hq + (size_t)g * G) * kNW;
    uint32_t* crow = codes + ((size_t)bg * Lcap + (size_t)(L - 1)) * kNW;
    auto rot_key = [&](int h, int col, float v) {
      if (h < G)
        sm.rot.qrot[h][col] = v;
      else
        sm.rot.xnew[col] = v;
    };
    auto code_key = [&](int h, int word, uint32_t bits) {
      if (h == G) {
        crow[word] = bits;
      } else {
        if constexpr (FINE) sm.qc[h * kNW + word] = bits;
        if (blockIdx.x == 0) q_codes[cbase + (size_t)h * kNW + word] = bits;
      }
    };
    qenc_core<2 * kD, kScoreThreads>(b, g, Hq, Hkv, q, R, W, sm.rot.qe, rot_key, code_key, key,
                                     kv_f32 != 0);
    if (wave_has && pb + kScorePagesPerWave > Np - 1)  // wave-uniform: the last page's wave
      merge_appended_row<MBF>(bg, NpCap, Np - 1, pb, (L - 1) % kPS == 0, sm.rot.xnew, meta, pl);
  } else if (blockIdx.x == 0 || (FINE && wg_has)) {
    const size_t cbase = ((size_t)b * Hq + (size_t)g * G) * kNW;
    qenc_core<2 * kD, kScoreThreads>(b, g, Hq, Hkv, q, R, W, sm.rot.qe, to_lds,
                      [&](int h, int word, uint32_t bits) {
                        if constexpr (FINE) sm.qc[h * kNW + word] = bits;
                        if (blockIdx.x == 0) q_codes[cbase + (size_t)h * kNW + word] = bits;
                      });
  } else if (wg_has) {
    qenc_core<kD, kScoreThreads>(b, g, Hq, Hkv, q, R, W, sm.rot.qe, to_lds,
                                 [](int, int, uint32_t) {});
  }
  uint32_t* ctl = counters + (size_t)bg * kCountersPerGroup;
  float2* wr = wave_range + (size_t)bg * (NpCap / kScorePagesPerWave);
  if (wave_has) {
    float A[8], B[8];
    score_ab<MBF>(G, [&](int h, int d) { return sm.rot.qrot[h][d]; }, A, B);
    float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
    score_finish<MBF, true, 1>(bg, NpCap, Np, pb, pl, A, B, scores, [&](int, float v) {
      lo = v;
      hi = v;
    });
    lo = wave_min(lo);
    hi = wave_max(hi);
    if ((tid & 63) == 0) {
      float* dst = reinterpret_cast<float*>(wr + pb / kScorePagesPerWave);
      Mem<true>::st(dst, lo);
      Mem<true>::st(dst + 1, hi);
    }
  }
  const bool last1 = arrive_last(ctl, gridDim.x, &s_last);
  if (!FINE && !last1) return;

  int P = 0;
  int32_t* out = kept + (size_t)bg * p_max;
  const int own_lo = blockIdx.x * ppw;
  // FINE: this workgroup's own pages' distances into LDS, their code loads
  // sharing the round trip of the top-P's staging loads
  auto own_dist = [&]() {
    if constexpr (FINE) {
      if (wave_has) {
        u32x4 c[4];
        ham_wave_codes<kNW>(bg, Lcap, pb, ham_codes, c);
        uint32_t w[2];
        ham_wave_dist(L, pb, G, sm.qc, c, w);
        const int l = tid & (kWave - 1);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          *reinterpret_cast<uint32_t*>(sm.own_h + (pb - own_lo) * kPS + 128 * j + 2 * l) = w[j];
      }
    }
  };
  if (last1) {
    P = keep_count_dev(Np, keep_num, keep_den, keep_abs);
    for (int i = P + tid; i < p_max; i += kScoreThreads) out[i] = -1;
    if (tid == 0) kept_count[bg] = P;
    if (P > 0) {
      // the range of all bounds from the waves' published {lo, hi}, one per thread
      static_assert(kMaxCtx / kPS / kScorePagesPerWave <= kScoreThreads,
                    "one wave range per thread");
      const int n_waves = (Np + kScorePagesPerWave - 1) / kScorePagesPerWave;
      float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
      if (tid < n_waves) {
        const float* src = reinterpret_cast<const float*>(wr + tid);
        lo = Mem<true>::ld(src);
        hi = Mem<true>::ld(src + 1);
      }
      if constexpr (FINE) {
        top_pages_strided<kScoreThreads, true>(scores + (size_t)bg * NpCap, Np, P, lo, hi,
                                               sm.fine.scores, sm.fine.top,
                                               [&](int pos, int c) {
                                                 out[pos] = c;
                                                 sm.fine.skept[pos] = c;
                                               },
                                               own_dist);
      } else {
        top_pages_strided<kScoreThreads, true>(scores + (size_t)bg * NpCap, Np, P, lo, hi,
                                               sm.sel.sbuf, sm.sel.top,
                                               [&](int pos, int c) { out[pos] = c; });
      }
    }
  }
  if constexpr (FINE) {
    if (!last1) {
      // H of all keys of this workgroup's pages, then count in and leave
      if (wave_has) ham_page_wave<kNW>(bg, Lcap, L, pb, G, ham_codes, sm.qc, hall);
      wait_all_mem();
      __syncthreads();
      if (tid == 0) add_agent_u32(ctl + 1, 1u);
      return;
    }
    // The top-P workgroup waits for the others' distances.  Each of them has
    // already arrived above and waits on nothing before counting in, so the
    // wait ends; it is bounded all the same (HHR_DEV_TIMEOUT).  Then the
    // counter goes back to zero: every other workgroup has counted in.
    wait_count(ctl + 1, gridDim.x - 1u, status);
    if (tid == 0) st_agent_u32(ctl + 1, 0u);
    const int nbins = kNW * 32 * G + 1;
    ham_gather_kept<kScoreThreads>(bg, Lcap, P, nbins, hall, sm.own_h, own_lo,
                                   own_lo + ppw, sm.fine);
    ham_select_core<kScoreThreads, false>(bg, P, top_k, nbins, sel_idx, sel_count, sm.fine);
  }
}

// S6 + S7 for hhr_decode.  grid (n_split, B*Hkv), 256 threads: workgroup j
// picks the keys of output ranks [64 j, 64 j + 64) straight from the
// distances and histograms (pick_window), writes that slice of sel_idx (and
// workgroup 0 the count), and attends over them exactly as k_attn would.
template <bool KF32>
__global__ __launch_bounds__(256) void k_attn_pick(
    const float* __restrict__ q, const void* __restrict__ kcache, const void* __restrict__ vcache,
    const int32_t* __restrict__ seq_len, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ kept_count, const uint16_t* __restrict__ dist,
    const int* __restrict__ hist, const uint16_t* __restrict__ cum, int p_max, int Hq, int Hkv,
    int Lcap, int top_k, int n_split,
    float scale, int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_count,
    float* __restrict__ part, uint32_t* __restrict__ status) {
  __shared__ AttnSmem<KF32> sm;
  __shared__ PickSmem ps;
  const int bg = blockIdx.y;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  const int tid = threadIdx.x;
  const int L = clamped_len(seq_len, b, Lcap, blockIdx.x == 0 && g == 0 ? status : nullptr);
  const int P = L > 0 ? max(0, min(kept_count[bg], p_max)) : 0;
  const int k0 = blockIdx.x * kCh;
  const int count = pick_window<256>(bg, P, p_max, 128 * (Hq / Hkv) + 1, top_k, k0, kept, dist,
                                     hist, cum, sm.sidx, ps);
  if (tid < kCh && k0 + tid < top_k) sel_idx[(size_t)bg * top_k + k0 + tid] = sm.sidx[tid];
  if (blockIdx.x == 0 && tid == 0) sel_count[bg] = count;
  if (k0 >= count) return;  // block-uniform
  attn_chunk<KF32, false>(b, g, Hq, Hkv, Lcap, top_k, k0, min(kCh, count - k0), scale, q, kcache,
                          vcache, nullptr,
                          part + ((size_t)bg * n_split + blockIdx.x) * kMaxG * kPartStride, status,
                          sm);
}

// The chunk merge of one (b, g, query head), then a slice of the (b, g)'s H
// histogram back to zero.  grid (G, B*Hkv).
__global__ __launch_bounds__(kCombThreads) void k_attn_merge(
    const float* __restrict__ part, const int32_t* __restrict__ sel_count,
    float* __restrict__ out, int* __restrict__ hist, int Hq, int Hkv, int top_k, int n_split) {
  __shared__ CombSmem sm;
  const int bg = blockIdx.y;
  const int h = blockIdx.x;
  const int cnt = max(0, min(sel_count[bg], top_k));
  attn_combine<false>(bg / Hkv, bg % Hkv, h, Hq, Hkv, (cnt + kCh - 1) / kCh, n_split, part, out,
                      sm);
  const int nbins = 128 * (Hq / Hkv) + 1;
  for (int i = h * kCombThreads + threadIdx.x; i < nbins; i += gridDim.x * kCombThreads)
    hist[(size_t)bg * nbins + i] = 0;
}

}  // namespace

// Pages per scoring workgroup: 256, halved (down to 64) while the grid would
// have fewer workgroups than the chip has CUs.
static int score_pages_per_wg(const hhr_shape& s) {
  const int NpCap = s.max_ctx / kPS;
  const long long BG = (long long)s.batch * s.n_kv_heads;
  int ppw = kScorePagesPerWg;
  while (ppw > kScoreMinPagesPerWg && (long long)((NpCap + ppw - 1) / ppw) * BG < kScoreTargetWgs)
    ppw /= 2;
  return ppw;
}

bool one_launch_select(const hhr_shape& s) {
  const long long wgs = (long long)((s.max_ctx / kPS + kScorePagesPerWg - 1) / kScorePagesPerWg) *
                        s.batch * s.n_kv_heads;
  return wgs <= kScoreToppMaxWgs && s.code_bits == 32 * kNW;
}

hipError_t launch_score_topp(const hhr_shape& s, const float* q, const int32_t* seq_len,
                             const float* R, const float* W, const void* meta, int32_t keep_num,
                             int32_t keep_den, int32_t keep_abs, int32_t p_max,
                             const CompositeBuffers& buf, hipStream_t stream,
                             const AppendArgs* app, const FineArgs* fine) {
  const int BG = s.batch * s.n_kv_heads;
  const int NpCap = s.max_ctx / kPS;
  const int ppw = score_pages_per_wg(s);
  const dim3 grid((NpCap + ppw - 1) / ppw, BG);
  if (!one_launch_select(s)) {
    // many rounds of one-CU workgroups: the launch boundaries of the staged
    // stages cost less than the latency each round would leave exposed.  The
    // fused kernel encodes 128-bit query codes only; other widths run staged.
    if (fine) return hipErrorInvalidValue;  // callers check one_launch_select first
    hipError_t e = hipSuccess;
    if (app)
      e = launch_append_last_row(s, app->k_cache, seq_len, R, W, app->codes, app->meta,
                                 buf.status, stream);
    if (e == hipSuccess) e = launch_encode_queries(s, q, R, W, buf.q_rot, buf.q_codes, stream);
    if (e == hipSuccess)
      e = launch_page_scores(s, buf.q_rot, seq_len, meta, buf.scores, buf.status, stream);
    if (e == hipSuccess)
      e = launch_top_pages(s, buf.scores, seq_len, keep_num, keep_den, keep_abs, p_max, buf.kept,
                           buf.kept_count, buf.status, stream);
    return e;
  }
  void* m = app ? app->meta : const_cast<void*>(meta);  // written only with APPEND
  const void* kc = app ? app->k_cache : nullptr;
  uint32_t* cd = app ? app->codes : nullptr;
  const int kf32 = s.kv_dtype == HHR_F32;
  const uint32_t* hc = fine ? fine->codes : nullptr;
  uint16_t* hall = fine ? buf.hall : nullptr;
  const int tk = fine ? fine->top_k : 0;
  int32_t* si = fine ? fine->sel_idx : nullptr;
  int32_t* sc = fine ? fine->sel_count : nullptr;
#define HHR_SCORE_TOPP(MBF, APP, FIN)                                                          \
  hipLaunchKernelGGL((k_score_topp<MBF, APP, FIN>), grid, dim3(kScoreThreads), 0, stream, q,   \
                     seq_len, R, W, m, kc, kf32, cd, keep_num, keep_den, keep_abs, p_max,      \
                     s.n_q_heads, s.n_kv_heads, s.max_ctx, buf.scores, buf.wave_range,         \
                     buf.q_codes, buf.kept, buf.kept_count, buf.counters, buf.status, hc, hall, \
                     tk, si, sc, ppw)
#define HHR_SCORE_TOPP_F(MBF, APP)     \
  if (fine)                            \
    HHR_SCORE_TOPP(MBF, APP, true);    \
  else                                 \
    HHR_SCORE_TOPP(MBF, APP, false);
  const bool mbf = s.meta_dtype == HHR_BF16;
  if (mbf && app) {
    HHR_SCORE_TOPP_F(true, true)
  } else if (mbf) {
    HHR_SCORE_TOPP_F(true, false)
  } else if (app) {
    HHR_SCORE_TOPP_F(false, true)
  } else {
    HHR_SCORE_TOPP_F(false, false)
  }
#undef HHR_SCORE_TOPP_F
#undef HHR_SCORE_TOPP
  return hipGetLastError();
}

hipError_t launch_select_composite(const hhr_shape& s, const float* q, const int32_t* seq_len,
                                   const float* R, const float* W, const uint32_t* codes,
                                   const void* meta, int32_t keep_num, int32_t keep_den,
                                   int32_t keep_abs, int32_t p_max, int32_t top_k,
                                   int32_t* sel_idx, int32_t* sel_count,
                                   const CompositeBuffers& buf, bool finish,
                                   hipStream_t stream, const AppendArgs* app) {
  if (finish && one_launch_select(s)) {
    // S2..S6 in one launch
    const FineArgs fine{codes, top_k, sel_idx, sel_count};
    return launch_score_topp(s, q, seq_len, R, W, meta, keep_num, keep_den, keep_abs, p_max, buf,
                             stream, app, &fine);
  }
  hipError_t e = launch_score_topp(s, q, seq_len, R, W, meta, keep_num, keep_den, keep_abs,
                                   p_max, buf, stream, app);
  if (e != hipSuccess) return e;
  if (finish)
    return launch_hamming_topk(s, buf.q_codes, codes, seq_len, buf.kept, buf.kept_count, p_max,
                               top_k, sel_idx, sel_count, buf.dist, buf.chist, buf.status,
                               stream);
  return launch_ham_dist(s, buf.q_codes, codes, seq_len, buf.kept, buf.kept_count, p_max,
                         buf.dist, buf.chist, buf.cum, stream);
}

hipError_t launch_attend_picked(const hhr_shape& s, const float* q, const void* k_cache,
                                const void* v_cache, const int32_t* seq_len, int32_t p_max,
                                int32_t top_k, float scale, int32_t* sel_idx,
                                int32_t* sel_count, float* out, float* part, int32_t n_split,
                                const CompositeBuffers& buf, hipStream_t stream) {
  const int BG = s.batch * s.n_kv_heads;
  dim3 grid(n_split, BG);
  if (s.kv_dtype == HHR_F32)
    hipLaunchKernelGGL(k_attn_pick<true>, grid, dim3(256), 0, stream, q, k_cache, v_cache,
                       seq_len, buf.kept, buf.kept_count, buf.dist, buf.chist, buf.cum, p_max,
                       s.n_q_heads, s.n_kv_heads, s.max_ctx, top_k, n_split, scale, sel_idx,
                       sel_count, part, buf.status);
  else
    hipLaunchKernelGGL(k_attn_pick<false>, grid, dim3(256), 0, stream, q, k_cache, v_cache,
                       seq_len, buf.kept, buf.kept_count, buf.dist, buf.chist, buf.cum, p_max,
                       s.n_q_heads, s.n_kv_heads, s.max_ctx, top_k, n_split, scale, sel_idx,
                       sel_count, part, buf.status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_merge, dim3(s.n_q_heads / s.n_kv_heads, BG), dim3(kCombThreads), 0,
                     stream, part, sel_count, out, buf.chist, s.n_q_heads, s.n_kv_heads, top_k,
                     n_split);
  return hipGetLastError();
}

}  // namespace hhr
