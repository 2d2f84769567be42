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

struct ScoreRotSmem {
  QencSmem qe;
  float qrot[kMaxG][kD];
  float xnew[kD];  // the appended key's rotation (APPEND)
};

struct ScoreTopSmem {
  union {
    ScoreRotSmem rot;
    struct {
      __attribute__((aligned(16))) float sbuf[kMaxCtx / kPS];
      uint16_t cidx[kPrefilterMaxPages];  // pages of the compacted bounds
      TopScratch top;
    } sel;
  };
};

// A lower bound of the top-P cut from the scoring workgroups (see
// top_prefiltered): while it pays, every workgroup holding pages publishes a
// value that q = ceil(P / (J - 1)) of its bounds reach (all of them when it
// holds fewer), J = the workgroups holding pages.  The P largest bounds are
// then all at or above the smallest published value as long as every holding
// workgroup but one holds at least q pages: with contiguous runs all but the
// last hold ppw pages; round robin, each holds at least max(floor(nblk /
// Jg), 1) blocks, all whole but the sequence's last.  It pays when the top-P
// would otherwise hold more than 4 bounds per thread: at 128K (8192 pages)
// the step takes 42.6 instead of 43.2 us, while at 32K (2048 pages, 2 per
// thread) the workgroups' extra histogram pass cost 1 us more than the
// smaller selection saved.
constexpr int kPrefilterMinPages = 4 * kScoreThreads;

// J: the workgroups holding pages (ScoreBlocks::holders).
__device__ __forceinline__ int prefilter_quota(int Np, int P, int ppw, int J, int held) {
  if (Np <= kPrefilterMinPages || Np > kPrefilterMaxPages || J < 2 || P <= 0) return 0;
  const int q = (P + J - 2) / (J - 1);
  return q <= ppw / 2 && q <= held ? q : 0;  // 0: off (nothing dropped, or no valid bound)
}

// The 16-page blocks of one (b, g) that the scoring waves read: wave w < nwv
// (the waves with pages) of workgroup x reads block x * nwv + w (contiguous
// runs), or x + Jg w (round robin over the grid's Jg workgroups); nbc or more:
// none.  Either way each of the cache's nbc blocks has one wave.
struct ScoreBlocks {
  int nbc, nwv, Jg;
  bool rr;
  __device__ __forceinline__ int block(int x, int w) const {
    return w < nwv ? (rr ? x + Jg * w : x * nwv + w) : nbc;
  }
  // The workgroups holding some of nblk blocks: x < holders(nblk).
  __device__ __forceinline__ int holders(int nblk) const {
    return rr ? min(Jg, nblk) : (nblk + nwv - 1) / nwv;
  }
  // Pages that every holding workgroup but one holds at least.
  __device__ __forceinline__ int held(int nblk) const {
    return rr ? kScorePagesPerWave * max(nblk / Jg, 1) : kScorePagesPerWave * nwv;
  }
  // Whether block blk (in [0, nbc)) is workgroup x's.
  __device__ __forceinline__ bool holds(int x, int blk) const {
    return rr ? blk % Jg == x && blk / Jg < nwv : blk / nwv == x;
  }
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
// the grid would not cover the chip).  Which 16-page blocks a wave scores
// depends on how full the sequence's cache is (ScoreBlocks): a sequence
// filling more than half of it is read in one contiguous run of blocks per
// workgroup, a shorter one round robin over the workgroups, so that its pages
// spread over all of them (a 16K sequence in a 128K cache: 11.3 instead of
// 14.3 us for this kernel; on a full cache round robin measured 25.4
// against 22.2 us, and blocks permuted by an odd multiplier 22.3 against
// 22.0 us).  Each workgroup rotates its group's queries itself (64 KiB of R
// from L2, issued after its metadata loads so both are in flight together);
// the first workgroup of each (b, g) to finish its bounds also writes the
// query codes (the sign bits need W's columns in registers, which would not
// fit beside the metadata).
//
// APPEND: row L - 1 of every sequence is a key appended since the last encode
// (its K row is in kcache).  The workgroup that holds the last page encodes
// it with its queries (rotation, and after the bounds its code bits: the same
// per-column sums), writes its code, and the wave that holds the page folds it into the page's
// {min, max} (or starts the page with it) in registers before the bound, and
// stores the page's metadata back.  Nothing else touches that page, so no
// other workgroup can see it half-updated.
//
// While the pre-filter pays (prefilter_quota), every workgroup holding pages
// also publishes a lower bound of the cut (publish_lower_bound, into wg_thr
// [B*Hkv][gridDim.x]) before it arrives, and the last one takes the top-P
// among the pages at or above the smallest of them (top_prefiltered).
template <bool MBF, bool APPEND>
__global__ __launch_bounds__(kScoreThreads) void k_score_topp(
    const float* __restrict__ q, const int32_t* __restrict__ seq_len,
    const float* __restrict__ R, const float* __restrict__ W, void* __restrict__ meta,
    const void* __restrict__ kcache, int kv_f32, uint32_t* __restrict__ codes,
    int keep_num, int keep_den, int keep_abs, int p_max, int Hq, int Hkv, int Lcap,
    float* __restrict__ scores, float2* __restrict__ wave_range,
    uint32_t* __restrict__ q_codes, int32_t* __restrict__ kept,
    int32_t* __restrict__ kept_count, uint32_t* __restrict__ counters,
    float* __restrict__ wg_thr, uint32_t* __restrict__ status, int ppw) {
  __shared__ ScoreTopSmem sm;
  __shared__ uint32_t s_order;
  __shared__ float s_wlo[kScoreThreads / kWave], s_whi[kScoreThreads / kWave];
  __shared__ int s_bcnt[64];
  __shared__ uint32_t s_bmin[64];
  // Workgroups go to the 8 XCDs round robin by linear id; the ids are regrouped
  // so that the workgroups sharing an XCD take consecutive (b, g, x): a (b, g)
  // whose workgroups fill an XCD then reads its R through one L2.  Any
  // bijection is correct; this one only chooses which L2 serves which R.
  const int nwg = (int)(gridDim.x * gridDim.y);
  const int id = (int)(blockIdx.y * gridDim.x + blockIdx.x);
  const int lin = nwg % 8 == 0 ? (id % 8) * (nwg / 8) + id / 8 : id;
  const int wx = lin % (int)gridDim.x;
  const int bg = lin / (int)gridDim.x;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int NpCap = Lcap / kPS;
  // a wave loads its pages' metadata only once the sequence length says they
  // exist (clamped to the last one), so a short sequence in a long cache reads
  // only its own pages
  const int L = clamped_len(seq_len, b, Lcap, wx == 0 && g == 0 ? status : nullptr);
  const int Np = (L + kPS - 1) / kPS;
  const int nblk = (Np + kScorePagesPerWave - 1) / kScorePagesPerWave;
  const ScoreBlocks sb{(NpCap + kScorePagesPerWave - 1) / kScorePagesPerWave,
                       ppw / kScorePagesPerWave, (int)gridDim.x, 2 * Np <= NpCap};
  const int wv = tid >> 6;
  const int blk = sb.block(wx, wv);  // wave-uniform
  const int pb = blk * kScorePagesPerWave;
  const bool wave_has = blk < nblk;          // wave-uniform
  PageLoads<1> pl;
  if (wave_has) score_load<MBF, 1>(bg, NpCap, Np, pb, meta, pl);
  const int J = sb.holders(nblk);
  const bool wg_has = wx < J;  // block-uniform
  // the workgroup holding the last page, when a key was appended (block-uniform)
  const bool owner = APPEND && L > 0 && sb.holds(wx, nblk - 1);
  const void* key = nullptr;  // the appended key's row
  uint32_t* crow = nullptr;   // and its code
  if (APPEND && L > 0) {
    const size_t krow = ((size_t)bg * Lcap + (size_t)(L - 1)) * kD;
    key = kv_f32 ? (const void*)((const float*)kcache + krow)
                 : (const void*)((const uint16_t*)kcache + krow);
    crow = codes + ((size_t)bg * Lcap + (size_t)(L - 1)) * kNW;
  }
  // the rotation of the queries (and, in the owner, of the appended key as row
  // G) before the bounds
  if (wg_has || owner) {
    qenc_core<kD, kScoreThreads>(b, g, Hq, Hkv, q, R, W, sm.rot.qe,
                                 [&](int h, int col, float v) {
                                   if (h < G)
                                     sm.rot.qrot[h][col] = v;
                                   else
                                     sm.rot.xnew[col] = v;
                                 },
                                 [](int, int, uint32_t) {}, owner ? key : nullptr,
                                 kv_f32 != 0);
    if (owner && wave_has && pb + kScorePagesPerWave > Np - 1)  // the last page's wave
      merge_appended_row<MBF>(bg, NpCap, Np - 1, pb, (L - 1) % kPS == 0, sm.rot.xnew, meta, pl);
  }
  uint32_t* ctl = counters + (size_t)bg * kCountersPerGroup;
  float2* wr = wave_range + (size_t)bg * ((NpCap + kScorePagesPerWave - 1) / kScorePagesPerWave);
  const int P = keep_count_dev(Np, keep_num, keep_den, keep_abs);
  const int quota = prefilter_quota(Np, P, ppw, J, sb.held(nblk));  // block-uniform
  float mine = 0.f;                                 // this lane's bound (pf_lane)
  bool pf_lane = false;
  if (wave_has) {
    float A[8], B[8];
    score_ab<MBF>(G, [&](int h, int d) { return sm.rot.qrot[h][d]; }, A, B);
    float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
    score_finish<MBF, true, 1>(bg, NpCap, Np, pb, pl, A, B, scores, [&](int, float v) {
      lo = v;
      hi = v;
      mine = v;
      pf_lane = true;
    });
    lo = wave_min(lo);
    hi = wave_max(hi);
    if ((tid & 63) == 0) {
      float* dst = reinterpret_cast<float*>(wr + pb / kScorePagesPerWave);
      Mem<true>::st(dst, lo);
      Mem<true>::st(dst + 1, hi);
      s_wlo[tid >> 6] = lo;
      s_whi[tid >> 6] = hi;
    }
  } else if ((tid & 63) == 0) {
    s_wlo[tid >> 6] = __builtin_huge_valf();
    s_whi[tid >> 6] = -__builtin_huge_valf();
  }
  if (quota > 0 && wg_has) {  // block-uniform: this workgroup's lower bound of the cut
    lower_bound_init(s_bcnt, s_bmin);
    __syncthreads();  // s_wlo, s_whi and the histogram words
    float wlo = __builtin_huge_valf(), whi = -__builtin_huge_valf();
#pragma unroll
    for (int k = 0; k < kScoreThreads / kWave; ++k) {
      wlo = fminf(wlo, s_wlo[k]);
      whi = fmaxf(whi, s_whi[k]);
    }
    publish_lower_bound(mine, pf_lane, wlo, whi, quota, s_bcnt, s_bmin,
                        wg_thr + (size_t)bg * gridDim.x + wx);
  }
  // The code bits of the queries (and of the appended key, as row G) need W's
  // columns in registers, which would not fit beside the metadata; the first
  // workgroup of the (b, g) to finish its bounds computes them while the
  // others still run, off the top-P's path (the last arriver does it after
  // the top-P only when it is also the first, a grid of one).
  const size_t cbase = ((size_t)b * Hq + (size_t)g * G) * kNW;
  auto code_pass = [&]() {
    auto code_of = [&](int h, int word, uint32_t bits) {
      if (h == G)
        crow[word] = bits;
      else
        q_codes[cbase + (size_t)h * kNW + word] = bits;
    };
    auto no_rot = [](int, int, float) {};
    qenc_core<32 * kNW, kScoreThreads, decltype(no_rot), decltype(code_of), kNW, kD>(
        b, g, Hq, Hkv, q, R, W, sm.rot.qe, no_rot, code_of, key, kv_f32 != 0);
  };
  const uint32_t order = arrive_order(ctl, gridDim.x, &s_order);
  const bool last1 = order == gridDim.x - 1u;
  if (order == 0u && !last1) code_pass();  // block-uniform
  if (!last1) return;
  int32_t* out = kept + (size_t)bg * p_max;
  for (int i = P + tid; i < p_max; i += kScoreThreads) out[i] = -1;
  if (tid == 0) kept_count[bg] = P;
  if (quota > 0) {  // block-uniform: the pages below the published lower bound are out
    top_prefiltered<kScoreThreads>(scores + (size_t)bg * NpCap, Np, Np, P, AllPresent(),
                                   wg_thr + (size_t)bg * gridDim.x, J,
                                   sm.sel.sbuf, sm.sel.cidx, sm.sel.top,
                                   [&](int pos, int c) { out[pos] = c; });
  } else if (P > 0) {
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
    top_pages_strided<kScoreThreads, true>(scores + (size_t)bg * NpCap, Np, P, lo, hi,
                                           sm.sel.sbuf, sm.sel.top,
                                           [&](int pos, int c) { out[pos] = c; });
  }
  if (order == 0u) {  // block-uniform: a grid of one workgroup
    __syncthreads();  // the top-P's LDS is reused
    code_pass();
  }
}

// S6 + S7 for hhr_decode.  grid (n_split, B*Hkv), 256 threads: workgroup j
// picks the keys of output ranks [64 j, 64 j + 64) from the distances, their
// histogram and the per-block cumulative histograms (pick_load issues its
// loads at the start, together with the group's queries), writes that slice
// of sel_idx (and workgroup 0 the count), and attends over them exactly as
// k_attn would.
template <bool KF32>
__global__ __launch_bounds__(256) void k_attn_pick(
    const float* __restrict__ q, const void* __restrict__ kcache, const void* __restrict__ vcache,
    const int32_t* __restrict__ seq_len, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ kept_count, const uint16_t* __restrict__ dist,
    const int* __restrict__ hist, const uint16_t* __restrict__ cum, int p_max, int Hq, int Hkv,
    int Lcap, int top_k, int n_split, float scale, int32_t* __restrict__ sel_idx,
    int32_t* __restrict__ sel_count, float* __restrict__ part, uint32_t* __restrict__ status) {
  constexpr int kQPer = kMaxG * kD / 256;
  __shared__ AttnSmem<KF32> sm;
  __shared__ PickSmem ps;
  const int bg = blockIdx.y;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int nbins = 128 * G + 1;
  const int k0 = blockIdx.x * kCh;
  PickRegs pr;
  pick_load<256>(b, bg, p_max, Lcap, nbins, top_k, k0, seq_len, kept, kept_count, dist, hist,
                 blockIdx.x == 0 && g == 0 ? status : nullptr, pr);
  float qv[kQPer];
  const float* qg = q + ((size_t)b * Hq + (size_t)g * G) * kD;
#pragma unroll
  for (int i = 0; i < kQPer; ++i) qv[i] = qg[min(tid + 256 * i, G * kD - 1)];
  attn_put_q(sm, qv, G);
  const int count =
      pick_window(p_max, nbins, top_k, k0, kept, dist, hist, cum, bg, pr, sm.sidx, ps);
  if (tid < kCh && k0 + tid < top_k) sel_idx[(size_t)bg * top_k + k0 + tid] = sm.sidx[tid];
  if (blockIdx.x == 0 && tid == 0) sel_count[bg] = count;
  if (k0 >= count) return;  // block-uniform
  attn_chunk<KF32, true>(b, g, Hq, Hkv, Lcap, top_k, k0, min(kCh, count - k0), scale, q, kcache,
                          vcache, nullptr,
                          part + ((size_t)bg * n_split + blockIdx.x) * kMaxG * kPartStride,
                          status, sm, 0, kMaxG, true);
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
                             const AppendArgs* app) {
  const int BG = s.batch * s.n_kv_heads;
  const int NpCap = s.max_ctx / kPS;
  const int ppw = score_pages_per_wg(s);
  const dim3 grid((NpCap + ppw - 1) / ppw, BG);
  if (!one_launch_select(s)) {
    // many rounds of one-CU workgroups: the launch boundaries of the staged
    // stages cost less than the latency each round would leave exposed.  The
    // fused kernel encodes 128-bit query codes only; other widths run staged.
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
#define HHR_SCORE_TOPP(MBF, APP)                                                               \
  hipLaunchKernelGGL((k_score_topp<MBF, APP>), grid, dim3(kScoreThreads), 0, stream, q,         \
                     seq_len, R, W, m, kc, kf32, cd, keep_num, keep_den, keep_abs, p_max,      \
                     s.n_q_heads, s.n_kv_heads, s.max_ctx, buf.scores, buf.wave_range,         \
                     buf.q_codes, buf.kept, buf.kept_count, buf.counters, buf.wg_thr,       \
                     buf.status, ppw)
  const bool mbf = s.meta_dtype == HHR_BF16;
  if (mbf && app)
    HHR_SCORE_TOPP(true, true);
  else if (mbf)
    HHR_SCORE_TOPP(true, false);
  else if (app)
    HHR_SCORE_TOPP(false, true);
  else
    HHR_SCORE_TOPP(false, false);
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
#define HHR_ATTN_PICK(KF)                                                                      \
  hipLaunchKernelGGL((k_attn_pick<KF>), grid, dim3(256), 0, stream, q, k_cache, v_cache,       \
                     seq_len, buf.kept, buf.kept_count, buf.dist, buf.chist, buf.cum, p_max,    \
                     s.n_q_heads, s.n_kv_heads, s.max_ctx, top_k, n_split, scale, sel_idx,      \
                     sel_count, part, buf.status)
  if (s.kv_dtype == HHR_F32)
    HHR_ATTN_PICK(true);
  else
    HHR_ATTN_PICK(false);
#undef HHR_ATTN_PICK
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_merge, dim3(s.n_q_heads / s.n_kv_heads, BG), dim3(kCombThreads), 0,
                     stream, part, sel_count, out, buf.chist, s.n_q_heads, s.n_kv_heads, top_k,
                     n_split);
  return hipGetLastError();
}

}  // namespace hhr
