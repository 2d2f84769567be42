// extern "C" entry points of libhhr.so: host-side argument checks, workspace
// layout, and stream-ordered dispatch of the gfx950 kernels.  Every check runs
// before anything is enqueued, and none of the checks touches the HIP runtime,
// so the error paths are usable (and tested) on a machine without a GPU.

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "hhr_internal.h"

// Scratch of hhr_decode_no_alloc: the decode workspace (control block,
// distances, histograms, bounds, kept pages, attention partials) in a
// file-scope device array, for callers that cannot allocate.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: host code
// uses only the per-device address from hipGetSymbolAddress (no_alloc_scratch).
namespace {
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
}
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

thread_local char g_err[512] = "";

hhr_status fail(hhr_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

hhr_status ok() {
  g_err[0] = '\0';
  return HHR_OK;
}

hhr_status hip_fail(hipError_t e, const char* where) {
  return fail(HHR_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define HHR_TRY(expr)                    \
  do {                                   \
    hhr_status _st = (expr);             \
    if (_st != HHR_OK) return _st;       \
  } while (0)

#define HHR_LAUNCH(expr, where)                        \
  do {                                                 \
    hipError_t _e = (expr);                            \
    if (_e != hipSuccess) return hip_fail(_e, where);  \
  } while (0)

hhr_status check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(HHR_ERR_INVALID_ARG, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) & 15u)
    return fail(HHR_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return HHR_OK;
}

hhr_status check_opt_ptr(const void* p, const char* name) {
  return p == nullptr ? HHR_OK : check_ptr(p, name);
}

hhr_status check_shape(const hhr_shape* s) {
  if (s == nullptr) return fail(HHR_ERR_INVALID_ARG, "shape is NULL");
  if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1)
    return fail(HHR_ERR_INVALID_ARG, "batch, n_q_heads and n_kv_heads must be >= 1");
  if (s->n_q_heads % s->n_kv_heads != 0)
    return fail(HHR_ERR_INVALID_ARG, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)",
                s->n_q_heads, s->n_kv_heads);
  if (s->n_q_heads / s->n_kv_heads > hhr::kMaxG)
    return fail(HHR_ERR_UNSUPPORTED, "query heads per KV head must be <= %d", hhr::kMaxG);
  if (s->head_dim != hhr::kD) return fail(HHR_ERR_UNSUPPORTED, "head_dim must be 128");
  if (s->code_bits != 64 && s->code_bits != 128 && s->code_bits != 256)
    return fail(HHR_ERR_UNSUPPORTED, "code_bits must be 64, 128 or 256");
  if (s->page_size != hhr::kPS) return fail(HHR_ERR_UNSUPPORTED, "page_size must be 16");
  if (s->max_ctx < hhr::kPS || s->max_ctx % hhr::kPS != 0)
    return fail(HHR_ERR_INVALID_ARG, "max_ctx must be a positive multiple of 16");
  if (s->max_ctx > hhr::kMaxCtx)
    return fail(HHR_ERR_UNSUPPORTED, "max_ctx must be <= %d", hhr::kMaxCtx);
  if (s->kv_dtype != HHR_F32 && s->kv_dtype != HHR_BF16)
    return fail(HHR_ERR_INVALID_ARG, "kv_dtype must be HHR_F32 or HHR_BF16");
  if (s->meta_dtype != HHR_F32 && s->meta_dtype != HHR_BF16)
    return fail(HHR_ERR_INVALID_ARG, "meta_dtype must be HHR_F32 or HHR_BF16");
  if ((long long)s->batch * s->n_kv_heads > 65535 || (long long)s->batch * s->n_q_heads > 1 << 30)
    return fail(HHR_ERR_UNSUPPORTED, "batch * n_kv_heads must be <= 65535");
  return HHR_OK;
}

hhr_status check_keep(int32_t keep_num, int32_t keep_den, int32_t keep_abs) {
  if (keep_abs > 0) return HHR_OK;
  if (keep_abs < 0) return fail(HHR_ERR_INVALID_ARG, "keep_pages_abs must be >= 0");
  if (keep_num < 1 || keep_den < 1 || keep_num > keep_den)
    return fail(HHR_ERR_INVALID_ARG,
                "keep ratio must satisfy 1 <= keep_num <= keep_den (got %d/%d)", keep_num,
                keep_den);
  return HHR_OK;
}

hhr_status check_top_k(int32_t top_k) {
  if (top_k < 1) return fail(HHR_ERR_INVALID_ARG, "top_k must be >= 1");
  if (top_k > hhr::kMaxCand) return fail(HHR_ERR_UNSUPPORTED, "top_k must be <= %d", hhr::kMaxCand);
  return HHR_OK;
}

int32_t keep_count(int32_t n_pages, int32_t keep_num, int32_t keep_den, int32_t keep_abs) {
  if (n_pages <= 0) return 0;
  if (keep_abs > 0) return n_pages < keep_abs ? n_pages : keep_abs;
  if (keep_num < 1 || keep_den < 1) return 0;
  long long p = ((long long)keep_num * n_pages + keep_den - 1) / keep_den;
  if (p < 1) p = 1;
  return (int32_t)(p < n_pages ? p : n_pages);
}

hhr_status check_p_max(int32_t p_max) {
  if ((long long)p_max * hhr::kPS > hhr::kMaxCand)
    return fail(HHR_ERR_UNSUPPORTED,
                "at most %d candidate keys per (sequence, KV head): kept pages x 16 = %lld",
                hhr::kMaxCand, (long long)p_max * hhr::kPS);
  return HHR_OK;
}

size_t attn_part_bytes(const hhr_shape& s, int32_t n_split) {
  return (size_t)s.batch * s.n_kv_heads * n_split * hhr::kMaxG * hhr::kPartStride * sizeof(float);
}

int32_t n_split_for(int32_t top_k) { return (top_k + hhr::kAttnChunk - 1) / hhr::kAttnChunk; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

constexpr int kHisaMaxHeads = 64;
constexpr int kHisaMaxCand = 16384;

hhr_status check_hisa_shape(const hhr_hisa_shape* s) {
  if (s == nullptr) return fail(HHR_ERR_INVALID_ARG, "shape is NULL");
  if (s->batch < 1 || s->batch > 65535)
    return fail(HHR_ERR_INVALID_ARG, "batch must be in [1, 65535]");
  if (s->n_index_heads < 1) return fail(HHR_ERR_INVALID_ARG, "n_index_heads must be >= 1");
  if (s->n_index_heads > kHisaMaxHeads)
    return fail(HHR_ERR_UNSUPPORTED, "n_index_heads must be <= %d", kHisaMaxHeads);
  if (s->head_dim != hhr::kD) return fail(HHR_ERR_UNSUPPORTED, "head_dim must be 128");
  if (s->block < 16 || s->block > 1024 || s->block % 16 != 0)
    return fail(HHR_ERR_UNSUPPORTED, "block must be a multiple of 16 in [16, 1024]");
  if (s->max_ctx < s->block || s->max_ctx % s->block != 0)
    return fail(HHR_ERR_INVALID_ARG, "max_ctx must be a positive multiple of block");
  if (s->max_ctx / s->block > kHisaMaxCand || s->max_ctx > (1 << 24))
    return fail(HHR_ERR_UNSUPPORTED, "max_ctx / block must be <= %d and max_ctx <= 2^24",
                kHisaMaxCand);
  return HHR_OK;
}

hhr_status check_hisa_sel(const hhr_hisa_shape* s, int32_t keep_blocks, int32_t top_k) {
  if (keep_blocks < 1) return fail(HHR_ERR_INVALID_ARG, "keep_blocks must be >= 1");
  if ((long long)keep_blocks * s->block > kHisaMaxCand)
    return fail(HHR_ERR_UNSUPPORTED, "keep_blocks * block must be <= %d", kHisaMaxCand);
  if (top_k < 1) return fail(HHR_ERR_INVALID_ARG, "top_k must be >= 1");
  if (top_k > kHisaMaxCand) return fail(HHR_ERR_UNSUPPORTED, "top_k must be <= %d", kHisaMaxCand);
  return HHR_OK;
}

uint32_t* status_of(void* workspace) { return reinterpret_cast<uint32_t*>(workspace); }

}  // namespace

namespace hhr {

// Control block: status word and reserved words (256 B), kCountersPerGroup
// counters per (b, g), then the fine top-k H histograms; all of it is zero
// between calls, and every layout places its scratch after it.
static size_t counters_bytes(const hhr_shape& s) {
  return align_up(kCountersPerGroup * (size_t)s.batch * s.n_kv_heads * sizeof(uint32_t));
}

static size_t ham_hist_bytes(const hhr_shape& s) {
  const size_t BG = (size_t)s.batch * s.n_kv_heads;
  const size_t G = (size_t)(s.n_q_heads / s.n_kv_heads);
  return align_up(BG * ((size_t)s.code_bits * G + 1) * sizeof(int));
}

size_t ctrl_bytes(const hhr_shape& s) { return kAlign + counters_bytes(s) + ham_hist_bytes(s); }

HamScratch ham_scratch(const hhr_shape& s, int32_t p_max) {
  const size_t BG = (size_t)s.batch * s.n_kv_heads;
  HamScratch h;
  h.hist = kAlign + counters_bytes(s);
  h.dist = ctrl_bytes(s);
  h.end = h.dist + align_up(BG * (size_t)p_max * kPS * sizeof(uint16_t));
  return h;
}

AttnWorkspace attn_workspace(const hhr_shape& s, int32_t top_k) {
  AttnWorkspace a;
  a.counters = kAlign;
  a.part = ctrl_bytes(s);
  a.total = a.part + align_up(attn_part_bytes(s, n_split_for(top_k)));
  return a;
}

bool make_workspace(const hhr_shape& s, int32_t keep_num, int32_t keep_den, int32_t keep_abs,
                    int32_t top_k, Workspace* ws) {
  Workspace w;
  const int NpCap = s.max_ctx / kPS;
  w.p_max = keep_count(NpCap, keep_num, keep_den, keep_abs);
  w.n_split = n_split_for(top_k);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  const size_t BHq = (size_t)s.batch * s.n_q_heads;
  const size_t BHkv = (size_t)s.batch * s.n_kv_heads;
  // control block (same offsets in every layout): status word and reserved
  // words, counters per (b, g), fine top-k histograms
  w.ctrl = take(kAlign);
  w.counters = take(counters_bytes(s));
  w.ham_hist = take(ham_hist_bytes(s));
  const HamScratch hs = ham_scratch(s, w.p_max);
  w.ham_dist = take(hs.end - hs.dist);
  w.ham_cum = take(BHkv * (size_t)ham_cum_blocks(w.p_max) *
                   ((size_t)s.code_bits * (s.n_q_heads / s.n_kv_heads) + 1) * sizeof(uint16_t));
  w.q_rot = take(BHq * kD * sizeof(float));
  w.q_codes = take(BHq * (size_t)(s.code_bits / 32) * sizeof(uint32_t));
  w.scores = take(BHkv * NpCap * sizeof(float));
  w.wave_range = take(BHkv * (size_t)((NpCap + 15) / 16) * sizeof(float2));  // per 16-page block
  w.wg_thr = take(BHkv * (size_t)((NpCap + 63) / 64) * sizeof(float));
  w.kept = take(BHkv * (size_t)w.p_max * sizeof(int32_t));
  w.kept_count = take(BHkv * sizeof(int32_t));
  w.attn_part = take(attn_part_bytes(s, w.n_split));
  w.total = off;
  *ws = w;
  return true;
}

bool make_hisa_workspace(const hhr_hisa_shape& s, int32_t keep_blocks, int32_t top_k,
                         HisaWorkspace* ws) {
  (void)top_k;
  HisaWorkspace w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  const size_t B = (size_t)s.batch;
  w.ctrl = take(kAlign);
  w.counters = take(B * kHisaCounters * sizeof(uint32_t));
  w.block_scores = take(B * (s.max_ctx / s.block) * sizeof(float));
  w.kept_blocks = take(B * keep_blocks * sizeof(int32_t));
  w.kept_count = take(B * sizeof(int32_t));
  w.token_scores = take(B * (size_t)keep_blocks * s.block * sizeof(float));
  w.tail_reps = take(B * kD * sizeof(float));
  w.total = off;
  *ws = w;
  return true;
}

}  // namespace hhr

extern "C" {

const char* hhr_status_string(int32_t status) {
  switch (status) {
    case HHR_OK: return "HHR_OK";
    case HHR_ERR_INVALID_ARG: return "HHR_ERR_INVALID_ARG";
    case HHR_ERR_UNSUPPORTED: return "HHR_ERR_UNSUPPORTED";
    case HHR_ERR_WORKSPACE: return "HHR_ERR_WORKSPACE";
    case HHR_ERR_HIP: return "HHR_ERR_HIP";
    default: return "HHR_ERR_UNKNOWN";
  }
}

const char* hhr_last_error(void) { return g_err; }

int32_t hhr_abi_version(void) { return 5; }

int32_t hhr_keep_count(int32_t n_pages, int32_t keep_num, int32_t keep_den,
                       int32_t keep_pages_abs) {
  return keep_count(n_pages, keep_num, keep_den, keep_pages_abs);
}

size_t hhr_workspace_size(const hhr_shape* shape, int32_t keep_num, int32_t keep_den,
                          int32_t keep_pages_abs, int32_t top_k) {
  if (check_shape(shape) != HHR_OK || check_keep(keep_num, keep_den, keep_pages_abs) != HHR_OK ||
      check_top_k(top_k) != HHR_OK)
    return 0;
  hhr::Workspace ws;
  hhr::make_workspace(*shape, keep_num, keep_den, keep_pages_abs, top_k, &ws);
  if (check_p_max(ws.p_max) != HHR_OK) return 0;
  return ws.total;
}

hhr_status hhr_read_device_status(void* workspace, void* stream, uint32_t* flags) {
  HHR_TRY(check_ptr(workspace, "workspace"));
  if (flags == nullptr) return fail(HHR_ERR_INVALID_ARG, "flags is NULL");
  HHR_LAUNCH(hipStreamSynchronize(as_stream(stream)), "hipStreamSynchronize");
  uint32_t v = 0;
  HHR_LAUNCH(hipMemcpy(&v, workspace, sizeof(v), hipMemcpyDeviceToHost), "hipMemcpy");
  const uint32_t zero = 0;
  HHR_LAUNCH(hipMemcpy(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice), "hipMemcpy");
  *flags = v;
  return ok();
}

hhr_status hhr_append_keys(const hhr_shape* shape, const void* k_cache, const int32_t* start,
                           const int32_t* n_new, int32_t max_new, const float* R,
                           const float* W, uint32_t* codes, void* page_meta,
                           uint32_t* status_word, void* stream) {
  HHR_TRY(check_shape(shape));
  HHR_TRY(check_ptr(k_cache, "k_cache"));
  HHR_TRY(check_ptr(start, "start"));
  HHR_TRY(check_ptr(n_new, "n_new"));
  HHR_TRY(check_ptr(R, "R"));
  HHR_TRY(check_ptr(W, "W"));
  HHR_TRY(check_ptr(codes, "codes"));
  HHR_TRY(check_ptr(page_meta, "page_meta"));
  HHR_TRY(check_opt_ptr(status_word, "status_word"));
  if (max_new < 0 || max_new > shape->max_ctx)
    return fail(HHR_ERR_INVALID_ARG, "max_new must be in [0, max_ctx]");
  HHR_LAUNCH(hhr::launch_append_keys(*shape, k_cache, start, n_new, max_new, R, W, codes,
                                     page_meta, status_word, as_stream(stream)),
             "append_keys launch");
  return ok();
}

hhr_status hhr_encode_queries(const hhr_shape* shape, const float* q, const float* R,
                              const float* W, float* q_rot, uint32_t* q_codes, void* stream) {
  HHR_TRY(check_shape(shape));
  HHR_TRY(check_ptr(q, "q"));
  HHR_TRY(check_ptr(R, "R"));
  HHR_TRY(check_ptr(W, "W"));
  HHR_TRY(check_ptr(q_rot, "q_rot"));
  HHR_TRY(check_ptr(q_codes, "q_codes"));
  HHR_LAUNCH(hhr::launch_encode_queries(*shape, q, R, W, q_rot, q_codes, as_stream(stream)),
             "encode_queries launch");
  return ok();
}

hhr_status hhr_page_scores(const hhr_shape* shape, const float* q_rot, const int32_t* seq_len,
                           const void* page_meta, float* scores, uint32_t* status_word,
                           void* stream) {
  HHR_TRY(check_shape(shape));
  HHR_TRY(check_ptr(q_rot, "q_rot"));
  HHR_TRY(check_ptr(seq_len, "seq_len"));
  HHR_TRY(check_ptr(page_meta, "page_meta"));
  HHR_TRY(check_ptr(scores, "scores"));
  HHR_TRY(check_opt_ptr(status_word, "status_word"));
  HHR_LAUNCH(hhr::launch_page_scores(*shape, q_rot, seq_len, page_meta, scores, status_word,
                                     as_stream(stream)),
             "page_scores launch");
  return ok();
}

hhr_status hhr_top_pages(const hhr_shape* shape, const float* scores, const int32_t* seq_len,
                         int32_t keep_num, int32_t keep_den, int32_t keep_pages_abs,
                         int32_t* kept, int32_t* kept_count, uint32_t* status_word,
                         void* stream) {
  HHR_TRY(check_shape(shape));
  HHR_TRY(check_keep(keep_num, keep_den, keep_pages_abs));
  HHR_TRY(check_ptr(scores, "scores"));
  HHR_TRY(check_ptr(seq_len, "seq_len"));
  HHR_TRY(check_ptr(kept, "kept"));
  HHR_TRY(check_ptr(kept_count, "kept_count"));
  HHR_TRY(check_opt_ptr(status_word, "status_word"));
  const int32_t p_max = keep_count(shape->max_ctx / hhr::kPS, keep_num, keep_den, keep_pages_abs);
  HHR_LAUNCH(hhr::launch_top_pages(*shape, scores, seq_len, keep_num, keep_den, keep_pages_abs,
                                   p_max, kept, kept_count, status_word, as_stream(stream)),
             "top_pages launch");
  return ok();
}

hhr_status hhr_hamming_topk(const hhr_shape* shape, const uint32_t* q_codes,
                            const uint32_t* codes, const int32_t* seq_len, const int32_t* kept,
                            const int32_t* kept_count, int32_t p_max, int32_t top_k,
                            int32_t* sel_idx, int32_t* sel_count, uint16_t* dist,
                            void* workspace, size_t workspace_bytes, void* stream) {
  HHR_TRY(check_shape(shape));
  HHR_TRY(check_top_k(top_k));
  HHR_TRY(check_ptr(q_codes, "q_codes"));
  HHR_TRY(check_ptr(codes, "codes"));
  HHR_TRY(check_ptr(seq_len, "seq_len"));
  HHR_TRY(check_ptr(kept, "kept"));
  HHR_TRY(check_ptr(kept_count, "kept_count"));
  HHR_TRY(check_ptr(sel_idx, "sel_idx"));
  HHR_TRY(check_ptr(sel_count, "sel_count"));
  HHR_TRY(check_opt_ptr(dist, "dist"));
  HHR_TRY(check_ptr(workspace, "workspace"));
  if (p_max < 1 || p_max > shape->max_ctx / hhr::kPS)
    return fail(HHR_ERR_INVALID_ARG, "p_max must be in [1, max_ctx / 16]");
  HHR_TRY(check_p_max(p_max));
  const hhr::HamScratch hs = hhr::ham_scratch(*shape, p_max);
  if (workspace_bytes < hs.end)
    return fail(HHR_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, hs.end);
  char* base = static_cast<char*>(workspace);
  uint16_t* d = dist != nullptr ? dist : reinterpret_cast<uint16_t*>(base + hs.dist);
  HHR_LAUNCH(hhr::launch_hamming_topk(*shape, q_codes, codes, seq_len, kept, kept_count, p_max,
                                      top_k, sel_idx, sel_count, d,
                                      reinterpret_cast<int*>(base + hs.hist),
                                      status_of(workspace), as_stream(stream)),
             "hamming_topk launch");
  return ok();
}

hhr_status hhr_sparse_decode(const hhr_shape* shape, const float* q, const void* k_cache,
                             const void* v_cache, const int32_t* sel_idx,
                             const int32_t* sel_count, int32_t top_k, float scale, float* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  HHR_TRY(check_shape(shape));
  HHR_TRY(check_top_k(top_k));
  HHR_TRY(check_ptr(q, "q"));
  HHR_TRY(check_ptr(k_cache, "k_cache"));
  HHR_TRY(check_ptr(v_cache, "v_cache"));
  HHR_TRY(check_ptr(sel_idx, "sel_idx"));
  HHR_TRY(check_ptr(sel_count, "sel_count"));
  HHR_TRY(check_ptr(out, "out"));
  HHR_TRY(check_ptr(workspace, "workspace"));
  if (!(scale > 0.0f) || scale != scale) return fail(HHR_ERR_INVALID_ARG, "scale must be > 0");
  const int32_t n_split = n_split_for(top_k);
  const hhr::AttnWorkspace aw = hhr::attn_workspace(*shape, top_k);
  if (workspace_bytes < aw.total)
    return fail(HHR_ERR_WORKSPACE, "workspace has %zu bytes, sparse decode needs %zu",
                workspace_bytes, aw.total);
  char* base = static_cast<char*>(workspace);
  HHR_LAUNCH(hhr::launch_sparse_decode(*shape, q, k_cache, v_cache, sel_idx, sel_count, top_k,
                                       scale, out, reinterpret_cast<float*>(base + aw.part),
                                       n_split, status_of(workspace), as_stream(stream)),
             "sparse_decode launch");
  return ok();
}

// Workspace layout for these parameters and the composite kernels' buffers in it.
static hhr_status composite_buffers(const hhr_shape& shape, int32_t keep_num, int32_t keep_den,
                                    int32_t keep_abs, int32_t top_k, void* workspace,
                                    size_t workspace_bytes, hhr::Workspace* ws,
                                    hhr::CompositeBuffers* buf) {
  hhr::make_workspace(shape, keep_num, keep_den, keep_abs, top_k, ws);
  HHR_TRY(check_p_max(ws->p_max));
  if (workspace_bytes < ws->total)
    return fail(HHR_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                ws->total);
  char* base = static_cast<char*>(workspace);
  buf->status = status_of(workspace);
  buf->counters = reinterpret_cast<uint32_t*>(base + ws->counters);
  buf->scores = reinterpret_cast<float*>(base + ws->scores);
  buf->q_rot = reinterpret_cast<float*>(base + ws->q_rot);
  buf->wave_range = reinterpret_cast<float2*>(base + ws->wave_range);
  buf->wg_thr = reinterpret_cast<float*>(base + ws->wg_thr);
  buf->q_codes = reinterpret_cast<uint32_t*>(base + ws->q_codes);
  buf->kept = reinterpret_cast<int32_t*>(base + ws->kept);
  buf->kept_count = reinterpret_cast<int32_t*>(base + ws->kept_count);
  buf->dist = reinterpret_cast<uint16_t*>(base + ws->ham_dist);
  buf->chist = reinterpret_cast<int*>(base + ws->ham_hist);
  buf->cum = reinterpret_cast<uint16_t*>(base + ws->ham_cum);
  return HHR_OK;
}

hhr_status hhr_select_pages(const hhr_shape* shape, const float* q, const int32_t* seq_len,
                            const float* R, const float* W, const void* page_meta,
                            int32_t keep_num, int32_t keep_den, int32_t keep_pages_abs,
                            int32_t* kept, int32_t* kept_count, uint32_t* q_codes,
                            void* workspace, size_t workspace_bytes, void* stream) {
  HHR_TRY(check_shape(shape));
  HHR_TRY(check_keep(keep_num, keep_den, keep_pages_abs));
  HHR_TRY(check_ptr(q, "q"));
  HHR_TRY(check_ptr(seq_len, "seq_len"));
  HHR_TRY(check_ptr(R, "R"));
  HHR_TRY(check_ptr(W, "W"));
  HHR_TRY(check_ptr(page_meta, "page_meta"));
  HHR_TRY(check_ptr(kept, "kept"));
  HHR_TRY(check_ptr(kept_count, "kept_count"));
  HHR_TRY(check_opt_ptr(q_codes, "q_codes"));
  HHR_TRY(check_ptr(workspace, "workspace"));
  hhr::Workspace ws;
  hhr::CompositeBuffers buf;
  HHR_TRY(composite_buffers(*shape, keep_num, keep_den, keep_pages_abs, 1, workspace,
                            workspace_bytes, &ws, &buf));
  buf.kept = kept;
  buf.kept_count = kept_count;
  if (q_codes) buf.q_codes = q_codes;
  HHR_LAUNCH(hhr::launch_score_topp(*shape, q, seq_len, R, W, page_meta, keep_num, keep_den,
                                    keep_pages_abs, ws.p_max, buf, as_stream(stream)),
             "select_pages launch");
  return ok();
}

static hhr_status select_impl(const hhr_shape* shape, const float* q, const int32_t* seq_len,
                              const float* R, const float* W, const uint32_t* codes,
                              const void* page_meta, int32_t keep_num, int32_t keep_den,
                              int32_t keep_abs, int32_t top_k, int32_t* sel_idx,
                              int32_t* sel_count, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, bool finish, hhr::Workspace* layout,
                              hhr::CompositeBuffers* bufs,
                              const hhr::AppendArgs* app = nullptr,
                              uint32_t* status_word = nullptr) {
  HHR_TRY(check_shape(shape));
  HHR_TRY(check_keep(keep_num, keep_den, keep_abs));
  HHR_TRY(check_top_k(top_k));
  HHR_TRY(check_ptr(q, "q"));
  HHR_TRY(check_ptr(seq_len, "seq_len"));
  HHR_TRY(check_ptr(R, "R"));
  HHR_TRY(check_ptr(W, "W"));
  HHR_TRY(check_ptr(codes, "codes"));
  HHR_TRY(check_ptr(page_meta, "page_meta"));
  HHR_TRY(check_ptr(sel_idx, "sel_idx"));
  HHR_TRY(check_ptr(sel_count, "sel_count"));
  HHR_TRY(check_ptr(workspace, "workspace"));
  hhr::Workspace ws;
  hhr::CompositeBuffers buf;
  HHR_TRY(composite_buffers(*shape, keep_num, keep_den, keep_abs, top_k, workspace,
                            workspace_bytes, &ws, &buf));
  if (status_word) buf.status = status_word;  // device errors go there instead
  HHR_LAUNCH(hhr::launch_select_composite(*shape, q, seq_len, R, W, codes, page_meta, keep_num,
                                          keep_den, keep_abs, ws.p_max, top_k, sel_idx,
                                          sel_count, buf, finish, stream, app),
             "select launch");
  *layout = ws;
  *bufs = buf;
  return HHR_OK;
}

hhr_status hhr_select(const hhr_shape* shape, const float* q, const int32_t* seq_len,
                      const float* R, const float* W, const uint32_t* codes,
                      const void* page_meta, int32_t keep_num, int32_t keep_den,
                      int32_t keep_pages_abs, int32_t top_k, int32_t* sel_idx,
                      int32_t* sel_count, void* workspace, size_t workspace_bytes,
                      void* stream) {
  hhr::Workspace ws;
  hhr::CompositeBuffers buf;
  HHR_TRY(select_impl(shape, q, seq_len, R, W, codes, page_meta, keep_num, keep_den,
                      keep_pages_abs, top_k, sel_idx, sel_count, workspace, workspace_bytes,
                      as_stream(stream), true, &ws, &buf));
  return ok();
}

static hhr_status decode_impl(const hhr_shape* shape, const float* q, const int32_t* seq_len,
                              const float* R, const float* W, const uint32_t* codes,
                              const void* page_meta, const void* k_cache, const void* v_cache,
                              int32_t keep_num, int32_t keep_den, int32_t keep_pages_abs,
                              int32_t top_k, float scale, int32_t* sel_idx, int32_t* sel_count,
                              float* out, void* workspace, size_t workspace_bytes, void* stream,
                              bool append, uint32_t* status_word = nullptr) {
  HHR_TRY(check_shape(shape));
  HHR_TRY(check_ptr(k_cache, "k_cache"));
  HHR_TRY(check_ptr(v_cache, "v_cache"));
  HHR_TRY(check_ptr(out, "out"));
  if (!(scale > 0.0f) || scale != scale) return fail(HHR_ERR_INVALID_ARG, "scale must be > 0");
  // The append writes the new rows' codes and page metadata in place.
  hhr::AppendArgs app{k_cache, const_cast<uint32_t*>(codes), const_cast<void*>(page_meta)};
  hhr::Workspace ws;
  hhr::CompositeBuffers buf;
  // The coarse stage and the distances, then attention.  With few attention
  // chunks each attention workgroup picks its own keys from the distances and
  // their histogram (no selection launch); with many, one selection workgroup
  // per (b, g) runs first, which costs less than every attention workgroup
  // repeating the pick.  Same results.
  hhr::Workspace probe;
  hhr::make_workspace(*shape, keep_num, keep_den, keep_pages_abs, top_k, &probe);
  // The in-attention pick reads 128-bit-code histograms only.
  const bool pick = shape->code_bits == 32 * hhr::kNW &&
                    (long long)shape->batch * shape->n_kv_heads * probe.n_split <=
                        hhr::kPickInAttentionMaxWgs;
  HHR_TRY(select_impl(shape, q, seq_len, R, W, codes, page_meta, keep_num, keep_den,
                      keep_pages_abs, top_k, sel_idx, sel_count, workspace, workspace_bytes,
                      as_stream(stream), !pick, &ws, &buf, append ? &app : nullptr,
                      status_word));
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.attn_part);
  if (pick)
    HHR_LAUNCH(hhr::launch_attend_picked(*shape, q, k_cache, v_cache, seq_len, ws.p_max, top_k,
                                         scale, sel_idx, sel_count, out, part, ws.n_split, buf,
                                         as_stream(stream)),
               "attend launch");
  else
    HHR_LAUNCH(hhr::launch_sparse_decode(*shape, q, k_cache, v_cache, sel_idx, sel_count, top_k,
                                         scale, out, part, ws.n_split, buf.status,
                                         as_stream(stream)),
               "attend launch");
  return ok();
}

hhr_status hhr_decode(const hhr_shape* shape, const float* q, const int32_t* seq_len,
                      const float* R, const float* W, const uint32_t* codes,
                      const void* page_meta, const void* k_cache, const void* v_cache,
                      int32_t keep_num, int32_t keep_den, int32_t keep_pages_abs, int32_t top_k,
                      float scale, int32_t* sel_idx, int32_t* sel_count, float* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(shape, q, seq_len, R, W, codes, page_meta, k_cache, v_cache, keep_num,
                     keep_den, keep_pages_abs, top_k, scale, sel_idx, sel_count, out, workspace,
                     workspace_bytes, stream, false);
}

hhr_status hhr_decode_append(const hhr_shape* shape, const float* q, const int32_t* seq_len,
                             const float* R, const float* W, uint32_t* codes, void* page_meta,
                             const void* k_cache, const void* v_cache, int32_t keep_num,
                             int32_t keep_den, int32_t keep_pages_abs, int32_t top_k,
                             float scale, int32_t* sel_idx, int32_t* sel_count, float* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(shape, q, seq_len, R, W, codes, page_meta, k_cache, v_cache, keep_num,
                     keep_den, keep_pages_abs, top_k, scale, sel_idx, sel_count, out, workspace,
                     workspace_bytes, stream, true);
}


}  // extern "C"

// ------------------------------------------------------------- no-alloc decode
namespace {

// Clears n 32-bit words (the control block that must start each call at zero).
// A kernel rather than hipMemsetAsync, so that a captured graph replays it
// exactly.
__global__ __launch_bounds__(256) void k_zero_words(uint32_t* __restrict__ p, uint32_t n) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
hhr_status no_alloc_scratch(void** ptr) {
  int dev = 0;
  HHR_LAUNCH(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(HHR_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    HHR_LAUNCH(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(HHR_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return HHR_OK;
}

}  // namespace

extern "C" {

size_t hhr_no_alloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

hhr_status hhr_decode_no_alloc(const hhr_shape* shape, const float* q, const int32_t* seq_len,
                               const float* R, const float* W, const uint32_t* codes,
                               const void* page_meta, const void* k_cache, const void* v_cache,
                               int32_t keep_num, int32_t keep_den, int32_t keep_pages_abs,
                               int32_t top_k, float scale, int32_t* sel_idx, int32_t* sel_count,
                               float* out, uint32_t* status_word, void* stream) {
  // every host check of hhr_decode, before anything is enqueued
  HHR_TRY(check_shape(shape));
  HHR_TRY(check_keep(keep_num, keep_den, keep_pages_abs));
  HHR_TRY(check_top_k(top_k));
  for (const void* p : {(const void*)q, (const void*)seq_len, (const void*)R, (const void*)W,
                        (const void*)codes, page_meta, k_cache, v_cache, (const void*)sel_idx,
                        (const void*)sel_count, (const void*)out})
    HHR_TRY(check_ptr(p, "a pointer argument"));
  HHR_TRY(check_opt_ptr(status_word, "status_word"));
  if (!(scale > 0.0f) || scale != scale) return fail(HHR_ERR_INVALID_ARG, "scale must be > 0");
  hhr::Workspace ws;
  hhr::make_workspace(*shape, keep_num, keep_den, keep_pages_abs, top_k, &ws);
  HHR_TRY(check_p_max(ws.p_max));
  if (ws.total > kNoAllocScratchBytes)
    return fail(HHR_ERR_UNSUPPORTED,
                "this shape needs %zu bytes of scratch; the library's static scratch holds %zu",
                ws.total, kNoAllocScratchBytes);
  void* base = nullptr;
  HHR_TRY(no_alloc_scratch(&base));
  // the control block (status word, counters, histograms) starts at zero
  const uint32_t n_words = (uint32_t)(hhr::ctrl_bytes(*shape) / sizeof(uint32_t));
  hipLaunchKernelGGL(k_zero_words, dim3((n_words + 1023) / 1024), dim3(256), 0,
                     as_stream(stream), static_cast<uint32_t*>(base), n_words);
  HHR_LAUNCH(hipGetLastError(), "zero scratch launch");
  return decode_impl(shape, q, seq_len, R, W, codes, page_meta, k_cache, v_cache, keep_num,
                     keep_den, keep_pages_abs, top_k, scale, sel_idx, sel_count, out, base,
                     kNoAllocScratchBytes, stream, false, status_word);
}

// ------------------------------------------------------------------ HISA
size_t hhr_hisa_workspace_size(const hhr_hisa_shape* shape, int32_t keep_blocks, int32_t top_k) {
  if (check_hisa_shape(shape) != HHR_OK || check_hisa_sel(shape, keep_blocks, top_k) != HHR_OK)
    return 0;
  hhr::HisaWorkspace ws;
  hhr::make_hisa_workspace(*shape, keep_blocks, top_k, &ws);
  return ws.total;
}

hhr_status hhr_hisa_pool_keys(const hhr_hisa_shape* shape, const uint8_t* k8,
                              const float* k_scale, const int32_t* start, const int32_t* n_new,
                              int32_t max_new, float* reps, uint32_t* status_word, void* stream) {
  HHR_TRY(check_hisa_shape(shape));
  HHR_TRY(check_ptr(k8, "k8"));
  HHR_TRY(check_ptr(k_scale, "k_scale"));
  HHR_TRY(check_ptr(start, "start"));
  HHR_TRY(check_ptr(n_new, "n_new"));
  HHR_TRY(check_ptr(reps, "reps"));
  HHR_TRY(check_opt_ptr(status_word, "status_word"));
  if (max_new < 0 || max_new > shape->max_ctx)
    return fail(HHR_ERR_INVALID_ARG, "max_new must be in [0, max_ctx]");
  HHR_LAUNCH(hhr::launch_hisa_pool(*shape, k8, k_scale, start, n_new, max_new, reps, status_word,
                                   as_stream(stream)),
             "hisa_pool launch");
  return ok();
}

hhr_status hhr_hisa_block_scores(const hhr_hisa_shape* shape, const uint8_t* q8,
                                 const float* q_scale, const float* w, const float* reps,
                                 const int32_t* seq_len, float* block_scores,
                                 uint32_t* status_word, void* stream) {
  HHR_TRY(check_hisa_shape(shape));
  HHR_TRY(check_ptr(q8, "q8"));
  HHR_TRY(check_ptr(q_scale, "q_scale"));
  HHR_TRY(check_ptr(w, "w"));
  HHR_TRY(check_ptr(reps, "reps"));
  HHR_TRY(check_ptr(seq_len, "seq_len"));
  HHR_TRY(check_ptr(block_scores, "block_scores"));
  HHR_TRY(check_opt_ptr(status_word, "status_word"));
  HHR_LAUNCH(hhr::launch_hisa_block_scores(*shape, q8, q_scale, w, reps, seq_len, block_scores,
                                           status_word, as_stream(stream)),
             "hisa_block_scores launch");
  return ok();
}

hhr_status hhr_hisa_top_blocks(const hhr_hisa_shape* shape, const float* block_scores,
                               const int32_t* seq_len, int32_t keep_blocks,
                               int32_t* kept_blocks, int32_t* kept_count,
                               uint32_t* status_word, void* stream) {
  HHR_TRY(check_hisa_shape(shape));
  HHR_TRY(check_hisa_sel(shape, keep_blocks, 1));
  HHR_TRY(check_ptr(block_scores, "block_scores"));
  HHR_TRY(check_ptr(seq_len, "seq_len"));
  HHR_TRY(check_ptr(kept_blocks, "kept_blocks"));
  HHR_TRY(check_ptr(kept_count, "kept_count"));
  HHR_TRY(check_opt_ptr(status_word, "status_word"));
  HHR_LAUNCH(hhr::launch_hisa_top_blocks(*shape, block_scores, seq_len, keep_blocks, kept_blocks,
                                         kept_count, status_word, as_stream(stream)),
             "hisa_top_blocks launch");
  return ok();
}

hhr_status hhr_hisa_token_topk(const hhr_hisa_shape* shape, const uint8_t* q8,
                               const float* q_scale, const float* w, const uint8_t* k8,
                               const float* k_scale, const int32_t* seq_len,
                               const int32_t* kept_blocks, const int32_t* kept_count,
                               int32_t keep_blocks, int32_t top_k, int32_t* sel_idx,
                               int32_t* sel_count, float* token_scores, void* workspace,
                               size_t workspace_bytes, void* stream) {
  HHR_TRY(check_hisa_shape(shape));
  HHR_TRY(check_hisa_sel(shape, keep_blocks, top_k));
  HHR_TRY(check_ptr(q8, "q8"));
  HHR_TRY(check_ptr(q_scale, "q_scale"));
  HHR_TRY(check_ptr(w, "w"));
  HHR_TRY(check_ptr(k8, "k8"));
  HHR_TRY(check_ptr(k_scale, "k_scale"));
  HHR_TRY(check_ptr(seq_len, "seq_len"));
  HHR_TRY(check_ptr(kept_blocks, "kept_blocks"));
  HHR_TRY(check_ptr(kept_count, "kept_count"));
  HHR_TRY(check_ptr(sel_idx, "sel_idx"));
  HHR_TRY(check_ptr(sel_count, "sel_count"));
  HHR_TRY(check_opt_ptr(token_scores, "token_scores"));
  HHR_TRY(check_ptr(workspace, "workspace"));
  hhr::HisaWorkspace ws;
  hhr::make_hisa_workspace(*shape, keep_blocks, top_k, &ws);
  if (workspace_bytes < ws.total)
    return fail(HHR_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                ws.total);
  float* ts = token_scores ? token_scores
                           : reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.token_scores);
  // H5 inside the token-score launch when the rows are few (its arrival
  // counters live in the workspace)
  uint32_t* counters =
      hhr::hisa_fused_topk(*shape)
          ? reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + ws.counters)
          : nullptr;
  HHR_LAUNCH(hhr::launch_hisa_token_topk(*shape, q8, q_scale, w, k8, k_scale, seq_len,
                                         kept_blocks, kept_count, keep_blocks, top_k, sel_idx,
                                         sel_count, ts, status_of(workspace), as_stream(stream),
                                         false, counters),
             "hisa_token_topk launch");
  return ok();
}

static hhr_status hisa_select_impl(const hhr_hisa_shape* shape, const uint8_t* q8,
                                   const float* q_scale, const float* w, const uint8_t* k8,
                                   const float* k_scale, const float* reps,
                                   const int32_t* seq_len, int32_t keep_blocks, int32_t top_k,
                                   int32_t* sel_idx, int32_t* sel_count, void* workspace,
                                   size_t workspace_bytes, void* stream, bool shared) {
  HHR_TRY(check_hisa_shape(shape));
  HHR_TRY(check_hisa_sel(shape, keep_blocks, top_k));
  HHR_TRY(check_ptr(q8, "q8"));
  HHR_TRY(check_ptr(q_scale, "q_scale"));
  HHR_TRY(check_ptr(w, "w"));
  HHR_TRY(check_ptr(k8, "k8"));
  HHR_TRY(check_ptr(k_scale, "k_scale"));
  HHR_TRY(check_ptr(reps, "reps"));
  HHR_TRY(check_ptr(seq_len, "seq_len"));
  HHR_TRY(check_ptr(sel_idx, "sel_idx"));
  HHR_TRY(check_ptr(sel_count, "sel_count"));
  HHR_TRY(check_ptr(workspace, "workspace"));
  hhr::HisaWorkspace ws;
  hhr::make_hisa_workspace(*shape, keep_blocks, top_k, &ws);
  if (workspace_bytes < ws.total)
    return fail(HHR_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                ws.total);
  char* base = static_cast<char*>(workspace);
  uint32_t* status = status_of(workspace);
  float* bs = reinterpret_cast<float*>(base + ws.block_scores);
  int32_t* kept = reinterpret_cast<int32_t*>(base + ws.kept_blocks);
  int32_t* kc = reinterpret_cast<int32_t*>(base + ws.kept_count);
  float* ts = reinterpret_cast<float*>(base + ws.token_scores);
  hipStream_t st = as_stream(stream);
  float* tail = shared ? reinterpret_cast<float*>(base + ws.tail_reps) : nullptr;
  // H3 inside the block-score launch when the rows are few and short enough
  if (hhr::hisa_fused_top_blocks(*shape)) {
    uint32_t* counters = reinterpret_cast<uint32_t*>(base + ws.counters);
    HHR_LAUNCH(hhr::launch_hisa_block_scores(*shape, q8, q_scale, w, reps, seq_len, bs, status,
                                             st, k8, k_scale, tail, keep_blocks, kept, kc,
                                             counters),
               "hisa_block_scores launch");
  } else {
    HHR_LAUNCH(hhr::launch_hisa_block_scores(*shape, q8, q_scale, w, reps, seq_len, bs, status,
                                             st, k8, k_scale, tail),
               "hisa_block_scores launch");
    HHR_LAUNCH(hhr::launch_hisa_top_blocks(*shape, bs, seq_len, keep_blocks, kept, kc, status,
                                           st),
               "hisa_top_blocks launch");
  }
  // H5 inside the token-score launch when the rows are few
  HHR_LAUNCH(hhr::launch_hisa_token_topk(
                 *shape, q8, q_scale, w, k8, k_scale, seq_len, kept, kc, keep_blocks, top_k,
                 sel_idx, sel_count, ts, status, st, shared,
                 hhr::hisa_fused_topk(*shape) ? reinterpret_cast<uint32_t*>(base + ws.counters)
                                              : nullptr),
             "hisa_token_topk launch");
  return ok();
}

hhr_status hhr_hisa_select(const hhr_hisa_shape* shape, const uint8_t* q8, const float* q_scale,
                           const float* w, const uint8_t* k8, const float* k_scale,
                           const float* reps, const int32_t* seq_len, int32_t keep_blocks,
                           int32_t top_k, int32_t* sel_idx, int32_t* sel_count, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return hisa_select_impl(shape, q8, q_scale, w, k8, k_scale, reps, seq_len, keep_blocks, top_k,
                          sel_idx, sel_count, workspace, workspace_bytes, stream, false);
}

hhr_status hhr_hisa_prefill_select(const hhr_hisa_shape* shape, const uint8_t* q8,
                                   const float* q_scale, const float* w, const uint8_t* k8,
                                   const float* k_scale, const float* reps,
                                   const int32_t* q_len, int32_t keep_blocks, int32_t top_k,
                                   int32_t* sel_idx, int32_t* sel_count, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return hisa_select_impl(shape, q8, q_scale, w, k8, k_scale, reps, q_len, keep_blocks, top_k,
                          sel_idx, sel_count, workspace, workspace_bytes, stream, true);
}

}  // extern "C"
