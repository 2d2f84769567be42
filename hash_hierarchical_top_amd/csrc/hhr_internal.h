// Host-side internals of libhhr: kernel launchers and the workspace layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/hhr.h"
#include "hhr_consts.h"

namespace hhr {

constexpr int kMaxCtx = 262144;            // Lcap limit (NpCap <= 16384)
constexpr int kMaxCand = 32768;            // kept candidates per (b, g): p_max * 16
constexpr int kAttnChunk = 64;             // selected keys per split-K workgroup
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Byte offsets of the decode workspace regions.  Region 0 (the control block)
// holds the device status word at offset 0.
struct Workspace {
  size_t ctrl = 0, counters = 0, ham_dist = 0, ham_hist = 0, ham_cum = 0, q_rot = 0, q_codes = 0,
         scores = 0, wave_range = 0, wg_thr = 0, kept = 0, kept_count = 0, attn_part = 0,
         total = 0;
  int32_t p_max = 0, n_split = 0;
};

// Scratch of the fine top-k: the H histograms (zero between calls) are the
// last part of the control block; the distances follow it.  Offsets depend
// only on the shape and p_max.
struct HamScratch {
  size_t hist = 0, dist = 0, end = 0;
};
HamScratch ham_scratch(const hhr_shape& s, int32_t p_max);
constexpr int kCountersPerGroup = 8;  // control words per (b, g) after the first 256 bytes
constexpr int kScoreCounter = 0;      // k_score_topp's arrivals
// hhr_decode lets every attention workgroup pick its own keys while there are
// at most this many of them (B * Hkv * top_k / 64), else it selects first.
constexpr int kPickInAttentionMaxWgs = 1024;

// Workspace of hhr_sparse_decode alone: control block (its counters at the
// offset every layout uses), partials.
struct AttnWorkspace {
  size_t counters = 0, part = 0, total = 0;
};
AttnWorkspace attn_workspace(const hhr_shape& s, int32_t top_k);
size_t ctrl_bytes(const hhr_shape& s);

bool make_workspace(const hhr_shape& s, int32_t keep_num, int32_t keep_den, int32_t keep_abs,
                    int32_t top_k, Workspace* ws);

// ---- launchers (all asynchronous on `stream`) ----
hipError_t launch_append_keys(const hhr_shape& s, const void* k_cache, const int32_t* start,
                              const int32_t* n_new, int32_t max_new, const float* R,
                              const float* W, uint32_t* codes, void* meta, uint32_t* status,
                              hipStream_t stream);
hipError_t launch_encode_queries(const hhr_shape& s, const float* q, const float* R,
                                 const float* W, float* q_rot, uint32_t* q_codes,
                                 hipStream_t stream);
hipError_t launch_page_scores(const hhr_shape& s, const float* q_rot, const int32_t* seq_len,
                              const void* meta, float* scores, uint32_t* status,
                              hipStream_t stream);
hipError_t launch_top_pages(const hhr_shape& s, const float* scores, const int32_t* seq_len,
                            int32_t keep_num, int32_t keep_den, int32_t keep_abs, int32_t p_max,
                            int32_t* kept, int32_t* kept_count, uint32_t* status,
                            hipStream_t stream);
hipError_t launch_ham_dist(const hhr_shape& s, const uint32_t* q_codes, const uint32_t* codes,
                           const int32_t* seq_len, const int32_t* kept,
                           const int32_t* kept_count, int32_t p_max, uint16_t* dist, int* hist,
                           uint16_t* cum, hipStream_t stream);
hipError_t launch_hamming_topk(const hhr_shape& s, const uint32_t* q_codes, const uint32_t* codes,
                               const int32_t* seq_len, const int32_t* kept,
                               const int32_t* kept_count, int32_t p_max, int32_t top_k,
                               int32_t* sel_idx, int32_t* sel_count, uint16_t* dist, int* chist,
                               uint32_t* status, hipStream_t stream);
hipError_t launch_sparse_decode(const hhr_shape& s, const float* q, const void* k_cache,
                                const void* v_cache, const int32_t* sel_idx,
                                const int32_t* sel_count, int32_t top_k, float scale, float* out,
                                float* part, int32_t n_split, uint32_t* status,
                                hipStream_t stream);

// Composite paths (hhr_select, hhr_decode): S2..S4 in one launch that ends in
// the last-arriving workgroup of each (b, g), then S5, then S6 (or, for
// hhr_decode, S6 + S7 with every attention workgroup picking its own keys).
// counters: kCountersPerGroup words per (b, g) (zero before and after every
// call): word kScoreCounter counts k_score_topp's arrivals.  wave_range:
// {smallest, largest} bound of each 16-page block, [B*Hkv][ceil(NpCap/16)].
struct CompositeBuffers {
  uint32_t* status;
  uint32_t* counters;
  float* scores;
  float* q_rot;
  float2* wave_range;
  float* wg_thr;  // each scoring workgroup's lower bound of the top-P cut
  uint32_t* q_codes;
  int32_t* kept;
  int32_t* kept_count;
  uint16_t* dist;
  int* chist;
  uint16_t* cum;  // per-block cumulative H histograms (hhr_decode's pick)
};
// A key appended at row seq_len[b] - 1 of every sequence, to be encoded (its
// code and its page's metadata) by the coarse stage before it bounds the page.
struct AppendArgs {
  const void* k_cache;
  uint32_t* codes;
  void* meta;
};

// The coarse stage (S2..S4): kept pages, counts and query codes into buf;
// with app, the appended keys are encoded first.  One launch (k_score_topp)
// when one_launch_select(s), else staged launches.
hipError_t launch_score_topp(const hhr_shape& s, const float* q, const int32_t* seq_len,
                             const float* R, const float* W, const void* meta, int32_t keep_num,
                             int32_t keep_den, int32_t keep_abs, int32_t p_max,
                             const CompositeBuffers& buf, hipStream_t stream,
                             const AppendArgs* app = nullptr);
// True when the coarse stage runs as one launch (k_score_topp): the scoring
// grid is at most two rounds of one workgroup per CU and codes are 128-bit.
bool one_launch_select(const hhr_shape& s);
// S1 for the single row seq_len[b] - 1 of every sequence with seq_len[b] >= 1.
hipError_t launch_append_last_row(const hhr_shape& s, const void* k_cache,
                                  const int32_t* seq_len, const float* R, const float* W,
                                  uint32_t* codes, void* meta, uint32_t* status,
                                  hipStream_t stream);
hipError_t launch_select_composite(const hhr_shape& s, const float* q, const int32_t* seq_len,
                                   const float* R, const float* W, const uint32_t* codes,
                                   const void* meta, int32_t keep_num, int32_t keep_den,
                                   int32_t keep_abs, int32_t p_max, int32_t top_k,
                                   int32_t* sel_idx, int32_t* sel_count,
                                   const CompositeBuffers& buf, bool finish,
                                   hipStream_t stream, const AppendArgs* app = nullptr);
// S6 + S7 for hhr_decode after launch_select_composite(..., finish = false):
// every attention workgroup picks its own chunk of the selection.
hipError_t launch_attend_picked(const hhr_shape& s, const float* q, const void* k_cache,
                                const void* v_cache, const int32_t* seq_len, int32_t p_max,
                                int32_t top_k, float scale, int32_t* sel_idx,
                                int32_t* sel_count, float* out, float* part, int32_t n_split,
                                const CompositeBuffers& buf, hipStream_t stream);


// Control block: status word at byte 0; bytes 64..255 and kCountersPerGroup
// words per (b, g) from byte 256 are reserved for cross-workgroup scheduling.
constexpr size_t kCtrlTicketsOffset = 64;

// ---- HISA ----
struct HisaWorkspace {
  size_t ctrl = 0, counters = 0, block_scores = 0, kept_blocks = 0, kept_count = 0,
         token_scores = 0, tail_reps = 0, total = 0;
};
// Arrival counters per HISA query row (zero between calls): [0] the block
// scores' (fused H3), [1] the token scores' (fused H5).
constexpr int kHisaCounters = 2;
// Rows up to which H3 runs inside the block-score launch (hisa_fused_top_blocks).
constexpr int kHisaFusedMaxRows = 64;
bool hisa_fused_top_blocks(const hhr_hisa_shape& s);
bool make_hisa_workspace(const hhr_hisa_shape& s, int32_t keep_blocks, int32_t top_k,
                         HisaWorkspace* ws);

hipError_t launch_hisa_pool(const hhr_hisa_shape& s, const uint8_t* k8, const float* k_scale,
                            const int32_t* start, const int32_t* n_new, int32_t max_new,
                            float* reps, uint32_t* status, hipStream_t stream);
hipError_t launch_hisa_block_scores(const hhr_hisa_shape& s, const uint8_t* q8,
                                    const float* q_scale, const float* w, const float* reps,
                                    const int32_t* seq_len, float* block_scores,
                                    uint32_t* status, hipStream_t stream,
                                    const uint8_t* k8 = nullptr, const float* k_scale = nullptr,
                                    float* tail = nullptr, int32_t keep_blocks = 0,
                                    int32_t* kept = nullptr, int32_t* kept_count = nullptr,
                                    uint32_t* counters = nullptr);
// (With tail: query rows against one shared cache; each row's partly visible
// last block is first pooled over its visible rows into tail [B][128].)
hipError_t launch_hisa_top_blocks(const hhr_hisa_shape& s, const float* block_scores,
                                  const int32_t* seq_len, int32_t keep_blocks, int32_t* kept,
                                  int32_t* kept_count, uint32_t* status, hipStream_t stream);
hipError_t launch_hisa_token_topk(const hhr_hisa_shape& s, const uint8_t* q8,
                                  const float* q_scale, const float* w, const uint8_t* k8,
                                  const float* k_scale, const int32_t* seq_len,
                                  const int32_t* kept, const int32_t* kept_count,
                                  int32_t keep_blocks, int32_t top_k, int32_t* sel_idx,
                                  int32_t* sel_count, float* token_scores, uint32_t* status,
                                  hipStream_t stream, bool shared = false,
                                  uint32_t* counters = nullptr);
// Rows up to which H5 runs inside the token-score launch (counters non-NULL).
bool hisa_fused_topk(const hhr_hisa_shape& s);

}  // namespace hhr
