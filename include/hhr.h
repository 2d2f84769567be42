/*
 * hhr.h -- C ABI of libhhr.so: coarse-to-fine hash retrieval for long-context
 * decode (HHR / HATA) and the HISA hierarchical indexer, on AMD Instinct MI355X
 * (gfx950).
 *
 * Sources (page titles as printed):
 *   [HHR]  "HHR: Hierarchical Hash Retrieval for Efficient LLM Generation"
 *          (arXiv 2610.01230): abstract; Figure 1 (overview), Figure 2 (sign of
 *          a projection), Figure 4 (per-KV-head top-k recall); appendix Table 3
 *          (Llama-3.1-8B shape) and Table 4 (128-bit hash codes).
 *   [HATA] "HATA: Trainable and Hardware-Efficient Hash-Aware Top-k Attention
 *          for Scalable Large Model Inference" (arXiv 2506.02572): abstract.
 *   [HISA] "HISA: Efficient Hierarchical Indexing for Fine-Grained Sparse
 *          Attention" (arXiv 2603.28458): abstract.
 *
 * One decode step for one (sequence b, KV head g) with the G = Hq/Hkv query
 * heads h of its group:
 *   S1 append:   X = K R_g (rotated keys), code(k) = sign bits of K W_g,
 *                page metadata = per-page per-dim [min, max] of X      [HHR abstract]
 *   S2 query:    q'_h = q_h R_g, c_h = sign bits of q_h W_g
 *   S3 bound:    s(p) = sum_h sum_d max(q'_hd * mn_pd, q'_hd * mx_pd)  [HHR abstract, GKR]
 *   S4 prune:    keep the P pages with the largest s (ties: lower page)
 *   S5 Hamming:  H(t) = sum_h popcount(c_h XOR code(t)), t in kept pages [HHR abstract, LHP]
 *   S6 top-k:    the k keys with the smallest (H, t)                    [HATA abstract]
 *   S7 attend:   o_h = softmax(q_h K_sel^T * scale) V_sel               [HHR abstract]
 *
 * Conventions shared by every entry point
 *   - Pointers named in the argument lists are DEVICE pointers unless the
 *     comment says "host".  The caller allocates and owns every buffer; the
 *     library allocates nothing and keeps no state between calls.
 *   - Device pointers must be 16-byte aligned.
 *   - Every call is asynchronous and ordered on `stream` (a hipStream_t; NULL
 *     is the null stream).  Host-side argument checks run before anything is
 *     enqueued; on any non-OK return nothing has been enqueued.
 *   - Layouts are dense row-major C arrays; the bracketed shapes below list
 *     dimensions outermost first.  B = batch, Hq = query heads, Hkv = KV
 *     heads, d = head_dim (128), Lcap = max_ctx, ps = page_size (16),
 *     NpCap = Lcap / ps, nw = code_bits / 32 (2, 4 or 8).
 *   - Device-side data errors (a seq_len outside [0, Lcap], a selected
 *     position outside [0, Lcap)) never fault: the offending sequence is
 *     treated as empty / the position is skipped, and a bit is set in the
 *     workspace status word (read it with hhr_read_device_status).
 *   - Results are deterministic: repeated calls on the same inputs give
 *     bit-identical outputs.
 *   - Workspace: device memory of at least the size the matching
 *     *_workspace_size() function returns, zero-filled before its first use.
 *     It starts with a control block: the device status word at offset 0;
 *     bytes 64..255, eight words per (b, g) from offset 256 and then one
 *     H histogram per (b, g) (the fine top-k's) are reserved and zero
 *     between calls.  Every call leaves them zero again; the status word
 *     keeps its error bits until hhr_read_device_status clears it.  The
 *     control block sits at the same offsets in every HHR layout and every
 *     other region follows it, so one workspace may serve every HHR entry
 *     point; the HISA entry points use a workspace of their own.  Calls that
 *     share a workspace must not overlap in time (order them on one stream).
 */
#ifndef HHR_H_
#define HHR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */
typedef enum {
  HHR_OK = 0,
  HHR_ERR_INVALID_ARG = -1, /* null/misaligned pointer, inconsistent sizes     */
  HHR_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels implement   */
  HHR_ERR_WORKSPACE = -3,   /* workspace smaller than hhr_workspace_size()    */
  HHR_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed     */
} hhr_status;

/* Device status bits (hhr_read_device_status). */
#define HHR_DEV_BAD_SEQ_LEN 0x1u  /* a seq_len was < 0 or > max_ctx           */
#define HHR_DEV_BAD_INDEX 0x2u    /* a selected position was outside [0,Lcap) */
#define HHR_DEV_TIMEOUT 0x4u      /* reserved: no kernel of this version waits for
                                     another workgroup (hand-offs between workgroups
                                     go to whichever arrives last), so it is never set */

typedef enum { HHR_F32 = 0, HHR_BF16 = 1 } hhr_dtype;

/* Shape of one attention layer's KV cache and its retrieval metadata.
 * Supported: head_dim == 128, code_bits 64, 128 or 256 (Table 4 of [HHR]
 * uses 128; appendix Figure 10 of [HHR] varies the number of hash bits),
 * page_size == 16, max_ctx a multiple of 16 in [16, 262144],
 * n_q_heads a multiple of n_kv_heads with G = n_q_heads / n_kv_heads <= 16,
 * batch * n_kv_heads <= 65535.
 * Selection limits (the entry points taking keep and top_k parameters return
 * HHR_ERR_UNSUPPORTED beyond them, and hhr_workspace_size returns 0):
 *   - candidates per (b, g): p_max * 16 <= 32768, where p_max =
 *     hhr_keep_count(max_ctx / 16, keep_num, keep_den, keep_pages_abs) is the
 *     kept-page count of a full cache (so max_ctx 262144 allows keeping at most
 *     1/8 of the pages, max_ctx 32768 all of them);
 *   - 1 <= top_k <= 32768. */
typedef struct {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t code_bits;
  int32_t page_size;
  int32_t max_ctx;
  int32_t kv_dtype;   /* hhr_dtype of the K and V caches */
  int32_t meta_dtype; /* hhr_dtype of the page metadata (the page_meta layout below) */
} hhr_shape;

/* Page metadata layout, by meta_dtype (d = head_dim, NpCap = max_ctx / page_size):
 *   HHR_F32  : [B][Hkv][NpCap][d][2] f32, {min, max} of each rotated key dimension
 *              over the page's valid rows;
 *   HHR_BF16 : [B][Hkv][NpCap][d] uint32, the same {min, max} as bfloat16 bit patterns
 *              (min in bits 0..15, max in bits 16..31), the min rounded toward -inf and
 *              the max toward +inf from the f32 values, so the page bound computed from
 *              them is never below the one from f32 metadata (it is looser by at most one
 *              bfloat16 step per dimension) and the metadata is half the bytes.  The
 *              storage precision of the GKR bounds [HHR abstract, GKR] is not fixed
 *              by the method; this is a compressed form of them. */

/* Text for a status code (static storage). */
const char* hhr_status_string(int32_t status);
/* Detail of the last non-OK return on this host thread (thread-local storage). */
const char* hhr_last_error(void);
/* ABI version: bumped on any change to a declaration in this header. */
int32_t hhr_abi_version(void);

/* Number of kept pages for a sequence of n_pages pages:
 *   keep_pages_abs > 0 : min(n_pages, keep_pages_abs)
 *   otherwise          : min(n_pages, max(1, ceil(keep_num * n_pages / keep_den)))
 * and 0 when n_pages == 0.  Pure host function.  [HHR abstract: page pruning] */
int32_t hhr_keep_count(int32_t n_pages, int32_t keep_num, int32_t keep_den,
                       int32_t keep_pages_abs);

/* Bytes of device workspace hhr_select / hhr_decode need for this shape and
 * these selection parameters; 0 if the arguments are invalid.  Pure host. */
size_t hhr_workspace_size(const hhr_shape* shape, int32_t keep_num, int32_t keep_den,
                          int32_t keep_pages_abs, int32_t top_k);

/* Synchronise `stream`, copy the workspace status word to *flags (host) and
 * clear it on the device.  Blocking. */
hhr_status hhr_read_device_status(void* workspace, void* stream, uint32_t* flags);

/* ------------------------------------------------------------ S1: append */
/* Encode key rows [start[b], start[b] + n_new[b]) of every KV head, which the
 * caller has already written into k_cache, and refresh the metadata of every
 * page those rows touch.                              [HHR abstract: GKR, LHP]
 *   k_cache   [B][Hkv][Lcap][d]           kv_dtype (f32 or bf16)
 *   start     [B] int32                   first new row of each sequence
 *   n_new     [B] int32                   rows appended (0 allowed)
 *   max_new   host int                    >= max_b n_new[b]; sizes the grid
 *   R         [Hkv][d][d] f32             head-wise orthogonal rotation
 *   W         [Hkv][d][code_bits] f32     head-wise hash projection
 *   codes     [B][Hkv][Lcap][nw] uint32   out: bit j of a key's code is
 *             [ (k W)_j >= 0 ], stored in word j/32 at bit j%32; written for
 *             the new rows only
 *   page_meta page metadata, meta_dtype layout   out: {min, max} over the valid rows
 *             (rows < start+n_new) of each touched page of X = k R
 * Rows of a touched page below start are read from k_cache (already present).
 * The products run on MFMA with bf16 hi/lo splits of R, W (and of f32 keys),
 * so each projected value is within ~2^-16 * sum_d |k_d M_dj| of exact.
 * Device errors: start < 0 or start + n_new > Lcap sets HHR_DEV_BAD_SEQ_LEN
 * in `status_word` (may be NULL: then such sequences are skipped silently). */
hhr_status hhr_append_keys(const hhr_shape* shape, const void* k_cache, const int32_t* start,
                           const int32_t* n_new, int32_t max_new, const float* R,
                           const float* W, uint32_t* codes, void* page_meta,
                           uint32_t* status_word, void* stream);

/* ------------------------------------------------------------ S2: query  */
/* q_rot[b][h] = q[b][h] R_g(h) and q_codes[b][h] = sign bits of q[b][h] W_g(h),
 * with g(h) = h / G.                                         [HHR abstract]
 *   q        [B][Hq][d] f32
 *   q_rot    [B][Hq][d] f32            out
 *   q_codes  [B][Hq][nw] uint32        out (same packing as the key codes) */
hhr_status hhr_encode_queries(const hhr_shape* shape, const float* q, const float* R,
                              const float* W, float* q_rot, uint32_t* q_codes, void* stream);

/* ------------------------------------------------------------ S3: bound  */
/* Page logit bound summed over the group's query heads:
 *   scores[b][g][p] = sum_{h in g} sum_d max(q'_hd mn_pd, q'_hd mx_pd)
 * for p < ceil(seq_len[b] / ps); entries beyond are left untouched.
 *                                    [HHR abstract: page-level logit bounds]
 *   q_rot     [B][Hq][d] f32       from hhr_encode_queries
 *   seq_len   [B] int32
 *   page_meta page metadata in the meta_dtype layout
 *   scores    [B][Hkv][NpCap] f32  out
 *   status_word: device uint32 or NULL (HHR_DEV_BAD_SEQ_LEN) */
hhr_status hhr_page_scores(const hhr_shape* shape, const float* q_rot, const int32_t* seq_len,
                           const void* page_meta, float* scores, uint32_t* status_word,
                           void* stream);

/* ------------------------------------------------------------ S4: prune  */
/* Keep the P = hhr_keep_count(Np_b, ...) pages with the largest score, ties
 * to the lower page index; write them ascending.   [HHR abstract: pruning]
 *   scores     [B][Hkv][NpCap] f32
 *   seq_len    [B] int32
 *   kept       [B][Hkv][p_max] int32  out, ascending, -1 padded;
 *              p_max = hhr_keep_count(NpCap, keep_num, keep_den, keep_pages_abs)
 *   kept_count [B][Hkv] int32         out */
hhr_status hhr_top_pages(const hhr_shape* shape, const float* scores, const int32_t* seq_len,
                         int32_t keep_num, int32_t keep_den, int32_t keep_pages_abs,
                         int32_t* kept, int32_t* kept_count, uint32_t* status_word,
                         void* stream);

/* ------------------------------------------------------- S5+S6: fine top-k */
/* Among the valid keys t < seq_len[b] of the kept pages, select the top_k
 * with the smallest (H(t), t), H(t) = sum_{h in g} popcount(q_codes[h] ^
 * codes[t]); write their positions ascending.  [HHR abstract: LHP; HATA]
 *   q_codes    [B][Hq][nw] uint32
 *   codes      [B][Hkv][Lcap][nw] uint32
 *   kept, kept_count, p_max  as written by hhr_top_pages
 *   sel_idx    [B][Hkv][top_k] int32  out, ascending, -1 padded
 *   sel_count  [B][Hkv] int32         out: min(top_k, #valid candidates)
 *   dist       [B][Hkv][p_max*ps] uint16, out, or NULL: H of candidate
 *              i = (kept slot i/ps, row i%ps); 0xFFFF for rows >= seq_len
 *   workspace  >= hhr_workspace_size(...) bytes for the keep parameters that
 *              gave p_max (an H histogram per (b, g), zero between calls, and
 *              scratch for the distances when dist is NULL);
 *              HHR_ERR_WORKSPACE if smaller */
hhr_status hhr_hamming_topk(const hhr_shape* shape, const uint32_t* q_codes,
                            const uint32_t* codes, const int32_t* seq_len, const int32_t* kept,
                            const int32_t* kept_count, int32_t p_max, int32_t top_k,
                            int32_t* sel_idx, int32_t* sel_count, uint16_t* dist,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------ S7: attend */
/* o[b][h] = sum_i softmax_i(q[b][h] . K[b][g][sel_i] * scale) V[b][g][sel_i]
 * over i < sel_count[b][g]; o = 0 when sel_count == 0.  fp32 arithmetic.
 *                                [HHR abstract: hash-based sparse attention]
 *   q          [B][Hq][d] f32
 *   k_cache, v_cache [B][Hkv][Lcap][d] kv_dtype
 *   sel_idx    [B][Hkv][top_k] int32, sel_count [B][Hkv] int32
 *   out        [B][Hq][d] f32  out
 *   workspace  >= hhr_workspace_size(...) bytes (split-K partials) */
hhr_status hhr_sparse_decode(const hhr_shape* shape, const float* q, const void* k_cache,
                             const void* v_cache, const int32_t* sel_idx,
                             const int32_t* sel_count, int32_t top_k, float scale, float* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------- S2..S4: page selection */
/* hhr_select_pages: the coarse stage alone from raw queries, in one launch:
 * rotate the group's queries (S2), bound every page (S3), keep the top P
 * (S4).                                      [HHR abstract: GKR, pruning]
 *   q, seq_len, R, W, page_meta  as for hhr_select
 *   kept, kept_count  out, exactly as hhr_top_pages writes them from the
 *              bounds that hhr_page_scores computes (bit-identical bounds)
 *   q_codes    [B][Hq][nw] uint32 out (as hhr_encode_queries writes them), or
 *              NULL (then kept in the workspace only)
 *   workspace  >= hhr_workspace_size(shape, keep_num, keep_den,
 *              keep_pages_abs, 1) bytes; the bounds stay in it */
hhr_status hhr_select_pages(const hhr_shape* shape, const float* q, const int32_t* seq_len,
                            const float* R, const float* W, const void* page_meta,
                            int32_t keep_num, int32_t keep_den, int32_t keep_pages_abs,
                            int32_t* kept, int32_t* kept_count, uint32_t* q_codes,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------- S2..S6 and S2..S7 */
/* hhr_select: S2..S6 in one stream-ordered call, the coarse-to-fine
 * retrieval of [HHR abstract] (GKR page bounds prune the pages, then LHP
 * codes rank the keys of the surviving pages by Hamming distance; [HHR]
 * Figure 1 orders the stages coarse then fine; [HATA abstract]: the codes
 * need only order q.k, which a top-k needs).  Intermediates live in the
 * workspace.  Outputs sel_idx / sel_count as in hhr_hamming_topk.  The
 * coarse stage is one launch when it fits (at most 2 x 256 scoring
 * workgroups of 256 pages, 128-bit codes), else separate launches; the fine
 * stage is a distance launch and one selection workgroup per (b, g).  Same
 * results either way. */
hhr_status hhr_select(const hhr_shape* shape, const float* q, const int32_t* seq_len,
                      const float* R, const float* W, const uint32_t* codes,
                      const void* page_meta, int32_t keep_num, int32_t keep_den,
                      int32_t keep_pages_abs, int32_t top_k, int32_t* sel_idx,
                      int32_t* sel_count, void* workspace, size_t workspace_bytes,
                      void* stream);

/* hhr_decode: one decode step, S2..S7: select as hhr_select, then attend
 * over only the selected keys ([HHR abstract]: hash-based sparse attention,
 * with the exact q.k logits; the codes only select) with softmax scale
 * `scale` (1/sqrt(128) for the usual scaling).  sel_idx / sel_count receive
 * the selection; out receives o.  Arguments and limits as for hhr_select and
 * hhr_sparse_decode; the workspace is hhr_workspace_size(shape, keep_num,
 * keep_den, keep_pages_abs, top_k) bytes. */
hhr_status hhr_decode(const hhr_shape* shape, const float* q, const int32_t* seq_len,
                      const float* R, const float* W, const uint32_t* codes,
                      const void* page_meta, const void* k_cache, const void* v_cache,
                      int32_t keep_num, int32_t keep_den, int32_t keep_pages_abs, int32_t top_k,
                      float scale, int32_t* sel_idx, int32_t* sel_count, float* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* hhr_decode_append: the decode step of a sequence that has just appended one
 * token (S1 for that token, then S2..S7), in the same launches as hhr_decode.
 * Row seq_len[b] - 1 of every sequence with seq_len[b] >= 1 is the new key:
 * the caller has written its K row into k_cache (and its V row into v_cache);
 * rows [0, seq_len[b] - 1) must have been encoded before (hhr_append_keys or an
 * earlier step).  The call writes the new row's code into `codes` and folds its
 * rotated key into its page's metadata in `page_meta` (or starts the page with
 * it), exactly what hhr_append_keys with start = seq_len - 1, n_new = 1 stores up
 * to rounding: the new row's rotation and projection are f32 sums (not the
 * encoder's bf16-split MFMA products), within about 2^-19 of the exact value
 * relative to sum_d |k_d M_dj|.  Then it selects and attends as hhr_decode over all
 * seq_len[b] keys.                     [HHR abstract: GKR, LHP; decode step]
 * Arguments as for hhr_decode; codes and page_meta are read and written. */
hhr_status hhr_decode_append(const hhr_shape* shape, const float* q, const int32_t* seq_len,
                             const float* R, const float* W, uint32_t* codes, void* page_meta,
                             const void* k_cache, const void* v_cache, int32_t keep_num,
                             int32_t keep_den, int32_t keep_pages_abs, int32_t top_k,
                             float scale, int32_t* sel_idx, int32_t* sel_count, float* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* hhr_decode_no_alloc: hhr_decode without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Its scratch is a static device
 * array of the library, hhr_no_alloc_scratch_bytes() bytes (64 MiB) on every
 * GPU it runs on, held until the process ends; the call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine).  It clears the
 * scratch's control block with a small kernel, then runs exactly the kernels
 * of hhr_decode, so its outputs equal hhr_decode's bit for bit.
 *   Arguments as for hhr_decode, without workspace / workspace_bytes;
 *   status_word  device uint32 or NULL: device error bits (HHR_DEV_*) are
 *                OR-ed into it (the caller clears it); with NULL they are
 *                dropped.
 * Returns HHR_ERR_UNSUPPORTED when the shape's workspace
 * (hhr_workspace_size) exceeds the static scratch.  Every call on one GPU
 * uses the same scratch: calls that overlap in time on one GPU (other
 * streams, other host threads) race and must not be issued.  The first call
 * on each device looks up the scratch's address (hipGetSymbolAddress), so
 * make it outside stream capture. */
hhr_status hhr_decode_no_alloc(const hhr_shape* shape, const float* q, const int32_t* seq_len,
                               const float* R, const float* W, const uint32_t* codes,
                               const void* page_meta, const void* k_cache, const void* v_cache,
                               int32_t keep_num, int32_t keep_den, int32_t keep_pages_abs,
                               int32_t top_k, float scale, int32_t* sel_idx, int32_t* sel_count,
                               float* out, uint32_t* status_word, void* stream);
/* Bytes of the static scratch behind hhr_decode_no_alloc.  Pure host. */
size_t hhr_no_alloc_scratch_bytes(void);

/* ================================================================ HISA  */
/* Shape of a HISA indexer: per query, n_index_heads fp8 index heads of
 * head_dim 128 scored against one fp8 index key per past token; blocks of
 * `block` tokens are pooled for the coarse stage.                  [HISA]
 * Supported: head_dim == 128, n_index_heads in [1, 64], block a multiple of
 * 16 in [16, 1024], max_ctx a multiple of block, max_ctx / block <= 16384,
 * max_ctx <= 2^24, batch <= 65535.  Selection limits (HHR_ERR_UNSUPPORTED
 * beyond them): keep_blocks * block <= 16384 candidates, 1 <= top_k <= 16384. */
typedef struct {
  int32_t batch;
  int32_t n_index_heads;
  int32_t head_dim;
  int32_t block;
  int32_t max_ctx;
} hhr_hisa_shape;

/* H1: refresh the pooled representative of every block touched by rows
 * [start[b], start[b] + n_new[b]):  reps[b][blk] = mean over the block's
 * valid rows of k_scale[t] * e4m3fn(k8[t]).       [HISA: pooled block reps]
 *   k8      [B][Lcap][d] uint8 (OCP fp8 e4m3fn),  k_scale [B][Lcap] f32 (> 0)
 *   reps    [B][Lcap/block][d] f32 out */
hhr_status hhr_hisa_pool_keys(const hhr_hisa_shape* shape, const uint8_t* k8,
                              const float* k_scale, const int32_t* start, const int32_t* n_new,
                              int32_t max_new, float* reps, uint32_t* status_word, void* stream);

/* H2: block_scores[b][blk] = sum_h w[b][h] * ReLU(qhat_h . reps[b][blk]),
 * qhat_h = q_scale[b][h] * e4m3fn(q8[b][h]), for blk < ceil(seq_len/block).
 *   q8 [B][Hi][d] uint8, q_scale [B][Hi] f32 (> 0), w [B][Hi] f32 (>= 0)
 *   block_scores [B][Lcap/block] f32 out                 [HISA: coarse filter] */
hhr_status hhr_hisa_block_scores(const hhr_hisa_shape* shape, const uint8_t* q8,
                                 const float* q_scale, const float* w, const float* reps,
                                 const int32_t* seq_len, float* block_scores,
                                 uint32_t* status_word, void* stream);

/* H3: keep the keep_blocks blocks with the largest score (ties: lower block),
 * ascending; kept_count = min(keep_blocks, #blocks).
 *   kept_blocks [B][keep_blocks] int32 out (-1 padded), kept_count [B] int32 out */
hhr_status hhr_hisa_top_blocks(const hhr_hisa_shape* shape, const float* block_scores,
                               const int32_t* seq_len, int32_t keep_blocks,
                               int32_t* kept_blocks, int32_t* kept_count,
                               uint32_t* status_word, void* stream);

/* H4+H5: token scores s_t = sum_h w_h ReLU(qhat_h . khat_t) for the valid
 * tokens of the kept blocks (fp8 MFMA, fp32 accumulate), then the exact
 * top_k by (larger s, lower t), ascending.  [HISA: token-level refinement]
 *   sel_idx [B][top_k] int32 out (-1 padded), sel_count [B] int32 out
 *   token_scores [B][keep_blocks*block] f32 out or NULL (-inf for rows >= seq_len)
 *   workspace >= hhr_hisa_workspace_size(...)
 * Up to 64 rows this is one launch: the last workgroup of a row to finish its
 * scores takes that row's top-k (arrival counters in the workspace, zero
 * between calls); with more rows a score launch, then a top-k launch.  Same
 * results either way. */
hhr_status hhr_hisa_token_topk(const hhr_hisa_shape* shape, const uint8_t* q8,
                               const float* q_scale, const float* w, const uint8_t* k8,
                               const float* k_scale, const int32_t* seq_len,
                               const int32_t* kept_blocks, const int32_t* kept_count,
                               int32_t keep_blocks, int32_t top_k, int32_t* sel_idx,
                               int32_t* sel_count, float* token_scores, void* workspace,
                               size_t workspace_bytes, void* stream);

size_t hhr_hisa_workspace_size(const hhr_hisa_shape* shape, int32_t keep_blocks, int32_t top_k);

/* H2..H5 in one stream-ordered call: the HISA selection of [HISA abstract]
 * (a block-level coarse filter over pooled representatives, then the
 * original indexer only on the tokens of the kept blocks, keeping an exact
 * token-level top-k among them).  seq_len [B] int32 in [0, max_ctx]; reps as
 * hhr_hisa_pool_keys writes them over the sequence's rows; outputs as
 * hhr_hisa_token_topk.  The selected positions then feed hhr_sparse_decode
 * with an hhr_shape of n_kv_heads = 1. */
hhr_status hhr_hisa_select(const hhr_hisa_shape* shape, const uint8_t* q8, const float* q_scale,
                           const float* w, const uint8_t* k8, const float* k_scale,
                           const float* reps, const int32_t* seq_len, int32_t keep_blocks,
                           int32_t top_k, int32_t* sel_idx, int32_t* sel_count, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Prefill indexer: H2..H5 for a chunk of query rows against ONE shared index-key
 * cache, each row over its own causal prefix (the O(L^2) per-layer case the
 * HISA abstract names).  Row r sees tokens t < q_len[r] (its position + 1), and
 * nothing after it, in both stages: the coarse filter scores the blocks
 * blk < ceil(q_len[r] / block), a block wholly inside the prefix with the shared
 * pooled representative (pooled once over the cache by hhr_hisa_pool_keys) and
 * the row's partly visible last block with the mean of its visible rows only
 * (computed by the call, the same arithmetic as hhr_hisa_pool_keys); the token
 * stage scores only tokens t < q_len[r].  So row r selects exactly what
 * hhr_hisa_select selects for a sequence of q_len[r] tokens whose
 * representatives were pooled over those tokens.             [HISA abstract]
 *   shape.batch = M query rows; max_ctx = the cache capacity
 *   q8 [M][Hi][d] uint8, q_scale [M][Hi] f32 (> 0), w [M][Hi] f32 (>= 0)
 *   k8 [Lcap][d] uint8, k_scale [Lcap] f32, reps [Lcap/block][d] f32 (shared)
 *   q_len [M] int32 in [0, Lcap]
 *   sel_idx [M][top_k] int32 out (ascending, -1 padded), sel_count [M] int32 out
 *   workspace >= hhr_hisa_workspace_size(shape, keep_blocks, top_k) (per row) */
hhr_status hhr_hisa_prefill_select(const hhr_hisa_shape* shape, const uint8_t* q8,
                                   const float* q_scale, const float* w, const uint8_t* k8,
                                   const float* k_scale, const float* reps,
                                   const int32_t* q_len, int32_t keep_blocks, int32_t top_k,
                                   int32_t* sel_idx, int32_t* sel_count, void* workspace,
                                   size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* HHR_H_ */
