// S7 sparse decode: softmax attention over only the selected K/V rows
// [HHR abstract: hash-based sparse attention], split over 64-key chunks of the
// selected set with an online-softmax (m, l, o) combine.  k_attn runs one
// chunk per workgroup (attn_chunk), or, when a group has many query heads and
// the grid is small, one chunk for 4 of the heads per workgroup (grid.z picks
// the heads: the 64 rows are gathered once per head group, and each wave then
// attends one head instead of several); k_attn_combine merges one (b, g,
// query head) per workgroup of kCombThreads threads (attn_combine).

#include "hhr_device.h"
#include "hhr_internal.h"
#include "stages.h"

namespace hhr {

namespace {

template <bool KF32>
__global__ __launch_bounds__(256) void k_attn(
    const float* __restrict__ q, const void* __restrict__ kcache, const void* __restrict__ vcache,
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_count,
    float* __restrict__ part, uint32_t* __restrict__ status, int Hq, int Hkv, int Lcap,
    int top_k, int n_split, float scale) {
  __shared__ AttnSmem<KF32> sm;
  const int bg = blockIdx.y;
  const int cnt = max(0, min(sel_count[bg], top_k));
  const int k0 = blockIdx.x * kCh;
  if (k0 >= cnt) return;
  const int hper = (Hq / Hkv + gridDim.z - 1) / gridDim.z;  // query heads per workgroup
  const int h_lo = blockIdx.z * hper;
  attn_chunk<KF32, false>(bg / Hkv, bg % Hkv, Hq, Hkv, Lcap, top_k, k0, min(kCh, cnt - k0), scale,
                          q, kcache, vcache, sel_idx,
                          part + ((size_t)bg * n_split + blockIdx.x) * kMaxG * kPartStride, status,
                          sm, h_lo, h_lo + hper);
}

__global__ __launch_bounds__(kCombThreads) void k_attn_combine(
    const float* __restrict__ part, const int32_t* __restrict__ sel_count,
    float* __restrict__ out, int Hq, int Hkv, int top_k, int n_split) {
  __shared__ CombSmem sm;
  const int bg = blockIdx.y;
  const int cnt = max(0, min(sel_count[bg], top_k));
  attn_combine<false>(bg / Hkv, bg % Hkv, blockIdx.x, Hq, Hkv, (cnt + kCh - 1) / kCh, n_split,
                      part, out, sm);
}

}  // namespace

hipError_t launch_sparse_decode(const hhr_shape& s, const float* q, const void* k_cache,
                                const void* v_cache, const int32_t* sel_idx,
                                const int32_t* sel_count, int32_t top_k, float scale, float* out,
                                float* part, int32_t n_split, uint32_t* status,
                                hipStream_t stream) {
  // f32 caches with more than 4 query heads per KV head and fewer chunks than
  // CUs: split the heads over grid.z, 4 per workgroup (one per wave).  bf16
  // caches take all 16 head rows in each MFMA, so a split would only repeat
  // the chunk's gather.
  const int G = s.n_q_heads / s.n_kv_heads;
  const long long chunks = (long long)n_split * s.batch * s.n_kv_heads;
  const int hsplit =
      (s.kv_dtype == HHR_F32 && G > 4 && chunks < 256) ? (G + 3) / 4 : 1;
  dim3 grid(n_split, s.batch * s.n_kv_heads, hsplit);
  if (s.kv_dtype == HHR_F32)
    hipLaunchKernelGGL(k_attn<true>, grid, dim3(256), 0, stream, q, k_cache, v_cache, sel_idx,
                       sel_count, part, status, s.n_q_heads, s.n_kv_heads, s.max_ctx, top_k,
                       n_split, scale);
  else
    hipLaunchKernelGGL(k_attn<false>, grid, dim3(256), 0, stream, q, k_cache, v_cache, sel_idx,
                       sel_count, part, status, s.n_q_heads, s.n_kv_heads, s.max_ctx, top_k,
                       n_split, scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_combine, dim3(s.n_q_heads / s.n_kv_heads, s.batch * s.n_kv_heads),
                     dim3(kCombThreads), 0, stream, part, sel_count, out, s.n_q_heads,
                     s.n_kv_heads, top_k, n_split);
  return hipGetLastError();
}

}  // namespace hhr
