// S7 sparse decode: softmax attention over only the selected K/V rows
// [HHR abstract: hash-based sparse attention], split over chunks of the
// selected set with an online-softmax (m, l, o) combine.

#include "hhr_device.h"
#include "hhr_internal.h"

namespace hhr {

namespace {

constexpr int kCh = kAttnChunk;  // 64 selected keys per workgroup
constexpr int kPartStride = kD + 2;  // o[128], m, l

template <bool KF32>
__device__ __forceinline__ void load_row8(const void* base, size_t row, int d0, float* out) {
  if constexpr (KF32) {
    const floatx4 a = *(const floatx4*)((const float*)base + row * kD + d0);
    const floatx4 c = *(const floatx4*)((const float*)base + row * kD + d0 + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[j] = a[j];
      out[4 + j] = c[j];
    }
  } else {
    const u32x4 v = *(const u32x4*)((const uint16_t*)base + row * kD + d0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[2 * j] = bf16_to_f32(v[j] & 0xFFFFu);
      out[2 * j + 1] = bf16_to_f32(v[j] >> 16);
    }
  }
}

template <bool KF32>
__device__ __forceinline__ float2 load_row2(const void* base, size_t row, int d0) {
  if constexpr (KF32) {
    return *(const float2*)((const float*)base + row * kD + d0);
  } else {
    const uint32_t v = *(const uint32_t*)((const uint16_t*)base + row * kD + d0);
    return make_float2(bf16_to_f32(v & 0xFFFFu), bf16_to_f32(v >> 16));
  }
}

// One workgroup = one chunk of up to 64 selected keys of one (b, g), all G
// query heads.  Writes unnormalised partials o~ = sum_i exp(x_i - m) V_i,
// m = max_i x_i, l = sum_i exp(x_i - m) for each head.
template <bool KF32>
__global__ __launch_bounds__(256) void k_attn_partial(
    const float* __restrict__ q, const void* __restrict__ kcache, const void* __restrict__ vcache,
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_count,
    float* __restrict__ part, uint32_t* __restrict__ status, int Hq, int Hkv, int Lcap,
    int top_k, int n_split, float scale) {
  __shared__ float sq[kMaxG][kD];
  __shared__ float sp[kMaxG][kCh];
  __shared__ float red[4][kMaxG][kD];
  __shared__ int sidx[kCh];
  __shared__ float sm[kMaxG], sl[kMaxG];

  const int bg = blockIdx.y;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  const int G = Hq / Hkv;
  const int sp_id = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  float* pout = part + ((size_t)bg * n_split + sp_id) * kMaxG * kPartStride;

  const int cnt = min(sel_count[bg], top_k);
  const int k0 = sp_id * kCh;
  if (k0 >= cnt) {
    if (tid < G) {
      pout[tid * kPartStride + kD] = -__builtin_huge_valf();
      pout[tid * kPartStride + kD + 1] = 0.f;
    }
    return;
  }
  const int nk = min(kCh, cnt - k0);

  for (int i = tid; i < G * kD; i += 256)
    sq[i / kD][i % kD] = q[((size_t)b * Hq + (size_t)g * G) * kD + i];
  if (tid < kCh) {
    int idx = -1;
    if (tid < nk) {
      idx = sel_idx[(size_t)bg * top_k + k0 + tid];
      if (idx < 0 || idx >= Lcap) {
        if (status) atomicOr(status, HHR_DEV_BAD_INDEX);
        idx = -1;
      }
    }
    sidx[tid] = idx;
  }
  __syncthreads();

  const size_t row_base = (size_t)bg * Lcap;
  // logits: 16 lanes per key (8 dims each), 4 keys per wave, 16 keys per pass
  {
    const int sub = l & 15;
    const int kk = l >> 4;
    for (int it = 0; it < kCh / 16; ++it) {
      const int key = it * 16 + w * 4 + kk;
      const int idx = key < nk ? sidx[key] : -1;
      float kv[8];
      if (idx >= 0) load_row8<KF32>(kcache, row_base + idx, 8 * sub, kv);
      else
#pragma unroll
        for (int j = 0; j < 8; ++j) kv[j] = 0.f;
      for (int h = 0; h < G; ++h) {
        float dot = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) dot = fmaf(sq[h][8 * sub + j], kv[j], dot);
        dot += __shfl_xor(dot, 8);
        dot += __shfl_xor(dot, 4);
        dot += __shfl_xor(dot, 2);
        dot += __shfl_xor(dot, 1);
        if (sub == 0) sp[h][key] = idx >= 0 ? dot * scale : -__builtin_huge_valf();
      }
    }
  }
  __syncthreads();

  // softmax numerators per head (one wave per head, lane = key)
  for (int h = w; h < G; h += 4) {
    const float x = sp[h][l];
    const float m = wave_max(x);
    const float p = (x == -__builtin_huge_valf()) ? 0.f : expf(x - m);
    const float s = wave_sum(p);
    sp[h][l] = p;
    if (l == 0) {
      sm[h] = m;
      sl[h] = s;
    }
  }
  __syncthreads();

  // o~_h[d] = sum_k p_h[k] V[k][d]; lane owns dims {2l, 2l+1}, wave w takes keys w, w+4, ...
  float acc[kMaxG][2];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) acc[h][0] = acc[h][1] = 0.f;
  for (int key = w; key < nk; key += 4) {
    const int idx = sidx[key];
    if (idx < 0) continue;
    const float2 v = load_row2<KF32>(vcache, row_base + idx, 2 * l);
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      if (h < G) {
        const float p = sp[h][key];
        acc[h][0] = fmaf(p, v.x, acc[h][0]);
        acc[h][1] = fmaf(p, v.y, acc[h][1]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    if (h < G) {
      red[w][h][2 * l] = acc[h][0];
      red[w][h][2 * l + 1] = acc[h][1];
    }
  }
  __syncthreads();
  for (int i = tid; i < G * kD; i += 256) {
    const int h = i / kD, d = i % kD;
    pout[h * kPartStride + d] = (red[0][h][d] + red[1][h][d]) + (red[2][h][d] + red[3][h][d]);
  }
  if (tid < G) {
    pout[tid * kPartStride + kD] = sm[tid];
    pout[tid * kPartStride + kD + 1] = sl[tid];
  }
}

// One workgroup per (b, query head): o = sum_s exp(m_s - M) o~_s / sum_s exp(m_s - M) l_s.
__global__ __launch_bounds__(kD) void k_attn_combine(const float* __restrict__ part,
                                                     const int32_t* __restrict__ sel_count,
                                                     float* __restrict__ out, int Hq, int Hkv,
                                                     int top_k, int n_split) {
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int h = bh % Hq;
  const int G = Hq / Hkv;
  const int g = h / G;
  const int j = h % G;
  const int bg = b * Hkv + g;
  const int d = threadIdx.x;
  const int cnt = min(sel_count[bg], top_k);
  const int ns = (cnt + kCh - 1) / kCh;
  const float* p = part + (size_t)bg * n_split * kMaxG * kPartStride + j * kPartStride;
  float M = -__builtin_huge_valf();
  for (int s = 0; s < ns; ++s) M = fmaxf(M, p[(size_t)s * kMaxG * kPartStride + kD]);
  float o = 0.f, lsum = 0.f;
  if (cnt > 0 && M != -__builtin_huge_valf()) {
    for (int s = 0; s < ns; ++s) {
      const float* ps = p + (size_t)s * kMaxG * kPartStride;
      const float ms = ps[kD];
      if (ms == -__builtin_huge_valf()) continue;
      const float f = expf(ms - M);
      lsum = fmaf(f, ps[kD + 1], lsum);
      o = fmaf(f, ps[d], o);
    }
    o = o / lsum;
  }
  out[(size_t)bh * kD + d] = o;
}

}  // namespace

hipError_t launch_sparse_decode(const hhr_shape& s, const float* q, const void* k_cache,
                                const void* v_cache, const int32_t* sel_idx,
                                const int32_t* sel_count, int32_t top_k, float scale, float* out,
                                float* part, int32_t n_split, uint32_t* status,
                                hipStream_t stream) {
  dim3 grid(n_split, s.batch * s.n_kv_heads);
  if (s.kv_dtype == HHR_F32)
    hipLaunchKernelGGL(k_attn_partial<true>, grid, dim3(256), 0, stream, q, k_cache, v_cache,
                       sel_idx, sel_count, part, status, s.n_q_heads, s.n_kv_heads, s.max_ctx,
                       top_k, n_split, scale);
  else
    hipLaunchKernelGGL(k_attn_partial<false>, grid, dim3(256), 0, stream, q, k_cache, v_cache,
                       sel_idx, sel_count, part, status, s.n_q_heads, s.n_kv_heads, s.max_ctx,
                       top_k, n_split, scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_combine, dim3(s.batch * s.n_q_heads), dim3(kD), 0, stream, part,
                     sel_count, out, s.n_q_heads, s.n_kv_heads, top_k, n_split);
  return hipGetLastError();
}

}  // namespace hhr
