// S7 sparse decode: softmax attention over only the selected K/V rows
// [HHR abstract: hash-based sparse attention], split over chunks of the
// selected set with an online-softmax (m, l, o) combine.
//
// k_attn: one workgroup takes a chunk of up to 64 selected keys of one (b, g)
// for all G query heads.  It gathers the chunk's K and V rows into LDS with
// every load in flight at once (row indices are clamped and the data masked,
// never branched on, so the loads are not serialised), computes logits, chunk
// softmax numerators and the unnormalised partial output from LDS, and writes
// (o~, m, l).  k_attn_combine: one workgroup per (b, query head, 32 output
// dims) merges the chunks' partials: o = sum_s e^(m_s - M) o~_s / sum_s
// e^(m_s - M) l_s with M = max_s m_s.

#include "hhr_device.h"
#include "hhr_internal.h"

namespace hhr {

namespace {

constexpr int kCh = kAttnChunk;       // 64 selected keys per workgroup
constexpr int kPartStride = kD + 2;   // o~[128], m, l
constexpr int kRowPad = 8;            // LDS row padding (bank spread), in elements

template <bool KF32>
struct RowT {
  typedef uint16_t T;
  static constexpr int kBytes = kD * 2;
};
template <>
struct RowT<true> {
  typedef float T;
  static constexpr int kBytes = kD * 4;
};

template <bool KF32>
__device__ __forceinline__ float lds_elem(const typename RowT<KF32>::T* row, int d) {
  if constexpr (KF32) return row[d];
  else return bf16_to_f32(row[d]);
}

template <bool KF32>
__global__ __launch_bounds__(256) void k_attn(
    const float* __restrict__ q, const void* __restrict__ kcache, const void* __restrict__ vcache,
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_count,
    float* __restrict__ part, uint32_t* __restrict__ status, int Hq, int Hkv, int Lcap,
    int top_k, int n_split, float scale) {
  typedef typename RowT<KF32>::T ET;
  constexpr int kStride = kD + kRowPad;
  constexpr int kVec = 16 / sizeof(ET);             // elements per 16-byte load
  constexpr int kChunksPerRow = kD / kVec;          // 16 (bf16) or 32 (f32)
  constexpr int kLoads = kCh * kChunksPerRow / 256; // per thread, per matrix: 4 or 8
  __shared__ __attribute__((aligned(16))) ET sk[kCh * kStride];
  __shared__ __attribute__((aligned(16))) ET sv[kCh * kStride];
  __shared__ float sq[kMaxG][kD];
  __shared__ float sp[kMaxG][kCh];
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

  const int cnt = max(0, min(sel_count[bg], top_k));
  const int k0 = sp_id * kCh;
  if (k0 >= cnt) return;
  const int nk = min(kCh, cnt - k0);

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
  for (int i = tid; i < G * kD; i += 256)
    sq[i / kD][i % kD] = q[((size_t)b * Hq + (size_t)g * G) * kD + i];
  __syncthreads();

  // gather: every thread issues all of its K and V loads before storing any
  {
    const ET* kb = (const ET*)kcache + (size_t)bg * Lcap * kD;
    const ET* vb = (const ET*)vcache + (size_t)bg * Lcap * kD;
    u32x4 kreg[kLoads], vreg[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + 256 * i;
      const int r = c / kChunksPerRow;
      const int cc = c % kChunksPerRow;
      const int idx = max(sidx[r], 0);
      kreg[i] = *(const u32x4*)(kb + (size_t)idx * kD + cc * kVec);
      vreg[i] = *(const u32x4*)(vb + (size_t)idx * kD + cc * kVec);
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int r = (tid + 256 * i) / kChunksPerRow;
      if (sidx[r] < 0) {
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
        vreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + 256 * i;
      const int r = c / kChunksPerRow;
      const int cc = c % kChunksPerRow;
      *(u32x4*)(sk + r * kStride + cc * kVec) = kreg[i];
      *(u32x4*)(sv + r * kStride + cc * kVec) = vreg[i];
    }
  }
  __syncthreads();

  // logits: thread (key = l, head group w) -> heads w, w+4, ...
  for (int h = w; h < G; h += 4) {
    const ET* row = sk + l * kStride;
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < kD / kVec; ++c) {
      const u32x4 v = *(const u32x4*)(row + c * kVec);
      if constexpr (KF32) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dot = fmaf(sq[h][4 * c + j], __uint_as_float(v[j]), dot);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dot = fmaf(sq[h][8 * c + 2 * j], bf16_to_f32(v[j] & 0xFFFFu), dot);
          dot = fmaf(sq[h][8 * c + 2 * j + 1], bf16_to_f32(v[j] >> 16), dot);
        }
      }
    }
    sp[h][l] = (l < nk && sidx[l] >= 0) ? dot * scale : -__builtin_huge_valf();
  }
  __syncthreads();

  // chunk softmax numerators: one wave per head, lane = key
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

  // partial o~_h[d] = sum_k p_h[k] V[k][d]: lane owns dims {2l, 2l+1}, wave w heads w, w+4, ...
  float* pout = part + ((size_t)bg * n_split + sp_id) * kMaxG * kPartStride;
  for (int h = w; h < G; h += 4) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll 8
    for (int k = 0; k < kCh; ++k) {
      const float p = sp[h][k];
      const ET* row = sv + k * kStride;
      a0 = fmaf(p, lds_elem<KF32>(row, 2 * l), a0);
      a1 = fmaf(p, lds_elem<KF32>(row, 2 * l + 1), a1);
    }
    *(float2*)(pout + h * kPartStride + 2 * l) = make_float2(a0, a1);
    if (l == 0) {
      pout[h * kPartStride + kD] = sm[h];
      pout[h * kPartStride + kD + 1] = sl[h];
    }
  }

}

// One workgroup per (b, query head, 32-dim slice): thread t takes chunk slot
// t/8 (32 chunks per pass) and dims 4*(t%8) .. +3 of the slice.
constexpr int kCombDims = 32;

__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ part,
                                                      const int32_t* __restrict__ sel_count,
                                                      float* __restrict__ out, int Hq, int Hkv,
                                                      int top_k, int n_split) {
  __shared__ float sM[4];
  __shared__ floatx4 red[32][kCombDims / 4];
  __shared__ float redl[32];
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int h = bh % Hq;
  const int G = Hq / Hkv;
  const int g = h / G;
  const int j = h % G;
  const int bg = b * Hkv + g;
  const int d0 = blockIdx.y * kCombDims;
  const int tid = threadIdx.x;
  const int cnt = max(0, min(sel_count[bg], top_k));
  const int ns = (cnt + kCh - 1) / kCh;
  const size_t sstride = (size_t)kMaxG * kPartStride;
  const float* p = part + (size_t)bg * n_split * sstride + j * kPartStride;
  // M = max over chunks of m_s (all m_s loaded at once)
  float M = -__builtin_huge_valf();
  for (int s = tid; s < ns; s += 256) M = fmaxf(M, p[(size_t)s * sstride + kD]);
  M = wave_max(M);
  if ((tid & 63) == 0) sM[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(sM[0], sM[1]), fmaxf(sM[2], sM[3]));
  const int slot = tid >> 3;
  const int q4 = tid & 7;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  float lacc = 0.f;
  if (cnt > 0 && M != -__builtin_huge_valf()) {
    for (int s0 = 0; s0 < ns; s0 += 64) {
      // two chunk slots per thread per round, loads issued together
      const int sa = min(s0 + slot, ns - 1), sb = min(s0 + 32 + slot, ns - 1);
      const float* pa = p + (size_t)sa * sstride;
      const float* pbp = p + (size_t)sb * sstride;
      const float ma = pa[kD], la = pa[kD + 1];
      const float mb = pbp[kD], lb = pbp[kD + 1];
      const floatx4 oa = *(const floatx4*)(pa + d0 + 4 * q4);
      const floatx4 ob = *(const floatx4*)(pbp + d0 + 4 * q4);
      const float fa = (s0 + slot < ns && ma != -__builtin_huge_valf()) ? expf(ma - M) : 0.f;
      const float fb = (s0 + 32 + slot < ns && mb != -__builtin_huge_valf()) ? expf(mb - M) : 0.f;
      lacc = fmaf(fa, la, lacc);
      lacc = fmaf(fb, lb, lacc);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = fmaf(fb, ob[k], fmaf(fa, oa[k], acc[k]));
    }
  }
  red[slot][q4] = acc;
  if (q4 == 0) redl[slot] = lacc;
  __syncthreads();
  if (tid < kCombDims) {
    const int qd = tid >> 2, k = tid & 3;
    float o = 0.f, lsum = 0.f;
    for (int s = 0; s < 32; ++s) {
      o += red[s][qd][k];
      lsum += redl[s];
    }
    out[(size_t)bh * kD + d0 + tid] = (cnt > 0 && lsum > 0.f) ? o / lsum : 0.f;
  }
}

}  // namespace

hipError_t launch_sparse_decode(const hhr_shape& s, const float* q, const void* k_cache,
                                const void* v_cache, const int32_t* sel_idx,
                                const int32_t* sel_count, int32_t top_k, float scale, float* out,
                                float* part, int32_t n_split, uint32_t* status,
                                hipStream_t stream) {
  dim3 grid(n_split, s.batch * s.n_kv_heads);
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
  hipLaunchKernelGGL(k_attn_combine, dim3(s.batch * s.n_q_heads, kD / kCombDims), dim3(256), 0,
                     stream, part, sel_count, out, s.n_q_heads, s.n_kv_heads, top_k, n_split);
  return hipGetLastError();
}

}  // namespace hhr
