// Decode plan and the VALU split-KV decode (fp32 caches, and any n_h).
//
// Plan: exclusive prefix sum of the clamped sequence lengths; the decode and
// combine kernels derive their work split from it (split_begin / split_of).
// It also records, for every split, the sequence holding its first token and
// that sequence's global token range, so a decode workgroup starts without a
// search.
//
// VALU decode: the same computation as the MFMA kernel ("DeepSeek-V2：在“大力出
// 奇迹”的AI军备竞赛中，四两拨千斤", liang.world, ch.2 §1 per-head softmax
// attention, §2 absorbed W^UK, §3 score = q^C.k^C + q^R.k^R) written plainly:
// per segment and head, 256 tokens at a time, one thread per token for the
// 576-long score and one thread per latent column for O~.  It keeps the
// fp32 config at fp32 precision end to end and serves head counts the MFMA
// kernel is not built for.
#include "mla_common.h"

namespace mla {
namespace {

__global__ void __launch_bounds__(1024) plan_kernel(PlanArgs pa) {
  __shared__ int32_t part[1024 + 8192];
  plan_block<1024>(pa, part, 8192);
}

template <typename T>
__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = fmaxf(r, red[i]);
  return r;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r += red[i];
  return r;
}

template <typename T>
__global__ void __launch_bounds__(256) decode_simple_kernel(
    int32_t n_h, const T* __restrict__ qabs, const T* __restrict__ c_KV, const T* __restrict__ k_R,
    int64_t row_stride, int32_t num_pages, const int32_t* __restrict__ page_table, int32_t max_pages,
    int32_t page_size, const int32_t* __restrict__ prefix, int32_t B, int32_t G, float* __restrict__ part_ml,
    T* __restrict__ part_o, int32_t* __restrict__ flags) {
  __shared__ float qs[D_K];
  __shared__ float ps[256];
  __shared__ int64_t rows[256];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int64_t N = prefix[B];
  const int64_t P0 = split_begin(blockIdx.x, N, G), P1 = split_begin(blockIdx.x + 1, N, G);
  if (P0 >= P1) return;
  for (int b = seq_of(prefix, B, P0); b < B && prefix[b] < P1; ++b) {
    const int64_t s0 = max((int64_t)prefix[b], P0), s1 = min((int64_t)prefix[b + 1], P1);
    if (s0 >= s1) continue;
    const int32_t t0 = (int32_t)(s0 - prefix[b]), t1 = (int32_t)(s1 - prefix[b]);
    const int64_t slot = (int64_t)blockIdx.x + b;
    for (int h = 0; h < n_h; ++h) {
      __syncthreads();
      for (int k = tid; k < D_K; k += 256) qs[k] = to_f32(qabs[(int64_t)b * n_h * D_K + qabs_offset(n_h, sizeof(T) == 2, h, k)]);
      __syncthreads();
      float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
      for (int cs = t0; cs < t1; cs += 256) {
        const int t = cs + tid;
        float s = -INFINITY;
        int64_t row = 0;
        if (t < t1) {
          row = pool_row(page_table, max_pages, num_pages, page_size, b, t, flags);
          const T* c = c_KV + row * row_stride;
          const T* r = k_R + row * row_stride;
          float acc = 0.f;
          for (int k = 0; k < D_C; ++k) acc = fmaf(qs[k], to_f32(c[k]), acc);
          for (int k = 0; k < D_R; ++k) acc = fmaf(qs[D_C + k], to_f32(r[k]), acc);
          s = acc;
        }
        const float mc = block_max<T>(s, red);
        const float m_new = fmaxf(m, mc);
        const float alpha = m == -INFINITY ? 0.f : exp2f(m - m_new);
        const float p = t < t1 ? exp2f(s - m_new) : 0.f;
        ps[tid] = p;
        rows[tid] = row;
        const float sc = block_sum(p, red);
        l = l * alpha + sc;
        o0 *= alpha;
        o1 *= alpha;
        const int cnt = min(256, t1 - cs);
        for (int j = 0; j < cnt; ++j) {
          const T* c = c_KV + rows[j] * row_stride;
          o0 = fmaf(ps[j], to_f32(c[tid]), o0);
          o1 = fmaf(ps[j], to_f32(c[tid + 256]), o1);
        }
        m = m_new;
      }
      T* dst = part_o + (slot * n_h + h) * D_C;
      dst[tid] = from_f32<T>(o0);
      dst[tid + 256] = from_f32<T>(o1);
      if (tid == 0) {
        part_ml[(slot * n_h + h) * 2 + 0] = m;
        part_ml[(slot * n_h + h) * 2 + 1] = l;
      }
    }
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& pa, hipStream_t s) {
  plan_kernel<<<1, 1024, 0, s>>>(pa);
  return hipGetLastError();
}

hipError_t launch_decode_simple(const mla_dims& d, int32_t B, const void* qabs, const void* c_KV,
                                const void* k_R, int64_t row_stride, int32_t num_pages,
                                const int32_t* page_table, int32_t max_pages, const int32_t* prefix,
                                int32_t n_splits, float* part_ml, void* part_o, int32_t* flags,
                                hipStream_t s) {
  if (d.dtype == MLA_FP32)
    decode_simple_kernel<float><<<n_splits, 256, 0, s>>>(d.n_h, (const float*)qabs, (const float*)c_KV,
                                                         (const float*)k_R, row_stride, num_pages, page_table,
                                                         max_pages, d.page_size, prefix, B, n_splits, part_ml,
                                                         (float*)part_o, flags);
  else
    decode_simple_kernel<bf16><<<n_splits, 256, 0, s>>>(d.n_h, (const bf16*)qabs, (const bf16*)c_KV,
                                                        (const bf16*)k_R, row_stride, num_pages, page_table,
                                                        max_pages, d.page_size, prefix, B, n_splits, part_ml,
                                                        (bf16*)part_o, flags);
  return hipGetLastError();
}

}  // namespace mla
