// Cross-split combine and W^UV epilogue.
//   Combine (log-sum-exp merge of the per-split softmax partials): with the
//   partials (m_s, l_s, O_s) of one (sequence, head) in log2 units,
//   m* = max m_s, L = sum_s 2^(m_s - m*) l_s, O~ = sum_s 2^(m_s - m*) O_s / L,
//   lse = (m* + log2 L) ln 2.  This is the per-head softmax of
//   "DeepSeek-V2：在“大力出奇迹”的AI军备竞赛中，四两拨千斤" (liang.world), ch.2 §1,
//   evaluated piecewise.
//   Epilogue: o_i = W^UV_i O~_i -- the value up-projection v^C_j = W^UV c_j
//   (ch.2 §2) applied once to the softmax-weighted latent, which is the
//   absorption of W^UV on the output side (ch.2 §2, absorption paragraph).
//
// Workgroup (head h, 32 sequences): the 32 combined latents go to LDS
// (fp32), then each thread computes one output column d for 16 sequences
// while W^UV_h is read once per workgroup (row d, contiguous over the latent).
#include "mla_common.h"

namespace mla {
namespace {

constexpr int CB_SEQ = 32;

template <typename T>
__global__ void __launch_bounds__(256) combine_kernel(int32_t B, int32_t n_h, const int32_t* __restrict__ prefix,
                                                      int32_t G, const float* __restrict__ part_ml,
                                                      const float* __restrict__ part_o, const T* __restrict__ W_UV,
                                                      float* __restrict__ out, float* __restrict__ lse) {
  __shared__ float ol[CB_SEQ][D_C + 4];
  __shared__ float mst[CB_SEQ];
  __shared__ int32_t wfirst[CB_SEQ], wcount[CB_SEQ];
  __shared__ float invL[CB_SEQ];
  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * CB_SEQ;
  const int nb = min(CB_SEQ, B - b0);
  const int64_t N = prefix[B];
  // per-sequence split range and merge weights (one thread per sequence)
  if (tid < nb) {
    const int b = b0 + tid;
    const int64_t sb = prefix[b], n = prefix[b + 1] - sb;
    if (n <= 0) {
      wfirst[tid] = 0;
      wcount[tid] = 0;
      invL[tid] = 0.f;
      mst[tid] = 0.f;
      if (lse) lse[(int64_t)b * n_h + h] = -INFINITY;
    } else {
      const int64_t w0 = split_of(sb, N, G), w1 = split_of(sb + n - 1, N, G);
      const int cnt = (int)(w1 - w0 + 1);
      float mstar = -INFINITY;
      for (int i = 0; i < cnt; ++i) mstar = fmaxf(mstar, part_ml[((w0 + i + b) * n_h + h) * 2]);
      float L = 0.f;
      for (int i = 0; i < cnt; ++i) {
        const float* ml = part_ml + ((w0 + i + b) * n_h + h) * 2;
        L += exp2f(ml[0] - mstar) * ml[1];
      }
      wfirst[tid] = (int32_t)w0;
      wcount[tid] = cnt;
      invL[tid] = 1.f / L;
      mst[tid] = mstar;
      if (lse) lse[(int64_t)b * n_h + h] = (mstar + log2f(L)) * 0.69314718055994531f;
    }
  }
  __syncthreads();
  for (int bb = 0; bb < nb; ++bb) {
    const int b = b0 + bb;
    const int cnt = wcount[bb];
    float a0 = 0.f, a1 = 0.f;
    for (int i = 0; i < cnt; ++i) {
      const int64_t slot = wfirst[bb] + i + b;
      const float* src = part_o + (slot * n_h + h) * D_C;
      const float wgt = exp2f(part_ml[(slot * n_h + h) * 2] - mst[bb]);
      a0 = fmaf(wgt, src[tid], a0);
      a1 = fmaf(wgt, src[tid + 256], a1);
    }
    ol[bb][tid] = a0 * invL[bb];
    ol[bb][tid + 256] = a1 * invL[bb];
  }
  __syncthreads();
  // o[b][h][d] = sum_c W^UV[h*128 + d][c] * O~[b][c]; thread -> (d, half of the sequences)
  const int d = tid & (D_H - 1), half = tid >> 7;
  const T* wr = W_UV + ((int64_t)h * D_H + d) * D_C;
  float acc[CB_SEQ / 2];
#pragma unroll
  for (int j = 0; j < CB_SEQ / 2; ++j) acc[j] = 0.f;
  for (int c = 0; c < D_C; c += 4) {
    const float w0 = to_f32(wr[c]), w1 = to_f32(wr[c + 1]), w2 = to_f32(wr[c + 2]), w3 = to_f32(wr[c + 3]);
#pragma unroll
    for (int j = 0; j < CB_SEQ / 2; ++j) {
      const float* ov = &ol[half * (CB_SEQ / 2) + j][c];
      acc[j] = fmaf(w0, ov[0], fmaf(w1, ov[1], fmaf(w2, ov[2], fmaf(w3, ov[3], acc[j]))));
    }
  }
#pragma unroll
  for (int j = 0; j < CB_SEQ / 2; ++j) {
    const int bb = half * (CB_SEQ / 2) + j;
    if (bb < nb) out[((int64_t)(b0 + bb) * n_h + h) * D_H + d] = wcount[bb] > 0 ? acc[j] : 0.f;
  }
}

}  // namespace

hipError_t launch_combine(const mla_dims& d, int32_t B, const int32_t* prefix, int32_t n_splits,
                          const float* part_ml, const float* part_o, const void* W_UV, float* out,
                          float* lse, hipStream_t s) {
  dim3 grid(d.n_h, (B + CB_SEQ - 1) / CB_SEQ);
  if (d.dtype == MLA_FP32)
    combine_kernel<float><<<grid, 256, 0, s>>>(B, d.n_h, prefix, n_splits, part_ml, part_o, (const float*)W_UV,
                                               out, lse);
  else
    combine_kernel<bf16><<<grid, 256, 0, s>>>(B, d.n_h, prefix, n_splits, part_ml, part_o, (const bf16*)W_UV,
                                              out, lse);
  return hipGetLastError();
}

}  // namespace mla
