// Query absorption: q~_i = W^UK_i^T q^C_i and RoPE(q^R_i) at the query
// position, both scaled by softmax_scale * log2(e): 576 values per
// (sequence, head) in the decode workspace, placed by qabs_offset (rows of 576
// for fp32, the attention kernel's load order for bf16).
//   "DeepSeek-V2：在“大力出奇迹”的AI军备竞赛中，四两拨千斤" (liang.world), ch.2 §2:
//   by associativity W^UK is absorbed into the query side, so the score with
//   k^C_j = W^UK c_j is q^C . W^UK c_j = (W^UK^T q^C) . c_j and keys are never
//   rebuilt; ch.2 §3: the RoPE half q^R is rotated and dotted with the shared
//   k^R.  "DeepSeek 系列模型技术深度解读" (tuntang.top), "RoPE 的兼容性处理":
//   q_t = [W^UQ c^Q ; W^QR h . RoPE(t)].
//
// Per head the product is [B x d_h] x [d_h x d_c] with the contraction over
// W^UK's row index.  fp32 (VALU): workgroup (head h, 32 sequences), W^UK_h
// (128 x 512) streamed through LDS in 32-row chunks; each thread owns 2 latent
// columns for the 32 sequences, q^C comes from LDS.  bf16: the MFMA kernel below.
#include <algorithm>

#include "absorb_mfma.h"

namespace mla {
namespace {

constexpr int AB_SEQ = 32;
constexpr int AB_DK = 32;

template <typename T>
__global__ void __launch_bounds__(256) absorb_kernel(int32_t B, int32_t n_h, const T* __restrict__ q_C,
                                                     const T* __restrict__ q_R, const int32_t* __restrict__ pos_q,
                                                     const T* __restrict__ W_UK, float qscale, RopeTab rope,
                                                     T* __restrict__ qabs) {
  __shared__ float qs[AB_SEQ][D_H + 1];
  __shared__ float ws[AB_DK][D_C];
  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * AB_SEQ;
  const int nb = min(AB_SEQ, B - b0);
  for (int i = tid; i < AB_SEQ * D_H; i += 256) {
    const int bb = i / D_H, d = i % D_H;
    qs[bb][d] = bb < nb ? to_f32(q_C[((int64_t)(b0 + bb) * n_h + h) * D_H + d]) : 0.f;
  }
  float acc[AB_SEQ][2];
#pragma unroll
  for (int bb = 0; bb < AB_SEQ; ++bb) acc[bb][0] = acc[bb][1] = 0.f;
  const T* W = W_UK + (int64_t)h * D_H * D_C;
  for (int d0 = 0; d0 < D_H; d0 += AB_DK) {
    __syncthreads();
    for (int i = tid; i < AB_DK * D_C; i += 256) ws[i / D_C][i % D_C] = to_f32(W[(int64_t)(d0 + i / D_C) * D_C + i % D_C]);
    __syncthreads();
#pragma unroll 4
    for (int dd = 0; dd < AB_DK; ++dd) {
      const float w0 = ws[dd][tid], w1 = ws[dd][tid + 256];
#pragma unroll
      for (int bb = 0; bb < AB_SEQ; ++bb) {
        const float qv = qs[bb][d0 + dd];
        acc[bb][0] = fmaf(qv, w0, acc[bb][0]);
        acc[bb][1] = fmaf(qv, w1, acc[bb][1]);
      }
    }
  }
  for (int bb = 0; bb < nb; ++bb) {
    T* dst = qabs + ((int64_t)(b0 + bb) * n_h + h) * D_K;
    dst[tid] = from_f32<T>(acc[bb][0] * qscale);
    dst[tid + 256] = from_f32<T>(acc[bb][1] * qscale);
  }
  // RoPE half: 32 pairs per sequence
  for (int i = tid; i < nb * (D_R / 2); i += 256) {
    const int bb = i / (D_R / 2), k = i % (D_R / 2);
    const int b = b0 + bb;
    const T* src = q_R + ((int64_t)b * n_h + h) * D_R;
    const float x0 = to_f32(src[2 * k]), x1 = to_f32(src[2 * k + 1]);
    float cs, sn;
    rope_cos_sin(pos_q[b], k, rope, &cs, &sn);
    T* dst = qabs + ((int64_t)b * n_h + h) * D_K + D_C;
    dst[2 * k] = from_f32<T>((x0 * cs - x1 * sn) * qscale);
    dst[2 * k + 1] = from_f32<T>((x0 * sn + x1 * cs) * qscale);
  }
}

// ---------------------------------------------------------------- bf16 (MFMA)
// absorb_mfma.h: workgroup (head, latent-column quarter, 64 sequences).  The
// last workgroup of the grid runs the decode plan instead.
__global__ void __launch_bounds__(256) absorb_mfma_kernel(int32_t B, int32_t n_h, const bf16* __restrict__ q_C,
                                                          const bf16* __restrict__ q_R,
                                                          const int32_t* __restrict__ pos_q,
                                                          const bf16* __restrict__ W_UK, float qscale,
                                                          RopeTab rope, bf16* __restrict__ qabs, PlanArgs pa,
                                                          int32_t nby) {
  __shared__ __attribute__((aligned(1024))) char wl[D_H * 256];
  if (blockIdx.x == 4 * n_h) {
    if (blockIdx.y == 0) plan_block<256>(pa, (int32_t*)wl, D_H * 256 / 4 - 256);
    return;
  }
  absorb_mfma_block(blockIdx.x, blockIdx.y, nby, B, n_h, q_C, q_R, pos_q, W_UK, qscale, rope, qabs, wl);
}

}  // namespace

hipError_t launch_absorb(const mla_dims& d, int32_t B, const void* q_C, const void* q_R, const int32_t* pos_q,
                         const void* W_UK, void* qabs, const PlanArgs& pa, hipStream_t s) {
  const float qscale = d.softmax_scale * LOG2E;
  if (d.dtype == MLA_FP32) {
    hipError_t e = launch_plan(pa, s);
    if (e != hipSuccess) return e;
    dim3 grid(d.n_h, (B + AB_SEQ - 1) / AB_SEQ);
    absorb_kernel<float><<<grid, 256, 0, s>>>(B, d.n_h, (const float*)q_C, (const float*)q_R, pos_q,
                                              (const float*)W_UK, qscale, rope_table(d.rope_base), (float*)qabs);
  } else {
    // blocks of 64 sequences per workgroup: one, unless the grid would exceed
    // ~1024 workgroups; then each W^UK block serves several (long batches)
    const int32_t nblocks = (B + 63) / 64;
    const int32_t nby = std::max<int32_t>(1, (int32_t)((int64_t)nblocks * 4 * d.n_h / 1024));
    dim3 g2(4 * d.n_h + 1, (nblocks + nby - 1) / nby);
    absorb_mfma_kernel<<<g2, 256, 0, s>>>(B, d.n_h, (const bf16*)q_C, (const bf16*)q_R, pos_q, (const bf16*)W_UK,
                                         qscale, rope_table(d.rope_base), (bf16*)qabs, pa, nby);
  }
  return hipGetLastError();
}

}  // namespace mla
