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
// fp32 (VALU): workgroup (head h, 32 sequences); combined latents in LDS,
// each thread one output column for 16 sequences.
// bf16 (MFMA): workgroup (head h, 64 sequences); the combined latents are
// rounded to bf16 in LDS and o^T[d][b] = W^UV_h[d][:] . O~[b][:] runs as
// v_mfma_f32_32x32x16_bf16 (M = d, N = sequence, K = latent column), with
// W^UV rows read straight from global memory in the MFMA lane layout.
#include "mla_common.h"

namespace mla {
namespace {

constexpr int CB_SEQ = 32;

// Per-sequence merge parameters (one thread per sequence of the block).
struct MergeInfo {
  int32_t wfirst, count;
  float mstar, invL;
};

__device__ __forceinline__ MergeInfo merge_info(int32_t b, int32_t h, int32_t n_h, int64_t N, int32_t G,
                                                const int32_t* __restrict__ prefix,
                                                const float* __restrict__ part_ml, float* __restrict__ lse) {
  MergeInfo mi;
  const int64_t sb = prefix[b], n = prefix[b + 1] - sb;
  if (n <= 0) {
    mi.wfirst = 0;
    mi.count = 0;
    mi.mstar = 0.f;
    mi.invL = 0.f;
    if (lse) lse[(int64_t)b * n_h + h] = -INFINITY;
    return mi;
  }
  const int64_t w0 = split_of(sb, N, G), w1 = split_of(sb + n - 1, N, G);
  const int cnt = (int)(w1 - w0 + 1);
  float mstar = -INFINITY;
  for (int i = 0; i < cnt; ++i) mstar = fmaxf(mstar, part_ml[((w0 + i + b) * n_h + h) * 2]);
  float L = 0.f;
  for (int i = 0; i < cnt; ++i) {
    const float* ml = part_ml + ((w0 + i + b) * n_h + h) * 2;
    L += exp2f(ml[0] - mstar) * ml[1];
  }
  mi.wfirst = (int32_t)w0;
  mi.count = cnt;
  mi.mstar = mstar;
  mi.invL = 1.f / L;
  if (lse) lse[(int64_t)b * n_h + h] = (mstar + log2f(L)) * 0.69314718055994531f;
  return mi;
}

__global__ void __launch_bounds__(256) combine_f32_kernel(int32_t B, int32_t n_h, const int32_t* __restrict__ prefix,
                                                          int32_t G, const float* __restrict__ part_ml,
                                                          const float* __restrict__ part_o,
                                                          const float* __restrict__ W_UV, float* __restrict__ out,
                                                          float* __restrict__ lse) {
  __shared__ float ol[CB_SEQ][D_C + 4];
  __shared__ MergeInfo info[CB_SEQ];
  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * CB_SEQ;
  const int nb = min(CB_SEQ, B - b0);
  const int64_t N = prefix[B];
  if (tid < nb) info[tid] = merge_info(b0 + tid, h, n_h, N, G, prefix, part_ml, lse);
  __syncthreads();
  for (int bb = 0; bb < nb; ++bb) {
    const int b = b0 + bb;
    const MergeInfo mi = info[bb];
    float a0 = 0.f, a1 = 0.f;
    for (int i = 0; i < mi.count; ++i) {
      const int64_t slot = mi.wfirst + i + b;
      const float* src = part_o + (slot * n_h + h) * D_C;
      const float wgt = exp2f(part_ml[(slot * n_h + h) * 2] - mi.mstar);
      a0 = fmaf(wgt, src[tid], a0);
      a1 = fmaf(wgt, src[tid + 256], a1);
    }
    ol[bb][tid] = a0 * mi.invL;
    ol[bb][tid + 256] = a1 * mi.invL;
  }
  __syncthreads();
  // o[b][h][d] = sum_c W^UV[h*128 + d][c] * O~[b][c]; thread -> (d, half of the sequences)
  const int d = tid & (D_H - 1), half = tid >> 7;
  const float* wr = W_UV + ((int64_t)h * D_H + d) * D_C;
  float acc[CB_SEQ / 2];
#pragma unroll
  for (int j = 0; j < CB_SEQ / 2; ++j) acc[j] = 0.f;
  for (int c = 0; c < D_C; c += 4) {
    const float w0 = wr[c], w1 = wr[c + 1], w2 = wr[c + 2], w3 = wr[c + 3];
#pragma unroll
    for (int j = 0; j < CB_SEQ / 2; ++j) {
      const float* ov = &ol[half * (CB_SEQ / 2) + j][c];
      acc[j] = fmaf(w0, ov[0], fmaf(w1, ov[1], fmaf(w2, ov[2], fmaf(w3, ov[3], acc[j]))));
    }
  }
#pragma unroll
  for (int j = 0; j < CB_SEQ / 2; ++j) {
    const int bb = half * (CB_SEQ / 2) + j;
    if (bb < nb) out[((int64_t)(b0 + bb) * n_h + h) * D_H + d] = info[bb].count > 0 ? acc[j] : 0.f;
  }
}

// bf16: combined latents in LDS as [64 sequences][512] bf16 with 16-byte chunk
// c16 of sequence b at chunk c16 ^ (b & 15) (conflict-free column reads).
__global__ void __launch_bounds__(256) combine_mfma_kernel(int32_t B, int32_t n_h, const int32_t* __restrict__ prefix,
                                                           int32_t G, const float* __restrict__ part_ml,
                                                           const bf16* __restrict__ part_o,
                                                           const bf16* __restrict__ W_UV, float* __restrict__ out,
                                                           float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) char ol[64 * D_C * 2];
  __shared__ MergeInfo info[64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * 64;
  const int nb = min(64, B - b0);
  const int64_t N = prefix[B];
  if (tid < nb) info[tid] = merge_info(b0 + tid, h, n_h, N, G, prefix, part_ml, lse);
  __syncthreads();
  // combine: wave w merges sequences w, w+4, ...; lane owns latent columns 8*lane .. 8*lane+7
  for (int bb = wave; bb < 64; bb += 4) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (bb < nb) {
      const int b = b0 + bb;
      const MergeInfo mi = info[bb];
      for (int i = 0; i < mi.count; ++i) {
        const int64_t slot = mi.wfirst + i + b;
        const bf16x8 v = *(const bf16x8*)(part_o + (slot * n_h + h) * D_C + 8 * lane);
        const float wgt = exp2f(part_ml[(slot * n_h + h) * 2] - mi.mstar) * mi.invL;
#pragma unroll
        for (int k = 0; k < 8; ++k) a[k] = fmaf(wgt, (float)v[k], a[k]);
      }
    }
    bf16x8 r;
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = (bf16)a[k];
    *(bf16x8*)(ol + bb * 1024 + ((lane ^ (bb & 15)) << 4)) = r;
  }
  __syncthreads();
  // o^T[d][b]: wave w owns d = 32w .. 32w+31, both 32-sequence blocks
  f32x16 acc0, acc1;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    acc0[r] = 0.f;
    acc1[r] = 0.f;
  }
  const bf16* wr = W_UV + ((int64_t)h * D_H + 32 * wave + (lane & 31)) * D_C + 8 * (lane >> 5);
  const int bq0 = lane & 31, bq1 = 32 + (lane & 31);
#pragma unroll 8
  for (int ks = 0; ks < 32; ++ks) {
    const bf16x8 a = *(const bf16x8*)(wr + 16 * ks);
    const int c16 = 2 * ks + (lane >> 5);
    const bf16x8 q0 = *(const bf16x8*)(ol + bq0 * 1024 + ((c16 ^ (bq0 & 15)) << 4));
    const bf16x8 q1 = *(const bf16x8*)(ol + bq1 * 1024 + ((c16 ^ (bq1 & 15)) << 4));
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q0, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q1, acc1, 0, 0, 0);
  }
  // C layout: lane -> sequence (lane & 31) of the block, rows d = (r/4)*8 + 4*(lane>>5) + r%4
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int bb = 32 * j + (lane & 31);
    if (bb < nb) {
      const bool empty = info[bb].count == 0;
      float* dst = out + ((int64_t)(b0 + bb) * n_h + h) * D_H + 32 * wave + 4 * (lane >> 5);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x16& acc = j ? acc1 : acc0;
        f32x4 v = {acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]};
        if (empty) v = f32x4{0.f, 0.f, 0.f, 0.f};
        *(f32x4*)(dst + 8 * r4) = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_combine(const mla_dims& d, int32_t B, const int32_t* prefix, int32_t n_splits,
                          const float* part_ml, const void* part_o, const void* W_UV, float* out,
                          float* lse, hipStream_t s) {
  if (d.dtype == MLA_FP32) {
    dim3 grid(d.n_h, (B + CB_SEQ - 1) / CB_SEQ);
    combine_f32_kernel<<<grid, 256, 0, s>>>(B, d.n_h, prefix, n_splits, part_ml, (const float*)part_o,
                                            (const float*)W_UV, out, lse);
  } else {
    dim3 grid(d.n_h, (B + 63) / 64);
    combine_mfma_kernel<<<grid, 256, 0, s>>>(B, d.n_h, prefix, n_splits, part_ml, (const bf16*)part_o,
                                             (const bf16*)W_UV, out, lse);
  }
  return hipGetLastError();
}

}  // namespace mla
