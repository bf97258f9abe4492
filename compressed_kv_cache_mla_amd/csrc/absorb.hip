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

// ---------------------------------------------------------------- bf16 query path fused with the absorption
// The decode layer's q^C = W^UQ c^Q ("DeepSeek-V2：在“大力出奇迹”的AI军备竞赛中，
// 四两拨千斤" (liang.world), ch.2 §2 closing paragraph: the query has its own
// low-rank compression c^Q; "DeepSeek 系列模型技术深度解读" (tuntang.top),
// "RoPE 的兼容性处理": q^C_t = W^UQ c^Q_t) is computed where it is absorbed, so
// q^C never goes to memory.  Workgroup (head h, 32 sequences), 4 waves:
//  1. W^UK_h (128 x 512, its four 128-column quarters, 128 KB) is copied to
//     LDS with global_load_lds, in the chunk placement of absorb_mfma_block,
//     while
//  2. q^C_h^T[d][b] = sum_k W^UQ[128h + d][k] c^Q[b][k] runs as
//     v_mfma_f32_16x16x32_bf16 with A = a packed W^UQ block and B = a packed
//     c^Q block: wave w owns d = 32w .. 32w+31 (two 16-row blocks) for the 32
//     sequences (two 16-column blocks), over all d_cq/32 K-steps, with the
//     operand loads of FQ_KB K-steps issued before their MFMAs;
//  3. q^C_h is rounded to bf16, as the query projection stores it, into LDS,
//     and q~ = W^UK_h^T q^C_h runs as in absorb_mfma_block for each quarter
//     (wave w: latent columns 128cq + 32w .. +31), then the RoPE half.
// Grid (n_h, ceil(B / 32)): workgroup (h, y) is number y*n_h + h, so the
// workgroups of one head share an XCD (number mod 8) and its L2 serves their
// second reads of W^UQ_h and W^UK_h.  Rows of the packed c^Q past B (padding)
// only reach output columns of sequences that are not stored.
constexpr int FQ_KB = 6;

__global__ void __launch_bounds__(256) absorb_fused_kernel(int32_t B, int32_t n_h, int32_t d_cq,
                                                           const bf16* __restrict__ cQ, const bf16* __restrict__ W_UQ,
                                                           const bf16* __restrict__ q_R,
                                                           const int32_t* __restrict__ pos_q,
                                                           const bf16* __restrict__ W_UK, float qscale, RopeTab rope,
                                                           bf16* __restrict__ qabs) {
  __shared__ __attribute__((aligned(1024))) char wl[4 * D_H * 256];
  __shared__ __attribute__((aligned(16))) bf16 qcl[32 * D_H];   // q^C of the 32 sequences, [b][d]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // heads h and h^1 (which share the 128-byte lines of the q~ layout) are 8
  // workgroups apart, on one XCD
  const int h = (n_h & 15) ? (int)blockIdx.x
                           : (int)((blockIdx.x & ~15u) | ((blockIdx.x & 7) << 1) | ((blockIdx.x >> 3) & 1));
  const int b0 = blockIdx.y * 32;
  const int nb = min(32, B - b0);
  // 1. W^UK_h -> LDS: 128 copy instructions of 1 KB, 32 per quarter
  const char* wsrc = (const char*)(W_UK + (int64_t)h * D_H * D_C);
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int I = wave * 32 + k;
    const int cq = I >> 5, sigma = (I & 31) * 64 + lane;
    const int d = sigma >> 4, pos = sigma & 15;
    const int c16 = pos ^ ((d & 3) << 2);
    __builtin_amdgcn_global_load_lds((const void*)(wsrc + 256 * cq + (int64_t)d * 1024 + c16 * 16),
                                     (lds_void_t*)(wl + cq * (D_H * 256) + (I & 31) * 1024), 16, 0, 0);
  }
  // 2. q^C_h^T: C[d][b], lane holds d = 32w + 16t + 4(lane>>4) + i, b = 16j + (lane&15)
  const int nks = d_cq >> 5;
  const int64_t rbs = (int64_t)nks * 512;   // elements from one 16-row block to the next
  const bf16* wq = W_UQ + (int64_t)(8 * h + 2 * wave) * rbs + lane * 8;
  const bf16* xq = cQ + (int64_t)(b0 >> 4) * rbs + lane * 8;
  const bool two = nb > 16;
  f32x4 acc[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < nks; k0 += FQ_KB) {
    bf16x8 wv[2][FQ_KB], xv[2][FQ_KB];
#pragma unroll
    for (int i = 0; i < FQ_KB; ++i)
      if (k0 + i < nks) {
        wv[0][i] = *(const bf16x8*)(wq + 512 * (k0 + i));
        wv[1][i] = *(const bf16x8*)(wq + rbs + 512 * (k0 + i));
        xv[0][i] = *(const bf16x8*)(xq + 512 * (k0 + i));
        if (two) xv[1][i] = *(const bf16x8*)(xq + rbs + 512 * (k0 + i));
      }
#pragma unroll
    for (int i = 0; i < FQ_KB; ++i)
      if (k0 + i < nks) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          acc[t][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[t][i], xv[0][i], acc[t][0], 0, 0, 0);
          if (two) acc[t][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[t][i], xv[1][i], acc[t][1], 0, 0, 0);
        }
      }
  }
  // 3. q^C (bf16) -> LDS
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (j == 0 || two) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (bf16)acc[t][j][i];
        *(bf16x4*)(qcl + (16 * j + (lane & 15)) * D_H + 32 * wave + 16 * t + 4 * (lane >> 4)) = v;
      }
  __builtin_amdgcn_s_waitcnt(0);   // this wave's W^UK copies have landed
  __syncthreads();
  // q~^T[c][b] = sum_d W^UK_h[d][c] q^C[b][d]: v_mfma_f32_32x32x16_bf16 with
  // M = latent column c, N = sequence (lane & 31), K = d
  bf16x8 qf[8];
  {
    const int b = min(lane & 31, nb - 1);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8*)(qcl + b * D_H + 16 * ks + 8 * (lane >> 5));
  }
  const int t_row = 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int t_c16 = 4 * wave + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int t_half = (lane & 1) * 8;
#pragma unroll
  for (int cq = 0; cq < 4; ++cq) {
    const char* wq4 = wl + cq * (D_H * 256);
    f32x16 a;
#pragma unroll
    for (int r = 0; r < 16; ++r) a[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bf16x8 af;
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int d = 16 * ks + t_row + 4 * rr;
        const int c16 = t_c16 ^ ((d & 3) << 2);
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(wq4 + d * 256 + c16 * 16 + t_half));
        const bf16x4 vb = __builtin_bit_cast(bf16x4, v);
        af[4 * rr + 0] = vb[0];
        af[4 * rr + 1] = vb[1];
        af[4 * rr + 2] = vb[2];
        af[4 * rr + 3] = vb[3];
      }
      a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ks], a, 0, 0, 0);
    }
    const int bb = lane & 31;
    store_qabs_block(a, qscale, bb < nb ? qabs + (int64_t)(b0 + bb) * n_h * D_K : nullptr, n_h, h,
                     128 * cq + 32 * wave, lane);
  }
  // RoPE half: 32 sequences x 32 pairs
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = tid + 256 * j, bb = i >> 5, k = i & 31;
    if (bb < nb) {
      const int b = b0 + bb;
      const bf16x2 x = *(const bf16x2*)(q_R + ((int64_t)b * n_h + h) * D_R + 2 * k);
      const float x0 = (float)x[0], x1 = (float)x[1];
      float cs, sn;
      rope_cos_sin(pos_q[b], k, rope, &cs, &sn);
      bf16x2 o;
      o[0] = (bf16)((x0 * cs - x1 * sn) * qscale);
      o[1] = (bf16)((x0 * sn + x1 * cs) * qscale);
      *(bf16x2*)(qabs + (int64_t)b * n_h * D_K + qabs_offset(n_h, true, h, D_C + 2 * k)) = o;
    }
  }
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

hipError_t launch_absorb_fused(const mla_dims& d, int32_t B, int32_t d_cq, const void* cQ_packed,
                               const void* W_UQ_packed, const void* q_R, const int32_t* pos_q, const void* W_UK,
                               void* qabs, hipStream_t s) {
  if (!absorb_fused_supported(d, B, d_cq)) return hipErrorInvalidValue;
  dim3 grid(d.n_h, (B + 31) / 32);
  absorb_fused_kernel<<<grid, 256, 0, s>>>(B, d.n_h, d_cq, (const bf16*)cQ_packed, (const bf16*)W_UQ_packed,
                                           (const bf16*)q_R, pos_q, (const bf16*)W_UK, d.softmax_scale * LOG2E,
                                           rope_table(d.rope_base), (bf16*)qabs);
  return hipGetLastError();
}

}  // namespace mla
