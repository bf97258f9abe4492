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
// bf16 (MFMA): workgroup (head h, 16 sequences), one wave per sequence; the
// combined latents are rounded to bf16 in LDS and o^T[d][b] = W^UV_h[d][:] .
// O~[b][:] runs as v_mfma_f32_16x16x32_bf16 (M = d, N = sequence, K = latent).
#include "gemm_splitk.h"

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

// Decode step: the append's flags (word 1 of the flag area) join the decode's
// (word 0) once both launches before this one are done; word 1 goes back to 0.
// ext (may be NULL): a caller's flag word that also receives the step's flags.
__device__ __forceinline__ void merge_step_flags(int32_t* flags, int32_t* ext) {
  if (flags && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    const int32_t v = flags[1];
    int32_t all = flags[0] | v;
    if (v) {
      all = atomicOr(flags, v) | v;
      flags[1] = 0;
    }
    if (ext && all) atomicOr(ext, all);
  }
}

__global__ void __launch_bounds__(256) combine_f32_kernel(int32_t B, int32_t n_h, const int32_t* __restrict__ prefix,
                                                          int32_t G, const float* __restrict__ part_ml,
                                                          const float* __restrict__ part_o,
                                                          const float* __restrict__ W_UV, float* __restrict__ out,
                                                          float* __restrict__ lse, int32_t* merge_flags,
                                                          int32_t* ext_flags) {
  __shared__ float ol[CB_SEQ][D_C + 4];
  merge_step_flags(merge_flags, ext_flags);
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

// bf16: workgroup (head h, CS sequences), 16 waves.  Wave w merges
// sequences w, w + 16, ...: the per-slot weights 2^(m_s - m*) / L are formed
// lane-parallel over the slots (lane j holds slot j's weight), then every
// lane sums 8 latent columns over the slots with up to CB slots' loads in
// flight.  The merged latents go to LDS as bf16 [CS][512] (16-byte chunk c of
// sequence b at chunk c ^ (b & 15): conflict-free fragment reads), and
// o^T[d][b] = W^UV_h[d][:] . O~[b][:] runs as v_mfma_f32_16x16x32_bf16 in
// waves 0..7 (wave w: d = 16w .. 16w+15, CS/16 blocks of 16 sequences), W^UV
// rows read straight from global memory in the A layout, once per CS
// sequences.
constexpr int CB_MAX = 8;

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int CS>
__global__ void __launch_bounds__(1024) combine_mfma_kernel(int32_t B, int32_t n_h, const int32_t* __restrict__ prefix,
                                                            int32_t G, const float* __restrict__ part_ml,
                                                            const bf16* __restrict__ part_o,
                                                            const bf16* __restrict__ W_UV, float* __restrict__ out,
                                                            float* __restrict__ lse, int32_t* merge_flags,
                                                            bf16* __restrict__ out_packed, int32_t* ext_flags) {
  constexpr int NBQ = CS / 16;
  constexpr int CB = CB_MAX;
  constexpr bool PRE = CS == 16;   // registers allow the W^UV prefetch with one accumulator block
  merge_step_flags(merge_flags, ext_flags);
  __shared__ __attribute__((aligned(16))) char ol[CS * D_C * 2];
  __shared__ int empty_l[CS];
  __shared__ __attribute__((aligned(16))) float red[CS == 16 ? 16 * 64 * 8 : 4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * CS;
  const int nb = min(CS, B - b0);
  const int64_t N = prefix[B];
  // With one accumulator block (CS = 16) the epilogue waves' W^UV_h rows are
  // loaded first, so that their latency passes while the partials are merged.
  const bf16* wr = W_UV + ((int64_t)h * D_H + 16 * (wave & 7) + (lane & 15)) * D_C + 8 * (lane >> 4);
  bf16x8 wpre[PRE ? D_C / 32 : 1];
  if (PRE && wave < D_H / 16) {
#pragma unroll
    for (int ks = 0; ks < D_C / 32; ++ks) wpre[ks] = *(const bf16x8*)(wr + 32 * ks);
  }
  // Few sequences in the block (CS = 16 only): WPS waves share a sequence,
  // each merging every WPS-th slot, and their sums are added in LDS in a
  // fixed order; otherwise one wave merges a whole sequence.
  const int WPS = CS == 16 && nb <= 8 ? (nb <= 1 ? 16 : nb <= 2 ? 8 : nb <= 4 ? 4 : 2) : 1;
  if (WPS > 1) {
    const int bb = wave / WPS, pp = wave % WPS;
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int empty = 1;
    if (bb < nb) {
      const int b = b0 + bb;
      const int64_t sb = prefix[b], n = prefix[b + 1] - sb;
      if (n <= 0 && lse && lane == 0 && pp == 0) lse[(int64_t)b * n_h + h] = -INFINITY;
      if (n > 0) {
        empty = 0;
        const int64_t w0 = split_of(sb, N, G), w1 = split_of(sb + n - 1, N, G);
        const int cnt = (int)(w1 - w0 + 1);
        const float* ml = part_ml + ((w0 + b) * n_h + h) * 2;
        const int64_t mstride = (int64_t)2 * n_h;
        float mx = -INFINITY;
        for (int i = lane; i < cnt; i += 64) mx = fmaxf(mx, ml[i * mstride]);
        mx = wave_max64(mx);
        float L = 0.f;
        for (int i = lane; i < cnt; i += 64) L += exp2f(ml[i * mstride] - mx) * ml[i * mstride + 1];
        L = wave_sum64(L);
        const float invL = 1.f / L;
        if (lse && lane == 0 && pp == 0) lse[(int64_t)b * n_h + h] = (mx + log2f(L)) * 0.69314718055994531f;
        const bf16* po = part_o + ((w0 + b) * n_h + h) * D_C + 8 * lane;
        const int64_t sstride = (int64_t)n_h * D_C;
        for (int i0 = 0; i0 < cnt; i0 += 64) {
          const int m = min(64, cnt - i0);
          const float wl = lane < m ? exp2f(ml[(i0 + lane) * mstride] - mx) * invL : 0.f;
          for (int i = pp; i < m; i += WPS * CB) {
            bf16x8 v[CB];
#pragma unroll
            for (int u = 0; u < CB; ++u)
              if (i + u * WPS < m) v[u] = *(const bf16x8*)(po + sstride * (i0 + i + u * WPS));
#pragma unroll
            for (int u = 0; u < CB; ++u)
              if (i + u * WPS < m) {
                const float wg = __shfl(wl, i + u * WPS);
#pragma unroll
                for (int k = 0; k < 8; ++k) a[k] = fmaf(wg, (float)v[u][k], a[k]);
              }
          }
        }
      }
    }
    float4* rw = (float4*)(red + (wave * 64 + lane) * 8);
    rw[0] = float4{a[0], a[1], a[2], a[3]};
    rw[1] = float4{a[4], a[5], a[6], a[7]};
    __syncthreads();
    {
      const int sq = wave;   // sequence column written by this wave
      float t[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (sq < nb) {
        for (int q = 0; q < WPS; ++q) {
          const float4* rr = (const float4*)(red + ((sq * WPS + q) * 64 + lane) * 8);
          const float4 x0 = rr[0], x1 = rr[1];
          t[0] += x0.x; t[1] += x0.y; t[2] += x0.z; t[3] += x0.w;
          t[4] += x1.x; t[5] += x1.y; t[6] += x1.z; t[7] += x1.w;
        }
      }
      bf16x8 r;
#pragma unroll
      for (int k = 0; k < 8; ++k) r[k] = (bf16)t[k];
      *(bf16x8*)(ol + sq * 1024 + ((lane ^ (sq & 15)) << 4)) = r;
      if (lane == 0 && pp == 0 && bb < CS) empty_l[bb] = empty;
      if (lane == 0 && sq >= nb) empty_l[sq] = 1;
    }
  } else {
    for (int bb = wave; bb < CS; bb += 16) {
      float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      int empty = 1;
      if (bb < nb) {
        const int b = b0 + bb;
        const int64_t sb = prefix[b], n = prefix[b + 1] - sb;
        if (n <= 0 && lse && lane == 0) lse[(int64_t)b * n_h + h] = -INFINITY;
        if (n > 0) {
          empty = 0;
          const int64_t w0 = split_of(sb, N, G), w1 = split_of(sb + n - 1, N, G);
          const int cnt = (int)(w1 - w0 + 1);
          const float* ml = part_ml + ((w0 + b) * n_h + h) * 2;   // slot w0 + b + i at ml + 2*n_h*i
          const int64_t mstride = (int64_t)2 * n_h;
          float mx = -INFINITY;
          for (int i = lane; i < cnt; i += 64) mx = fmaxf(mx, ml[i * mstride]);
          mx = wave_max64(mx);
          float L = 0.f;
          for (int i = lane; i < cnt; i += 64) L += exp2f(ml[i * mstride] - mx) * ml[i * mstride + 1];
          L = wave_sum64(L);
          const float invL = 1.f / L;
          if (lse && lane == 0) lse[(int64_t)b * n_h + h] = (mx + log2f(L)) * 0.69314718055994531f;
          const bf16* po = part_o + ((w0 + b) * n_h + h) * D_C + 8 * lane;   // slot i at po + n_h*D_C*i
          const int64_t sstride = (int64_t)n_h * D_C;
          for (int i0 = 0; i0 < cnt; i0 += 64) {
            const int m = min(64, cnt - i0);
            const float wl = lane < m ? exp2f(ml[(i0 + lane) * mstride] - mx) * invL : 0.f;
            for (int i = 0; i < m; i += CB) {
              bf16x8 v[CB];
  #pragma unroll
              for (int u = 0; u < CB; ++u)
                if (i + u < m) v[u] = *(const bf16x8*)(po + sstride * (i0 + i + u));
  #pragma unroll
              for (int u = 0; u < CB; ++u)
                if (i + u < m) {
                  const float wg = __shfl(wl, i + u);
  #pragma unroll
                  for (int k = 0; k < 8; ++k) a[k] = fmaf(wg, (float)v[u][k], a[k]);
                }
            }
          }
        }
      }
      bf16x8 r;
  #pragma unroll
      for (int k = 0; k < 8; ++k) r[k] = (bf16)a[k];
      *(bf16x8*)(ol + bb * 1024 + ((lane ^ (bb & 15)) << 4)) = r;
      if (lane == 0) empty_l[bb] = empty;
    }
  }
  __syncthreads();
  if (wave >= D_H / 16) return;
  // o^T[d][b]: A = W^UV rows d (16 x 32 per MFMA), B = O~^T (32 latent columns x 16 sequences)
  f32x4 acc[NBQ];
#pragma unroll
  for (int j = 0; j < NBQ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int bq = lane & 15;
#pragma unroll
  for (int ks = 0; ks < D_C / 32; ++ks) {
    const int c16 = 4 * ks + (lane >> 4);
    const bf16x8 afr = PRE ? wpre[PRE ? ks : 0] : *(const bf16x8*)(wr + 32 * ks);
#pragma unroll
    for (int j = 0; j < NBQ; ++j) {
      const bf16x8 bfr = *(const bf16x8*)(ol + (16 * j + bq) * 1024 + ((c16 ^ bq) << 4));
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr, acc[j], 0, 0, 0);
    }
  }
  // C layout: lane holds d = 16w + 4*(lane>>4) + i, sequence 16j + (lane & 15)
#pragma unroll
  for (int j = 0; j < NBQ; ++j) {
    const int bb = 16 * j + bq;
    if (bb < nb) {
      f32x4 v = acc[j];
      if (empty_l[bb]) v = f32x4{0.f, 0.f, 0.f, 0.f};
      *(f32x4*)(out + ((int64_t)(b0 + bb) * n_h + h) * D_H + 16 * wave + 4 * (lane >> 4)) = v;
      if (out_packed) {
        // the same 4 values rounded to bf16, in the packed activation layout
        // of the output projection (row b0 + bb, columns h*d_h + ...: 4
        // consecutive elements of one lane group)
        bf16x4 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) pb[i] = (bf16)v[i];
        *(bf16x4*)(out_packed + packed_index(b0 + bb, h * D_H + 16 * wave + 4 * (lane >> 4), (int64_t)n_h * D_H)) = pb;
      }
    }
  }
}

}  // namespace

hipError_t launch_combine(const mla_dims& d, int32_t B, const int32_t* prefix, int32_t n_splits,
                          const float* part_ml, const void* part_o, const void* W_UV, float* out,
                          float* lse, int32_t* merge_flags, void* out_packed, hipStream_t s, int32_t* ext_flags) {
  bf16* op = d.dtype == MLA_BF16 ? (bf16*)out_packed : nullptr;
  if (d.dtype == MLA_FP32) {
    dim3 grid(d.n_h, (B + CB_SEQ - 1) / CB_SEQ);
    combine_f32_kernel<<<grid, 256, 0, s>>>(B, d.n_h, prefix, n_splits, part_ml, (const float*)part_o,
                                            (const float*)W_UV, out, lse, merge_flags, ext_flags);
  } else {
    // the most sequences per workgroup (W^UV is read once per block of them)
    // that still leave at least two workgroups per compute unit (64, for long
    // query batches such as prefill chunks) or one (32); else 16
    if (B > 32 && d.n_h * ((B + 63) / 64) >= 512) {
      dim3 grid(d.n_h, (B + 63) / 64);
      combine_mfma_kernel<64><<<grid, 1024, 0, s>>>(B, d.n_h, prefix, n_splits, part_ml, (const bf16*)part_o,
                                                    (const bf16*)W_UV, out, lse, merge_flags, op, ext_flags);
    } else if (B > 16 && d.n_h * ((B + 31) / 32) >= 256) {
      dim3 grid(d.n_h, (B + 31) / 32);
      combine_mfma_kernel<32><<<grid, 1024, 0, s>>>(B, d.n_h, prefix, n_splits, part_ml, (const bf16*)part_o,
                                                    (const bf16*)W_UV, out, lse, merge_flags, op, ext_flags);
    } else {
      dim3 grid(d.n_h, (B + 15) / 16);
      combine_mfma_kernel<16><<<grid, 1024, 0, s>>>(B, d.n_h, prefix, n_splits, part_ml, (const bf16*)part_o,
                                                    (const bf16*)W_UV, out, lse, merge_flags, op, ext_flags);
    }
  }
  return hipGetLastError();
}

}  // namespace mla
