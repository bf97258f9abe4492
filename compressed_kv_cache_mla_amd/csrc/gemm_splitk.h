// Skinny GEMM for a decode step's few rows: Y[M, N] = X[M, K] . W[N, K]^T
// with bf16 operands and fp32 accumulation, as device functions shared by
// the cache append (append_splitk.h), the query projection and the output
// projection (gemm.hip).
//
// Decode-step products have M <= 64 rows and weights of MBs to 100s of MBs,
// so they are bound by the weight stream.  The product is split over K into
// S chunks so that every compute unit streams a share of W: workgroup
// (16 output columns, chunk kc, 32 rows), 4 waves (quarters of the chunk,
// every operand load of a batch issued before its MFMAs,
// v_mfma_f32_16x16x32_bf16 with A = 16 rows of X, B = 16 rows of W); the
// chunk sums go to part[kc][m][N] in fp32.  The S chunks of an output element
// are then added in the fixed order kc = 0 .. S-1 and handed to an epilogue,
// either by a second launch over all elements or, in the same launch, by the
// last of the S workgroups of a (column, row) tile to finish, found with a
// counter.  Both orders of events give the same bits.
//
// W may be two matrices stacked by rows: output columns [0, n_split) come
// from W1 and [n_split, N) from W2 (the cache append's W^DKV and W^KR).
#pragma once

#include "mla_common.h"

namespace mla {

constexpr int GK_TOK = 32;                  // rows of X per workgroup (two MFMA tiles)
constexpr int GK_KB = 5;                    // K-steps of operand loads issued per batch
constexpr int GK_RED_FLOATS = 4 * GK_TOK * 17;   // LDS of the cross-wave reduction

struct GemmArgs {
  const bf16* X;      // [M, K], row stride ldx elements
  int64_t ldx;
  const bf16* W1;     // [n_split, K] row-major
  const bf16* W2;     // [N - n_split, K] row-major (may be NULL when n_split == N)
  int32_t n_split;
  int32_t M, N, K;
  int32_t S;          // K chunks, <= GK_S_MAX; K % (S * 128) == 0
  float* part;        // [S, M, N] fp32 chunk sums
  int32_t* counters;  // [ceil(M / 32), N / 16], zero before the first in-launch finish
};

// Chunk sums of workgroup (n_blk, kc, m_blk); red: GK_RED_FLOATS floats of LDS.
// COHERENT (in-launch finish): the sums are stored at system scope, written
// through every cache level, so that a workgroup on another XCD can read
// them in the same launch without a cache write-back fence.
template <bool COHERENT>
__device__ __forceinline__ void gemm_chunk(int n_blk, int kc, int m_blk, const GemmArgs& g, float* red) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n0 = n_blk * 16, m0 = m_blk * GK_TOK;
  const int K = g.K;
  const bf16* W = n0 < g.n_split ? g.W1 + (int64_t)n0 * K : g.W2 + (int64_t)(n0 - g.n_split) * K;
  const int kchunk = K / g.S, kw = kchunk / 4, nks = kw / 32;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int64_t k0 = (int64_t)kc * kchunk + wave * kw + kq;
  const bf16* wrow = W + (int64_t)r16 * K + k0;
  const bf16* xrow0 = g.X + (int64_t)min(m0 + r16, g.M - 1) * g.ldx + k0;
  const bf16* xrow1 = g.X + (int64_t)min(m0 + 16 + r16, g.M - 1) * g.ldx + k0;   // rows past M repeat row M-1
  f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  for (int b0 = 0; b0 < nks; b0 += GK_KB) {
    bf16x8 wv[GK_KB], xv0[GK_KB], xv1[GK_KB];
#pragma unroll
    for (int i = 0; i < GK_KB; ++i)
      if (b0 + i < nks) {
        wv[i] = *(const bf16x8*)(wrow + 32 * (b0 + i));
        xv0[i] = *(const bf16x8*)(xrow0 + 32 * (b0 + i));
        xv1[i] = *(const bf16x8*)(xrow1 + 32 * (b0 + i));
      }
#pragma unroll
    for (int i = 0; i < GK_KB; ++i)
      if (b0 + i < nks) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv0[i], wv[i], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv1[i], wv[i], acc1, 0, 0, 0);
      }
  }
  // C layout: lane holds output column lane%16, rows 4*(lane/16) + i of its tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    red[(wave * GK_TOK + 4 * (lane >> 4) + i) * 17 + r16] = acc0[i];
    red[(wave * GK_TOK + 16 + 4 * (lane >> 4) + i) * 17 + r16] = acc1[i];
  }
  __syncthreads();
  const int c = tid & 15;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int r = (tid >> 4) + 16 * half;
    const int m = m0 + r;
    auto rd = [&](int w) { return red[(w * GK_TOK + r) * 17 + c]; };
    if (m < g.M) {
      float* dst = g.part + ((int64_t)kc * g.M + m) * g.N + n0 + c;
      const float v = (rd(0) + rd(1)) + (rd(2) + rd(3));
      if (COHERENT)
        __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      else
        *dst = v;
    }
  }
}

constexpr int GK_S_MAX = 16;   // most K chunks of one product

// The finished value of columns 2cp, 2cp+1 of row m: its S chunk sums (all
// loaded first) added in the order kc = 0 .. S-1.  COHERENT: the sums are
// read at system scope.
template <bool COHERENT>
__device__ __forceinline__ float2 gemm_sum_pair(int m, int cp, const GemmArgs& g) {
  float v0[GK_S_MAX], v1[GK_S_MAX];
#pragma unroll
  for (int kc = 0; kc < GK_S_MAX; ++kc) {
    if (kc < g.S) {
      const float* src = g.part + ((int64_t)kc * g.M + m) * g.N + 2 * cp;
      if (COHERENT) {
        v0[kc] = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        v1[kc] = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      } else {
        const float2 v = *(const float2*)src;
        v0[kc] = v.x;
        v1[kc] = v.y;
      }
    }
  }
  float x0 = 0.f, x1 = 0.f;
#pragma unroll
  for (int kc = 0; kc < GK_S_MAX; ++kc)
    if (kc < g.S) {
      x0 += v0[kc];
      x1 += v1[kc];
    }
  return float2{x0, x1};
}

// In-launch finish of tile (n_blk, m_blk), called by each of its S workgroups
// right after gemm_chunk<true>: every workgroup waits until its chunk-sum
// stores have completed and counts itself in with a device-scope atomic; the
// one that brings the count to S adds the chunks (system-scope loads) and
// hands each column pair to epi(m, cp, x0, x1), then puts the counter back to
// zero for the next launch.
template <class Epi>
__device__ __forceinline__ void gemm_finish_tile(int n_blk, int m_blk, const GemmArgs& g, Epi&& epi,
                                                 int* lds_flag) {
  const int tid = threadIdx.x;
  __builtin_amdgcn_s_waitcnt(0);   // this thread's sum stores are complete
  __syncthreads();
  int32_t* cnt = g.counters + (int64_t)m_blk * (g.N / 16) + n_blk;
  if (tid == 0) *lds_flag = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g.S - 1;
  __syncthreads();
  if (!*lds_flag) return;
  {
    const int r = tid >> 3, cp = tid & 7;   // 32 rows x 8 column pairs
    const int m = m_blk * GK_TOK + r;
    if (m < g.M) {
      const float2 x = gemm_sum_pair<true>(m, n_blk * 8 + cp, g);
      epi(m, n_blk * 8 + cp, x.x, x.y);
    }
  }
  if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace mla
