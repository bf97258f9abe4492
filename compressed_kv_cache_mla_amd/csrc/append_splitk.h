// Split-K cache append for a decode step's few token rows (bf16), as device
// functions shared by the two-launch path (append.hip) and the fused decode
// step (step.hip).
//
// c^KV = W^DKV h_t and k^R = RoPE(W^KR h_t) ("DeepSeek-V2：在“大力出奇迹”的AI军备竞赛中，
// 四两拨千斤" (liang.world), ch.2 §2-§3; "DeepSeek 系列模型技术深度解读" (tuntang.top),
// "RoPE 的兼容性处理").  The [T x d_model] x [d_model x 576] product is split
// over d_model into SK_SPLIT chunks so that the weight stream is spread over
// the whole GPU: workgroup (16 output columns, chunk kc, 32 tokens), 4 waves
// (quarters of the chunk, every operand load issued before the MFMAs); its
// fp32 chunk sums go to part[kc][t][576].  The chunks of an output element are
// then added in the fixed order kc = 0 .. SK_SPLIT-1, RoPE is applied to the
// k^R pairs and the row is stored: either by a second launch over all
// elements, or, in the fused step, by the last of the SK_SPLIT workgroups of a
// (column, token) tile to finish, found with a counter.  Both give the same
// bits.
#pragma once

#include "mla_common.h"

namespace mla {

constexpr int SK_SPLIT = APPEND_SK_SPLIT;   // d_model chunks
constexpr int SK_KB = 5;      // K-steps of operand loads issued per batch (d_model 5120: all of them)

// Where and how the finished rows are stored.
struct AppendDst {
  const int32_t* seq_id;   // NULL: token t belongs to sequence t
  const int32_t* pos;
  const int32_t* page_table;
  int32_t num_seqs, max_pages, page_size, num_pages;
  bf16* c_KV;
  bf16* k_R;
  int64_t row_stride;
  RopeTab rope;
  int32_t* err_flag;       // may be NULL
};

// Tokens per workgroup: two 16-token MFMA tiles share each W^DKV / W^KR
// fragment load.
constexpr int SK_TOK = 32;
// LDS of a workgroup's cross-wave reduction (floats): [wave][token][16 + 1]
constexpr int SK_RED_FLOATS = 4 * SK_TOK * 17;

// Chunk sums of workgroup (col_blk, kc, tok_blk); red: SK_RED_FLOATS floats of
// LDS.  COHERENT (in-launch finish): the sums are stored at system scope, i.e.
// written through every cache level, so that a workgroup on another XCD can
// read them in the same launch without a cache write-back fence.
template <bool COHERENT = false>
__device__ __forceinline__ void append_splitk_block(int col_blk, int kc, int tok_blk, int32_t T_rows,
                                                    int32_t d_model, const bf16* __restrict__ h,
                                                    const bf16* __restrict__ W_DKV, const bf16* __restrict__ W_KR,
                                                    float* __restrict__ part, float* red) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col0 = col_blk * 16, tok0 = tok_blk * SK_TOK;
  const bf16* W = col0 < D_C ? W_DKV + (int64_t)col0 * d_model : W_KR + (int64_t)(col0 - D_C) * d_model;
  const int kchunk = d_model / SK_SPLIT, kw = kchunk / 4, nks = kw / 32;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int64_t k0 = (int64_t)kc * kchunk + wave * kw + kq;
  const bf16* wrow = W + (int64_t)r16 * d_model + k0;
  const bf16* hrow0 = h + (int64_t)min(tok0 + r16, T_rows - 1) * d_model + k0;
  const bf16* hrow1 = h + (int64_t)min(tok0 + 16 + r16, T_rows - 1) * d_model + k0;
  f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  for (int b0 = 0; b0 < nks; b0 += SK_KB) {
    bf16x8 wv[SK_KB], hv0[SK_KB], hv1[SK_KB];
#pragma unroll
    for (int i = 0; i < SK_KB; ++i)
      if (b0 + i < nks) {
        wv[i] = *(const bf16x8*)(wrow + 32 * (b0 + i));
        hv0[i] = *(const bf16x8*)(hrow0 + 32 * (b0 + i));
        hv1[i] = *(const bf16x8*)(hrow1 + 32 * (b0 + i));   // rows past T repeat row T-1
      }
#pragma unroll
    for (int i = 0; i < SK_KB; ++i)
      if (b0 + i < nks) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hv0[i], wv[i], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hv1[i], wv[i], acc1, 0, 0, 0);
      }
  }
  // C layout: lane holds output column lane%16, tokens 4*(lane/16) + i of its tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    red[(wave * SK_TOK + 4 * (lane >> 4) + i) * 17 + r16] = acc0[i];
    red[(wave * SK_TOK + 16 + 4 * (lane >> 4) + i) * 17 + r16] = acc1[i];
  }
  __syncthreads();
  const int c = tid & 15;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int r = (tid >> 4) + 16 * half;
    const int t = tok0 + r;
    auto rd = [&](int w) { return red[(w * SK_TOK + r) * 17 + c]; };
    if (t < T_rows) {
      float* dst = part + ((int64_t)kc * T_rows + t) * D_K + col0 + c;
      const float v = (rd(0) + rd(1)) + (rd(2) + rd(3));
      if (COHERENT)
        __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      else
        *dst = v;
    }
  }
}

// Final value of column pair cp (columns 2cp, 2cp+1) of token t: the chunk
// sums added in order, RoPE on k^R pairs, rounded and stored into the pool.
// COHERENT: the sums are read at system scope (from past every cache).
template <bool COHERENT = false>
__device__ __forceinline__ void append_finish_pair(int32_t T_rows, int t, int cp, const float* __restrict__ part,
                                                   const AppendDst& a) {
  float v0[SK_SPLIT], v1[SK_SPLIT];
#pragma unroll
  for (int kc = 0; kc < SK_SPLIT; ++kc) {
    const float* src = part + ((int64_t)kc * T_rows + t) * D_K + 2 * cp;
    if (COHERENT) {
      v0[kc] = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      v1[kc] = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    } else {
      const float2 v = *(const float2*)src;
      v0[kc] = v.x;
      v1[kc] = v.y;
    }
  }
  float x0 = 0.f, x1 = 0.f;
#pragma unroll
  for (int kc = 0; kc < SK_SPLIT; ++kc) {
    x0 += v0[kc];
    x1 += v1[kc];
  }
  const int32_t sq = a.seq_id ? a.seq_id[t] : t;
  const int32_t p = a.pos[t];
  if (sq < 0 || sq >= a.num_seqs) {
    if (a.err_flag && (cp & 7) == 0) atomicOr(a.err_flag, MLA_FLAG_BAD_SEQ_ID);
    return;
  }
  if (p < 0 || p >= a.max_pages * a.page_size) {
    if (a.err_flag && (cp & 7) == 0) atomicOr(a.err_flag, MLA_FLAG_BAD_POSITION);
    return;
  }
  const int64_t row = pool_row(a.page_table, a.max_pages, a.num_pages, a.page_size, sq, p, a.err_flag);
  const int c = 2 * cp;
  bf16* dst;
  if (c >= D_C) {
    float cs, sn;
    rope_cos_sin(p, (c - D_C) / 2, a.rope, &cs, &sn);
    const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
    x0 = y0;
    x1 = y1;
    dst = a.k_R + row * a.row_stride + (c - D_C);
  } else {
    dst = a.c_KV + row * a.row_stride + c;
  }
  dst[0] = (bf16)x0;
  dst[1] = (bf16)x1;
}

// In-launch finish of tile (col_blk, tok_blk), called by each of its SK_SPLIT
// workgroups right after append_splitk_block<true>: every workgroup waits
// until its system-scope chunk-sum stores have completed and counts itself in
// with a device-scope atomic; the one that brings the count to SK_SPLIT adds
// the chunks (system-scope loads, so no cache can hold stale sums) and stores
// the tile's 32 tokens x 16 columns, then puts the counter back to zero for
// the next launch.  The counters start at zero.
__device__ __forceinline__ void append_splitk_finish_tile(int col_blk, int tok_blk, int32_t T_rows,
                                                          const float* part, int32_t* counters,
                                                          const AppendDst& a, int* lds_flag) {
  const int tid = threadIdx.x;
  __builtin_amdgcn_s_waitcnt(0);   // this thread's sum stores are complete
  __syncthreads();
  int32_t* cnt = counters + (int64_t)tok_blk * (D_K / 16) + col_blk;
  if (tid == 0)
    *lds_flag = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == SK_SPLIT - 1;
  __syncthreads();
  if (!*lds_flag) return;
  {
    const int r = tid >> 3, cp = tid & 7;   // 32 tokens x 8 column pairs
    const int t = tok_blk * SK_TOK + r;
    if (t < T_rows) append_finish_pair<true>(T_rows, t, col_blk * 8 + cp, part, a);
  }
  if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace mla
