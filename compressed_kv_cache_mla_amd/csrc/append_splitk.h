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

#include "gemm_splitk.h"

namespace mla {

constexpr int SK_SPLIT = APPEND_SK_SPLIT;   // d_model chunks
constexpr int SK_TOK = GK_TOK;              // tokens per workgroup up to 32 tokens
constexpr int SK_RED_FLOATS = GK_RED_FLOATS;
// Token rows per workgroup: 32 (MT = 2) up to 32 tokens, 64 (MT = 4) above,
// so that a 33..64-token batch reads the weights once.
inline int append_mt(int32_t T) { return T > 32 ? 4 : 2; }
// From this many rows the two-launch append computes its chunk sums in 64 x 64
// tiles (append_wide_kernel, append.hip), 16-column tiles below.
constexpr int APPEND_WIDE_MIN_T = 256;
constexpr int AW_NT = 4;   // 16-column tiles per workgroup of the wide form
static_assert(D_C % (16 * AW_NT) == 0 && D_K % (16 * AW_NT) == 0, "wide append tiles");
// K-steps per load batch for MT row tiles (the 64-row form keeps its loads
// within the fused step's register budget).
__host__ __device__ constexpr int append_kb(int MT) { return MT == 4 ? 2 : GK_KB; }

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

// The append as a split-K product: X = h [T, d_model], W = [W^DKV ; W^KR]
// (576 output columns, k^R from column 512 on).
__device__ __forceinline__ GemmArgs append_gemm(int32_t T_rows, int32_t d_model, const bf16* h, const bf16* W_DKV,
                                                const bf16* W_KR, float* part, int32_t* counters) {
  GemmArgs g;
  g.x_rows = 0;
  g.X = h;
  g.ldx = d_model;
  g.W[0] = W_DKV;
  g.W[1] = W_KR;
  g.W[2] = g.W[3] = nullptr;
  g.seg_end[0] = D_C;
  g.seg_end[1] = g.seg_end[2] = g.seg_end[3] = D_K;
  g.M = T_rows;
  g.N = D_K;
  g.K = d_model;
  g.S = SK_SPLIT;
  g.part = part;
  g.counters = counters;
  return g;
}

// Chunk sums of workgroup (col_blk, kc, tok_blk) of 16*MT token rows; red:
// gk_red_floats(MT) floats of LDS.
template <bool COHERENT = false, int MT = 2>
__device__ __forceinline__ void append_splitk_block(int col_blk, int kc, int tok_blk, int32_t T_rows,
                                                    int32_t d_model, const bf16* __restrict__ h,
                                                    const bf16* __restrict__ W_DKV, const bf16* __restrict__ W_KR,
                                                    float* __restrict__ part, float* red) {
  gemm_chunk<COHERENT, MT, GK_X_ROWS, false, append_kb(MT)>(
      col_blk, kc, tok_blk, append_gemm(T_rows, d_model, h, W_DKV, W_KR, part, nullptr), red);
}

// Store of a finished column pair (columns 2cp, 2cp+1) of token t: RoPE on
// k^R pairs, rounded to bf16, into the token's pool row.
__device__ __forceinline__ void append_store_pair(int t, int cp, float x0, float x1, const AppendDst& a) {
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

// Final value of column pair cp of token t from the chunk sums (second launch).
__device__ __forceinline__ void append_finish_pair(int32_t T_rows, int32_t d_model, int t, int cp,
                                                   const float* __restrict__ part, const AppendDst& a) {
  const GemmArgs g = append_gemm(T_rows, d_model, nullptr, nullptr, nullptr, (float*)part, nullptr);
  const float2 x = gemm_sum_pair<false>(t, cp, g);
  append_store_pair(t, cp, x.x, x.y, a);
}

// In-launch finish of tile (col_blk, tok_blk) by the last of its SK_SPLIT
// workgroups (gemm_finish_tile), right after append_splitk_block<true>.
template <int MT = 2>
__device__ __forceinline__ void append_splitk_finish_tile(int col_blk, int tok_blk, int32_t T_rows, int32_t d_model,
                                                          float* part, int32_t* counters, const AppendDst& a,
                                                          int* lds_flag) {
  const GemmArgs g = append_gemm(T_rows, d_model, nullptr, nullptr, nullptr, part, counters);
  gemm_finish_tile<MT>(col_blk, tok_blk, g,
                       [&](int m, int cp, float x0, float x1) { append_store_pair(m, cp, x0, x1, a); }, lds_flag);
}

}  // namespace mla
