// Cache append: c^KV = W^DKV h_t and k^R = RoPE(W^KR h_t) written into the
// paged latent pool.
//   "DeepSeek-V2：在“大力出奇迹”的AI军备竞赛中，四两拨千斤" (liang.world), ch.2 §2:
//   c_t^KV = W^DKV h_t (d = 5120 -> d_c = 512); ch.2 §3: one decoupled key k^R_t
//   shared by all heads carries RoPE.  "DeepSeek 系列模型技术深度解读"
//   (tuntang.top), MLA section, "RoPE 的兼容性处理": k_t = [W^UK c_t^KV ;
//   W^KR h_t . RoPE(t)].  pptc.cn note §6 pitfall 2: k^R is cached beside c^KV.
//
// One launch handles T token rows.  The product [T x d_model] x [d_model x 576]
// is an MFMA GEMM (bf16 inputs, fp32 accumulation) for bf16 and a VALU GEMM for
// fp32; a decode step's few rows take the split-K variant at the end.  Workgroup tile: 32 tokens x 64 output columns; columns 0..511 come
// from W^DKV, 512..575 from W^KR (the ninth column tile is exactly k^R, so its
// RoPE pairs never straddle tiles).  The epilogue stages the fp32 tile in LDS,
// rotates the k^R pairs (angles in fp64), rounds to the cache type and writes
// each token's 64 columns (128 B for bf16) into its pool row.
#include "append_splitk.h"

namespace mla {
namespace {

constexpr int AT_TOK = 32;   // tokens per workgroup
constexpr int AT_COL = 64;   // output columns per workgroup
constexpr int AT_KC = 64;    // K chunk (d_model) per LDS stage, fp32 path

// Epilogue shared by both paths: res[tok][col] (fp32, in LDS) -> pool.
template <typename T>
__device__ void append_store(const float (*res)[AT_COL + 1], int32_t T_rows, int32_t tok0, int32_t col0,
                             const int32_t* __restrict__ seq_id, const int32_t* __restrict__ pos,
                             const int32_t* __restrict__ page_table, int32_t num_seqs, int32_t max_pages,
                             int32_t page_size, int32_t num_pages, T* __restrict__ c_KV, T* __restrict__ k_R,
                             int64_t row_stride, const RopeTab& rope, int32_t* err_flag) {
  const int tid = threadIdx.x;
  // 256 threads: 8 tokens at a time, 32 threads per token, 2 columns per thread.
  const int tt = tid >> 5, cp = tid & 31;
  const int max_tok = max_pages * page_size;
  for (int r = tt; r < AT_TOK; r += 8) {
    const int t = tok0 + r;
    if (t >= T_rows) break;
    const int32_t sq = seq_id ? seq_id[t] : t;
    const int32_t p = pos[t];
    if (sq < 0 || sq >= num_seqs) {
      if (cp == 0 && err_flag) atomicOr(err_flag, MLA_FLAG_BAD_SEQ_ID);
      continue;
    }
    if (p < 0 || p >= max_tok) {
      if (cp == 0 && err_flag) atomicOr(err_flag, MLA_FLAG_BAD_POSITION);
      continue;
    }
    const int64_t row = pool_row(page_table, max_pages, num_pages, page_size, sq, p, err_flag);
    float x0 = res[r][2 * cp], x1 = res[r][2 * cp + 1];
    if (col0 >= D_C) {
      // k^R pair k = cp: rotate by pos * base^(-2k/64)
      float cs, sn;
      rope_cos_sin(p, cp, rope, &cs, &sn);
      const float y0 = x0 * cs - x1 * sn;
      const float y1 = x0 * sn + x1 * cs;
      x0 = y0;
      x1 = y1;
      T* dst = k_R + row * row_stride + (col0 - D_C) + 2 * cp;
      dst[0] = from_f32<T>(x0);
      dst[1] = from_f32<T>(x1);
    } else {
      T* dst = c_KV + row * row_stride + col0 + 2 * cp;
      dst[0] = from_f32<T>(x0);
      dst[1] = from_f32<T>(x1);
    }
  }
}

// ---------------------------------------------------------------- fp32 (VALU)
__global__ void __launch_bounds__(256) append_f32_kernel(
    int32_t T_rows, int32_t d_model, const float* __restrict__ h, const float* __restrict__ W_DKV,
    const float* __restrict__ W_KR, const int32_t* __restrict__ seq_id, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ page_table, int32_t num_seqs, int32_t max_pages, int32_t page_size,
    float* __restrict__ c_KV, float* __restrict__ k_R, int64_t row_stride, int32_t num_pages, RopeTab rope,
    int32_t* err_flag) {
  __shared__ float hs[AT_TOK][AT_KC + 1];
  __shared__ float ws[AT_COL][AT_KC + 1];
  __shared__ float res[AT_TOK][AT_COL + 1];
  const int tid = threadIdx.x;
  const int tok0 = blockIdx.x * AT_TOK;
  const int col0 = blockIdx.y * AT_COL;
  const float* W = col0 < D_C ? W_DKV + (int64_t)col0 * d_model : W_KR + (int64_t)(col0 - D_C) * d_model;
  // thread -> 2 tokens x 4 columns
  const int tp = tid >> 4, cg = tid & 15;
  float acc[2][4] = {};
  for (int k0 = 0; k0 < d_model; k0 += AT_KC) {
    for (int i = tid; i < AT_TOK * AT_KC; i += 256) {
      const int r = i / AT_KC, c = i % AT_KC;
      const int t = tok0 + r;
      hs[r][c] = t < T_rows ? h[(int64_t)t * d_model + k0 + c] : 0.f;
    }
    for (int i = tid; i < AT_COL * AT_KC; i += 256) {
      const int r = i / AT_KC, c = i % AT_KC;
      ws[r][c] = W[(int64_t)r * d_model + k0 + c];
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < AT_KC; ++k) {
      const float a0 = hs[2 * tp][k], a1 = hs[2 * tp + 1][k];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float w = ws[cg + 16 * j][k];
        acc[0][j] = fmaf(a0, w, acc[0][j]);
        acc[1][j] = fmaf(a1, w, acc[1][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    res[2 * tp][cg + 16 * j] = acc[0][j];
    res[2 * tp + 1][cg + 16 * j] = acc[1][j];
  }
  __syncthreads();
  append_store<float>(res, T_rows, tok0, col0, seq_id, pos, page_table, num_seqs, max_pages, page_size,
                      num_pages, c_KV, k_R, row_stride, rope, err_flag);
}

// ---------------------------------------------------------------- bf16 (MFMA)
// 4 waves; wave w owns output columns col0 + 16w .. +15 of the 64-column tile
// for all 32 tokens, as two 16x16 blocks (tokens 0-15, 16-31), accumulating
// v_mfma_f32_16x16x32_bf16 over d_model.  Operands are read straight from
// global memory in the MFMA lane layout (lane l: row l%16, 8 consecutive K
// elements at 8*(l/16)), 16 B per lane.
__global__ void __launch_bounds__(256) append_bf16_kernel(
    int32_t T_rows, int32_t d_model, const bf16* __restrict__ h, const bf16* __restrict__ W_DKV,
    const bf16* __restrict__ W_KR, const int32_t* __restrict__ seq_id, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ page_table, int32_t num_seqs, int32_t max_pages, int32_t page_size,
    bf16* __restrict__ c_KV, bf16* __restrict__ k_R, int64_t row_stride, int32_t num_pages, RopeTab rope,
    int32_t* err_flag) {
  __shared__ float res[AT_TOK][AT_COL + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int tok0 = blockIdx.x * AT_TOK;
  const int col0 = blockIdx.y * AT_COL;
  const bf16* W = col0 < D_C ? W_DKV + (int64_t)col0 * d_model : W_KR + (int64_t)(col0 - D_C) * d_model;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  // B operand: W rows (output columns) 16w + r16; A operand: h rows (tokens).
  const bf16* wrow = W + (int64_t)(16 * wave + r16) * d_model + kq;
  const int t_a = min(tok0 + r16, T_rows - 1), t_b = min(tok0 + 16 + r16, T_rows - 1);
  const bf16* ha = h + (int64_t)t_a * d_model + kq;
  const bf16* hb = h + (int64_t)t_b * d_model + kq;
  f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0}, acc2 = {0, 0, 0, 0}, acc3 = {0, 0, 0, 0};
  int k = 0;
  for (; k + 64 <= d_model; k += 64) {
    const bf16x8 w0 = *(const bf16x8*)(wrow + k), w1 = *(const bf16x8*)(wrow + k + 32);
    const bf16x8 a0 = *(const bf16x8*)(ha + k), a1 = *(const bf16x8*)(ha + k + 32);
    const bf16x8 b0 = *(const bf16x8*)(hb + k), b1 = *(const bf16x8*)(hb + k + 32);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, w0, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0, w0, acc1, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, w1, acc2, 0, 0, 0);
    acc3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1, w1, acc3, 0, 0, 0);
  }
  for (; k < d_model; k += 32) {
    const bf16x8 w0 = *(const bf16x8*)(wrow + k);
    const bf16x8 a0 = *(const bf16x8*)(ha + k);
    const bf16x8 b0 = *(const bf16x8*)(hb + k);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, w0, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0, w0, acc1, 0, 0, 0);
  }
  // C layout (16x16): lane l holds column l%16 (here: output column) and
  // rows 4*(l/16) + i (here: tokens).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tr = 4 * (lane >> 4) + i;
    res[tr][16 * wave + r16] = acc0[i] + acc2[i];
    res[16 + tr][16 * wave + r16] = acc1[i] + acc3[i];
  }
  __syncthreads();
  append_store<bf16>(res, T_rows, tok0, col0, seq_id, pos, page_table, num_seqs, max_pages, page_size,
                     num_pages, c_KV, k_R, row_stride, rope, err_flag);
}

// Few tokens (a decode step): the product is weight-bandwidth bound, so the
// grid is spread over output columns.  Workgroup = 16 tokens x 16 output
// columns, 16 waves; wave w takes the w-th sixteenth of d_model and issues all
// of its operand loads (v_mfma_f32_16x16x32_bf16 fragments straight from
// global memory, up to SMALL_KB K-steps per batch) before its MFMAs, so one
// memory latency covers its slice; the 16 partial sums are added in LDS.
constexpr int SMALL_W = 16;
constexpr int SMALL_KB = 10;

__global__ void __launch_bounds__(64 * SMALL_W) append_bf16_small_kernel(
    int32_t T_rows, int32_t d_model, const bf16* __restrict__ h, const bf16* __restrict__ W_DKV,
    const bf16* __restrict__ W_KR, const int32_t* __restrict__ seq_id, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ page_table, int32_t num_seqs, int32_t max_pages, int32_t page_size,
    bf16* __restrict__ c_KV, bf16* __restrict__ k_R, int64_t row_stride, int32_t num_pages, RopeTab rope,
    int32_t* err_flag) {
  __shared__ float red[SMALL_W][16][17];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int tok0 = blockIdx.x * 16;
  const int col0 = blockIdx.y * 16;
  const bf16* W = col0 < D_C ? W_DKV + (int64_t)col0 * d_model : W_KR + (int64_t)(col0 - D_C) * d_model;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int kw = d_model / SMALL_W;                // K range of this wave (a multiple of 32)
  const int nks = kw / 32;
  const bf16* wrow = W + (int64_t)r16 * d_model + wave * kw + kq;
  const bf16* hrow = h + (int64_t)min(tok0 + r16, T_rows - 1) * d_model + wave * kw + kq;
  f32x4 acc = {0, 0, 0, 0};
  for (int k0 = 0; k0 < nks; k0 += SMALL_KB) {
    bf16x8 wv[SMALL_KB], hv[SMALL_KB];
#pragma unroll
    for (int i = 0; i < SMALL_KB; ++i)
      if (k0 + i < nks) {
        wv[i] = *(const bf16x8*)(wrow + 32 * (k0 + i));
        hv[i] = *(const bf16x8*)(hrow + 32 * (k0 + i));
      }
#pragma unroll
    for (int i = 0; i < SMALL_KB; ++i)
      if (k0 + i < nks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hv[i], wv[i], acc, 0, 0, 0);
  }
  // C layout: lane holds output column lane%16, tokens 4*(lane/16) + i
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][4 * (lane >> 4) + i][r16] = acc[i];
  __syncthreads();
  if (tid < 128) {
    const int r = tid >> 3, cp = tid & 7;          // token row, column pair
    const int t = tok0 + r;
    if (t < T_rows) {
      float x0 = 0.f, x1 = 0.f;
#pragma unroll
      for (int w = 0; w < SMALL_W; ++w) {
        x0 += red[w][r][2 * cp];
        x1 += red[w][r][2 * cp + 1];
      }
      const int32_t sq = seq_id ? seq_id[t] : t;
      const int32_t p = pos[t];
      if (sq < 0 || sq >= num_seqs) {
        if (err_flag) atomicOr(err_flag, MLA_FLAG_BAD_SEQ_ID);
      } else if (p < 0 || p >= max_pages * page_size) {
        if (err_flag) atomicOr(err_flag, MLA_FLAG_BAD_POSITION);
      } else {
        const int64_t row = pool_row(page_table, max_pages, num_pages, page_size, sq, p, err_flag);
        const int c = col0 + 2 * cp;
        bf16* dst;
        if (c >= D_C) {
          float cs, sn;
          rope_cos_sin(p, (c - D_C) / 2, rope, &cs, &sn);
          const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
          x0 = y0;
          x1 = y1;
          dst = k_R + row * row_stride + (c - D_C);
        } else {
          dst = c_KV + row * row_stride + c;
        }
        dst[0] = (bf16)x0;
        dst[1] = (bf16)x1;
      }
    }
  }
}

// Decode-step append with a workspace: split over d_model (append_splitk.h),
// chunk sums in the workspace, then one pass that adds them in a fixed order,
// applies RoPE and stores the rows (deterministic, no float atomics).
template <int MT>
__global__ void __launch_bounds__(256) append_splitk_kernel(int32_t T_rows, int32_t d_model,
                                                            const bf16* __restrict__ h,
                                                            const bf16* __restrict__ W_DKV,
                                                            const bf16* __restrict__ W_KR, float* __restrict__ part) {
  __shared__ float red[gk_red_floats(MT)];
  append_splitk_block<false, MT>(blockIdx.x, blockIdx.y, blockIdx.z, T_rows, d_model, h, W_DKV, W_KR, part, red);
}

// Wide form of the chunk sums for long row batches (T >= APPEND_WIDE_MIN_T,
// prefill chunks): workgroup (64 output columns, chunk kc, 64 rows), 4 waves
// over quarters of the chunk.  Per K-step a wave loads 4 activation and 4
// weight fragments and runs 16 MFMAs, so each activation fragment serves 4
// column tiles where append_splitk_kernel's 16-column workgroups load it once
// per tile (activation traffic / 4).  Each wave's sums are those of
// append_splitk_block (same fragments, same K-steps in the same order, A =
// activations, B = weights), and the waves are added as (w0 + w1) + (w2 +
// w3), so the chunk sums and the rows append_finish_kernel stores from them
// are bitwise those of the 16-column form, and of the decode step's append.
__global__ void __launch_bounds__(256) append_wide_kernel(int32_t T_rows, int32_t d_model, const bf16* __restrict__ h,
                                                          const bf16* __restrict__ W_DKV,
                                                          const bf16* __restrict__ W_KR, float* __restrict__ part) {
  constexpr int MT = 4, NT = AW_NT, ROWS = 16 * MT, COLS = 16 * NT, LD = COLS + 1, KB = 2;
  __shared__ float red[2][ROWS * LD];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n0 = blockIdx.x * COLS, kc = blockIdx.y, m0 = blockIdx.z * ROWS;
  const int K = d_model, kchunk = K / SK_SPLIT, kw = kchunk / 4, nks = kw / 32;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int64_t kbase = (int64_t)kc * kchunk + wave * kw;   // this wave's first k
  // columns n0 .. n0+63 lie in one weight (D_C is a multiple of 64)
  const bf16* W = n0 < D_C ? W_DKV + (int64_t)n0 * K : W_KR + (int64_t)(n0 - D_C) * K;
  const bf16* wp = W + (int64_t)r16 * K + kbase + kq;   // tile c at + 16 c K
  const bf16* xp[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t)   // rows past T repeat row T-1
    xp[t] = h + (int64_t)min(m0 + 16 * t + r16, T_rows - 1) * d_model + kbase + kq;
  f32x4 acc[MT][NT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int b0 = 0; b0 < nks; b0 += KB) {
    bf16x8 wv[NT][KB], xv[MT][KB];
#pragma unroll
    for (int i = 0; i < KB; ++i)
      if (b0 + i < nks) {
#pragma unroll
        for (int c = 0; c < NT; ++c) wv[c][i] = *(const bf16x8*)(wp + (int64_t)16 * c * K + 32 * (b0 + i));
#pragma unroll
        for (int t = 0; t < MT; ++t) xv[t][i] = *(const bf16x8*)(xp[t] + 32 * (b0 + i));
      }
#pragma unroll
    for (int i = 0; i < KB; ++i)
      if (b0 + i < nks) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int c = 0; c < NT; ++c)
            acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv[t][i], wv[c][i], acc[t][c], 0, 0, 0);
      }
  }
  // C layout: lane holds column 16c + lane%16, rows 16t + 4*(lane/16) + i
  auto slot = [&](int buf, int t, int c, int i) -> float& {
    return red[buf][(16 * t + 4 * (lane >> 4) + i) * LD + 16 * c + r16];
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) slot(buf, t, c, i) = acc[t][c][i];
  };
  auto add = [&](int buf) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][c][i] = acc[t][c][i] + slot(buf, t, c, i);
  };
  if (wave == 1) put(0);
  if (wave == 3) put(1);
  __syncthreads();
  if (wave == 0) add(0);   // w0 + w1
  if (wave == 2) add(1);   // w2 + w3
  __syncthreads();
  if (wave == 2) put(1);
  __syncthreads();
  if (wave == 0) {
    add(1);                // (w0 + w1) + (w2 + w3)
    put(0);
  }
  __syncthreads();
  // part[kc][m][576]: 64 columns of 4 rows per pass
  const int col = tid & 63;
#pragma unroll
  for (int j = 0; j < ROWS / 4; ++j) {
    const int r = 4 * j + (tid >> 6);
    const int m = m0 + r;
    if (m < T_rows) part[((int64_t)kc * T_rows + m) * D_K + n0 + col] = red[0][r * LD + col];
  }
}

__global__ void __launch_bounds__(256) append_finish_kernel(int32_t T_rows, int32_t d_model,
                                                            const float* __restrict__ part, AppendDst a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int t = (int)(idx / (D_K / 2)), cp = (int)(idx % (D_K / 2));
  if (t < T_rows) append_finish_pair(T_rows, d_model, t, cp, part, a);
}

}  // namespace

size_t append_workspace_bytes(const mla_dims& d, int32_t T) {
  if (d.dtype != MLA_BF16 || T > APPEND_WS_MAX_T || d.d_model % (SK_SPLIT * 4 * 32) != 0) return 0;
  return (size_t)SK_SPLIT * T * D_K * sizeof(float);
}

hipError_t launch_append(const mla_dims& d, int32_t T, const void* h, const void* W_DKV, const void* W_KR,
                         const int32_t* seq_id, const int32_t* pos, const int32_t* page_table,
                         int32_t num_seqs, int32_t max_pages, void* c_KV, void* k_R, int64_t row_stride,
                         int32_t num_pages, int32_t* err_flag, void* ws, size_t ws_bytes, hipStream_t s) {
  const size_t need = append_workspace_bytes(d, T);
  if (ws && need > 0 && ws_bytes >= need) {
    const int rows = 16 * append_mt(T);
    dim3 g1(D_K / 16, SK_SPLIT, (T + rows - 1) / rows);
    if (T >= APPEND_WIDE_MIN_T)
      append_wide_kernel<<<dim3(D_K / (16 * AW_NT), SK_SPLIT, (T + 63) / 64), 256, 0, s>>>(
          T, d.d_model, (const bf16*)h, (const bf16*)W_DKV, (const bf16*)W_KR, (float*)ws);
    else if (append_mt(T) == 4)
      append_splitk_kernel<4><<<g1, 256, 0, s>>>(T, d.d_model, (const bf16*)h, (const bf16*)W_DKV,
                                                (const bf16*)W_KR, (float*)ws);
    else
      append_splitk_kernel<2><<<g1, 256, 0, s>>>(T, d.d_model, (const bf16*)h, (const bf16*)W_DKV,
                                                (const bf16*)W_KR, (float*)ws);
    const int64_t n = (int64_t)T * (D_K / 2);
    const AppendDst a{seq_id, pos, page_table, num_seqs, max_pages, d.page_size, num_pages, (bf16*)c_KV,
                      (bf16*)k_R, row_stride, rope_table(d.rope_base), err_flag};
    append_finish_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(T, d.d_model, (const float*)ws, a);
    return hipGetLastError();
  }
  dim3 grid((T + AT_TOK - 1) / AT_TOK, D_K / AT_COL);
  if (d.dtype == MLA_FP32) {
    append_f32_kernel<<<grid, 256, 0, s>>>(T, d.d_model, (const float*)h, (const float*)W_DKV,
                                          (const float*)W_KR, seq_id, pos, page_table, num_seqs, max_pages,
                                          d.page_size, (float*)c_KV, (float*)k_R, row_stride, num_pages,
                                          rope_table(d.rope_base), err_flag);
  } else if (T <= 512 && d.d_model % (32 * SMALL_W) == 0) {
    dim3 g2((T + 15) / 16, D_K / 16);
    append_bf16_small_kernel<<<g2, 64 * SMALL_W, 0, s>>>(T, d.d_model, (const bf16*)h, (const bf16*)W_DKV,
                                                 (const bf16*)W_KR, seq_id, pos, page_table, num_seqs, max_pages,
                                                 d.page_size, (bf16*)c_KV, (bf16*)k_R, row_stride, num_pages,
                                                 rope_table(d.rope_base), err_flag);
  } else {
    append_bf16_kernel<<<grid, 256, 0, s>>>(T, d.d_model, (const bf16*)h, (const bf16*)W_DKV,
                                           (const bf16*)W_KR, seq_id, pos, page_table, num_seqs, max_pages,
                                           d.page_size, (bf16*)c_KV, (bf16*)k_R, row_stride, num_pages,
                                           rope_table(d.rope_base), err_flag);
  }
  return hipGetLastError();
}

}  // namespace mla
