// Weight-streaming projections around the decode attention:
//  * the query path, c^Q = W^DQ h, q^C = W^UQ c^Q, q^R = W^QR h
//    ("DeepSeek-V2：在“大力出奇迹”的AI军备竞赛中，四两拨千斤" (liang.world), ch.2 §2,
//    closing paragraph: the query gets its own low-rank compression c^Q;
//    "DeepSeek 系列模型技术深度解读" (tuntang.top), "RoPE 的兼容性处理": q_t =
//    [W^UQ c_t^Q ; W^QR h_t RoPE(t)]; q^R leaves here unrotated, the
//    absorption step rotates it at the query position);
//  * the output projection u = W^O [o_1; ...; o_{n_h}] (liang.world ch.2 §1,
//    the heads' outputs concatenated and multiplied by W_O).
// For bf16 both are the split-K skinny GEMM of gemm_splitk.h over packed
// weights (one launch per product, in-launch finish when split); products
// that share their input (W^DQ h and W^QR h) are one launch over the stacked
// weights, and c^Q leaves the first product already packed for the second.
// For fp32 a VALU kernel computes each output as one wave's dot product.
#include "gemm_splitk.h"

namespace mla {
namespace {

// Finished column pair (2cp, 2cp+1) of row m: stored to its segment's output.
template <typename YT>
__device__ __forceinline__ void gemm_store_pair(const GemmArgs& g, const GemmOut& o, int m, int cp, float x0,
                                                float x1) {
  const int n = 2 * cp;
  int beg;
  const int s = gemm_segment(g, n, &beg);
  void* Y = s == 0 ? o.Y[0] : s == 1 ? o.Y[1] : s == 2 ? o.Y[2] : o.Y[3];
  const int64_t ld = s == 0 ? o.ldy[0] : s == 1 ? o.ldy[1] : s == 2 ? o.ldy[2] : o.ldy[3];
  if constexpr (sizeof(YT) == 4) {
    *(float2*)((float*)Y + (int64_t)m * ld + (n - beg)) = float2{x0, x1};
  } else {
    // columns 2cp, 2cp+1 are neighbours in both layouts
    const int64_t off = ld >= 0 ? (int64_t)m * ld + (n - beg) : packed_index(m, n - beg, -ld);
    bf16x2 v;
    v[0] = (bf16)x0;
    v[1] = (bf16)x1;
    *(bf16x2*)((bf16*)Y + off) = v;
  }
}

// Grid: S * (N / 16) * ceil(M / (16 MT)) workgroups, the S chunks of a tile
// neighbours, then the column tiles, then the row blocks.
template <int MT, int XM, typename YT>
__global__ void __launch_bounds__(256) gemm_bf16_kernel(GemmArgs g, GemmOut o) {
  constexpr int KB = MT == 4 ? 4 : GK_KB;
  __shared__ float red[gk_red_floats(MT)];
  __shared__ int flag;
  const int nt = g.N / 16;
  const int bid = blockIdx.x;
  const int kc = bid % g.S, n_blk = (bid / g.S) % nt, m_blk = bid / (g.S * nt);
  auto epi = [&](int m, int cp, float x0, float x1) { gemm_store_pair<YT>(g, o, m, cp, x0, x1); };
  if (g.S == 1) {
    gemm_tile_direct<MT, XM, true, KB>(n_blk, m_blk, g, red, epi);
    return;
  }
  gemm_chunk<true, MT, XM, true, KB>(n_blk, kc, m_blk, g, red);
  gemm_finish_tile<MT>(n_blk, m_blk, g, epi, &flag);
}

// Wide workgroup for products with more than 16 rows: 16*NT columns x 16*MT
// rows (MT = 2 or 4, X packed), 4 waves over quarters of the K chunk.  Per
// K-step a wave loads MT activation and NT weight fragments (1 KB each) and
// runs MT*NT MFMAs, so that each activation fragment serves NT weight tiles
// (activation bytes per weight byte MT/NT instead of MT).  The four waves'
// sums are added in LDS in the order ((w3 + w2) + w1) + w0 into
// red[16MT][16NT + 1].
template <int MT, int NT, int KB, int XM>
__device__ __forceinline__ void gemm_accumulate_wide(int n_blk, int kc, int m_blk, const GemmArgs& g, float* red) {
  constexpr int LD = 16 * NT + 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n0 = n_blk * 16 * NT;
  const int K = g.K;
  int beg;
  const int seg = gemm_segment(g, n0, &beg);
  const int kchunk = K / g.S, kw = kchunk / 4, nks = kw / 32;
  const int64_t kbase = (int64_t)kc * kchunk + wave * kw;
  const int64_t tile = (int64_t)(K >> 5) * 512;   // elements from one 16-row block to the next
  const bf16* wp = gemm_weight(g, seg) + ((int64_t)((n0 - beg) >> 4) * (K >> 5) + (kbase >> 5)) * 512 + lane * 8;
  const bf16* xp = (const bf16*)g.X + ((int64_t)(m_blk * MT) * (K >> 5) + (kbase >> 5)) * 512 + lane * 8;
  // row-major X (bf16): lane reads row 16t + lane%16 (rows past M repeat row
  // M-1), columns 8*(lane/16) .. +7 of each 32-column K-step
  const bf16* xr[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
    xr[t] = (const bf16*)g.X + (int64_t)min(m_blk * 16 * MT + 16 * t + (lane & 15), g.M - 1) * g.ldx + kbase +
            8 * (lane >> 4);
  f32x4 acc[MT][NT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[t][c] = f32x4{0, 0, 0, 0};
  for (int b0 = 0; b0 < nks; b0 += KB) {
    bf16x8 wv[NT][KB], xv[MT][KB];
#pragma unroll
    for (int i = 0; i < KB; ++i)
      if (b0 + i < nks) {
#pragma unroll
        for (int c = 0; c < NT; ++c) wv[c][i] = *(const bf16x8*)(wp + c * tile + 512 * (b0 + i));
#pragma unroll
        for (int t = 0; t < MT; ++t)
          xv[t][i] = XM == GK_X_PACKED ? *(const bf16x8*)(xp + t * tile + 512 * (b0 + i))
                                       : *(const bf16x8*)(xr[t] + 32 * (b0 + i));
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
  for (int w = 3; w >= 0; --w) {
    if (wave == w) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float* p = red + (16 * t + 4 * (lane >> 4) + i) * LD + 16 * c + (lane & 15);
            *p = w == 3 ? acc[t][c][i] : acc[t][c][i] + *p;
          }
    }
    __syncthreads();
  }
}

// Grid: S * (N / (16 NT)) * ceil(M / (16 MT)) workgroups, ordered as for
// gemm_bf16_kernel.  S > 1: chunk sums to part (plain stores), added by
// gemm_finish_kernel in a second launch; measured on W^O at 64 rows (8
// chunks) this is 10% faster than the in-launch finish, whose every workgroup
// waits for its write-through stores.
template <int MT, int NT, int XM, typename YT>
__global__ void __launch_bounds__(256) gemm_wide_kernel(GemmArgs g, GemmOut o) {
  constexpr int ROWS = 16 * MT, COLS = 16 * NT, PAIRS = 8 * NT, LD = COLS + 1;
  __shared__ float red[ROWS * LD];
  const int ntw = g.N / COLS;
  const int bid = blockIdx.x, tid = threadIdx.x;
  const int kc = bid % g.S, n_blk = (bid / g.S) % ntw, m_blk = bid / (g.S * ntw);
  gemm_accumulate_wide<MT, NT, GW_KB, XM>(n_blk, kc, m_blk, g, red);
  if (g.S == 1) {
    for (int q = tid; q < ROWS * PAIRS; q += 256) {
      const int r = q / PAIRS, cp = q % PAIRS;
      const int m = m_blk * ROWS + r;
      if (m < g.M) gemm_store_pair<YT>(g, o, m, n_blk * PAIRS + cp, red[r * LD + 2 * cp], red[r * LD + 2 * cp + 1]);
    }
    return;
  }
  for (int q = tid; q < ROWS * COLS; q += 256) {
    const int r = q / COLS, c = q % COLS;
    const int m = m_blk * ROWS + r;
    if (m < g.M) g.part[((int64_t)kc * g.M + m) * g.N + n_blk * COLS + c] = red[r * LD + c];
  }
}

// Second launch of a split wide product: thread per output column pair; the
// S chunk sums added in the order kc = 0 .. S-1 (as in the in-launch finish).
template <typename YT>
__global__ void __launch_bounds__(256) gemm_finish_kernel(GemmArgs g, GemmOut o) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= (int64_t)g.M * (g.N / 2)) return;
  const int m = (int)(q / (g.N / 2)), cp = (int)(q % (g.N / 2));
  const float2 x = gemm_sum_pair<false>(m, cp, g);
  gemm_store_pair<YT>(g, o, m, cp, x.x, x.y);
}

// fp32: wave w of workgroup b computes output (m, n) = divmod(4b + w, N) from
// row-major X and packed W; the 64 lanes take every 64th k and the lane sums
// are added by a butterfly.
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmArgs g, GemmOut o) {
  const int lane = threadIdx.x & 63;
  const int64_t idx = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (idx >= (int64_t)g.M * g.N) return;
  const int m = (int)(idx / g.N), n = (int)(idx % g.N);
  int beg;
  const int s = gemm_segment(g, n, &beg);
  const float* w = (const float*)gemm_weight(g, s);
  const float* x = (const float*)g.X + (int64_t)m * g.ldx;
  float acc = 0.f;
  for (int k = lane; k < g.K; k += 64) acc = fmaf(x[k], w[packed_index(n - beg, k, g.K)], acc);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) {
    float* Y = (float*)(s == 0 ? o.Y[0] : s == 1 ? o.Y[1] : s == 2 ? o.Y[2] : o.Y[3]);
    const int64_t ld = s == 0 ? o.ldy[0] : s == 1 ? o.ldy[1] : s == 2 ? o.ldy[2] : o.ldy[3];
    Y[(int64_t)m * ld + (n - beg)] = acc;
  }
}

// One thread per 8-element lane chunk of the packed output: chunk q is lane
// q % 64 of block q / 64.
template <typename TI, typename TO>
__global__ void __launch_bounds__(256) pack_kernel(const TI* __restrict__ src, int64_t ld, int32_t rows,
                                                   int32_t K, int64_t n_chunks, TO* __restrict__ dst) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= n_chunks) return;
  const int64_t b = q >> 6;
  const int l = (int)(q & 63);
  const int64_t kb = K >> 5;
  const int64_t r = (b / kb) * 16 + (l & 15);
  const int64_t c = (b % kb) * 32 + (l >> 4) * 8;
  // 8 consecutive source elements (16 or 32 aligned bytes) -> 8 consecutive outputs
  typedef __attribute__((ext_vector_type(8))) TI vin_t;
  typedef __attribute__((ext_vector_type(8))) TO vout_t;
  vout_t v;
  if (r < rows) {
    const vin_t x = *(const vin_t*)(src + r * ld + c);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (TO)x[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (TO)0.f;
  }
  *(vout_t*)(dst + q * 8) = v;
}

template <int MT, int XM, typename YT>
void launch_bf16(const GemmArgs& g, const GemmOut& o, int64_t grid, hipStream_t s) {
  gemm_bf16_kernel<MT, XM, YT><<<dim3((unsigned)grid), 256, 0, s>>>(g, o);
}

template <int MT, typename YT>
void launch_wide(const GemmArgs& g, const GemmOut& o, int64_t grid, hipStream_t s) {
  bool rows = false;
  if constexpr (MT == 2) {
    rows = g.x_rows != 0;
    if (rows) gemm_wide_kernel<MT, GW_NT, GK_X_ROWS, YT><<<dim3((unsigned)grid), 256, 0, s>>>(g, o);
  }
  if (!rows) gemm_wide_kernel<MT, GW_NT, GK_X_PACKED, YT><<<dim3((unsigned)grid), 256, 0, s>>>(g, o);
  if (g.S > 1) {
    const int64_t pairs = (int64_t)g.M * (g.N / 2);
    gemm_finish_kernel<YT><<<dim3((unsigned)((pairs + 255) / 256)), 256, 0, s>>>(g, o);
  }
}

// One 16-row tile: narrow kernel, row-major activations up to GK_ROWS_MAX rows.
void launch_narrow(const GemmArgs& g, const GemmOut& o, int64_t grid, bool x_f32, bool y_f32, hipStream_t s) {
  static_assert(GK_ROWS_MAX <= 16, "row-major activations are instantiated for one 16-row tile");
  if (gemm_x_packed(g.M)) {
    if (y_f32) launch_bf16<1, GK_X_PACKED, float>(g, o, grid, s);
    else launch_bf16<1, GK_X_PACKED, bf16>(g, o, grid, s);
  } else if (y_f32 && x_f32) launch_bf16<1, GK_X_ROWS_F32, float>(g, o, grid, s);
  else if (y_f32) launch_bf16<1, GK_X_ROWS, float>(g, o, grid, s);
  else if (x_f32) launch_bf16<1, GK_X_ROWS_F32, bf16>(g, o, grid, s);
  else launch_bf16<1, GK_X_ROWS, bf16>(g, o, grid, s);
}

}  // namespace

int gemm_pick_splits(int32_t M, int32_t N, int32_t K) {
  const int mt = gemm_mt(M), nt = gemm_nt(M);
  // work in units of 16-column tiles
  const int64_t units = (int64_t)(N / (16 * nt)) * ((M + 16 * mt - 1) / (16 * mt)) * nt;
  if (units >= GK_UNSPLIT_TILES) return 1;
  const int64_t target = nt == 1 ? GK_TARGET_WG : 2 * GK_TARGET_WG;
  int S = 1;
  while (S < GK_S_MAX && units * S < target && K % (2 * S * 128) == 0) S *= 2;
  return S;
}

size_t gemm_part_bytes(int32_t M, int32_t N, int32_t S) { return S > 1 ? align256((size_t)S * M * N * 4) : 0; }

hipError_t launch_gemm(const GemmArgs& g, const GemmOut& o, bool f32_weights, bool x_f32, bool y_f32, hipStream_t s) {
  if (f32_weights) {
    const int64_t waves = (int64_t)g.M * g.N;
    if ((waves + 3) / 4 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    gemm_f32_kernel<<<dim3((unsigned)((waves + 3) / 4)), 256, 0, s>>>(g, o);
    return hipGetLastError();
  }
  const int mt = gemm_mt(g.M), nt = gemm_nt(g.M);
  const int cols = 16 * nt;
  for (int i = 0; i < GK_SEG; ++i)
    if (g.seg_end[i] % cols != 0) return hipErrorInvalidValue;
  const int64_t tiles = (int64_t)(g.N / cols) * ((g.M + 16 * mt - 1) / (16 * mt));
  if (g.N % cols != 0 || g.S < 1 || g.S > GK_S_MAX || g.K % (g.S * 128) != 0 ||
      (g.S > 1 && tiles > SPLITK_COUNTERS) || (mt > 1 && !gemm_x_packed(g.M)) ||
      (g.x_rows && (x_f32 || !gemm_x_rows_wide(g.M))))
    return hipErrorInvalidValue;
  const int64_t grid = (int64_t)g.S * tiles;
  if (mt == 1)
    launch_narrow(g, o, grid, x_f32, y_f32, s);
  else if (mt == 2)
    y_f32 ? launch_wide<2, float>(g, o, grid, s) : launch_wide<2, bf16>(g, o, grid, s);
  else
    y_f32 ? launch_wide<4, float>(g, o, grid, s) : launch_wide<4, bf16>(g, o, grid, s);
  return hipGetLastError();
}

hipError_t launch_pack(const void* src, int64_t ld, int32_t rows, int64_t rows_padded, int32_t K, bool src_f32,
                       bool to_bf16, void* dst, hipStream_t s) {
  if (rows_padded % 16 != 0 || K % 32 != 0 || rows > rows_padded) return hipErrorInvalidValue;
  const int64_t n_chunks = rows_padded * K / 8;
  const dim3 grid((unsigned)((n_chunks + 255) / 256));
  if (!src_f32)
    pack_kernel<bf16, bf16><<<grid, 256, 0, s>>>((const bf16*)src, ld, rows, K, n_chunks, (bf16*)dst);
  else if (to_bf16)
    pack_kernel<float, bf16><<<grid, 256, 0, s>>>((const float*)src, ld, rows, K, n_chunks, (bf16*)dst);
  else
    pack_kernel<float, float><<<grid, 256, 0, s>>>((const float*)src, ld, rows, K, n_chunks, (float*)dst);
  return hipGetLastError();
}

}  // namespace mla
