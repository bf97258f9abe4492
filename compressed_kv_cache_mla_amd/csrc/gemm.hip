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

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

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
  TO v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = r < rows ? (TO)src[r * ld + c + i] : (TO)0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) dst[q * 8 + i] = v[i];
}

template <int MT, int XM, typename YT>
void launch_bf16(const GemmArgs& g, const GemmOut& o, int64_t grid, hipStream_t s) {
  gemm_bf16_kernel<MT, XM, YT><<<dim3((unsigned)grid), 256, 0, s>>>(g, o);
}

// Row-major activations only occur with at most GK_ROWS_MAX rows, i.e. MT = 1.
template <int MT>
void launch_mt(const GemmArgs& g, const GemmOut& o, int64_t grid, bool x_f32, bool y_f32, hipStream_t s) {
  static_assert(GK_ROWS_MAX <= 16, "row-major activations are instantiated for one 16-row tile");
  const bool packed = gemm_x_packed(g.M);
  if constexpr (MT == 1) {
    if (!packed) {
      if (y_f32 && x_f32) launch_bf16<1, GK_X_ROWS_F32, float>(g, o, grid, s);
      else if (y_f32) launch_bf16<1, GK_X_ROWS, float>(g, o, grid, s);
      else if (x_f32) launch_bf16<1, GK_X_ROWS_F32, bf16>(g, o, grid, s);
      else launch_bf16<1, GK_X_ROWS, bf16>(g, o, grid, s);
      return;
    }
  }
  if (y_f32)
    launch_bf16<MT, GK_X_PACKED, float>(g, o, grid, s);
  else
    launch_bf16<MT, GK_X_PACKED, bf16>(g, o, grid, s);
}

}  // namespace

int gemm_pick_splits(int32_t M, int32_t N, int32_t K) {
  const int rows = 16 * gemm_mt(M);
  const int64_t tiles = (int64_t)(N / 16) * ((M + rows - 1) / rows);
  if (tiles >= GK_UNSPLIT_TILES) return 1;
  int S = 1;
  while (S < GK_S_MAX && tiles * S < GK_TARGET_WG && K % (2 * S * 128) == 0) S *= 2;
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
  const int mt = gemm_mt(g.M);
  const int64_t tiles = (int64_t)(g.N / 16) * ((g.M + 16 * mt - 1) / (16 * mt));
  if (g.S < 1 || g.S > GK_S_MAX || g.K % (g.S * 128) != 0 || (g.S > 1 && tiles > SPLITK_COUNTERS))
    return hipErrorInvalidValue;
  const int64_t grid = (int64_t)g.S * tiles;
  if (mt == 1)
    launch_mt<1>(g, o, grid, x_f32, y_f32, s);
  else if (mt == 2)
    launch_mt<2>(g, o, grid, x_f32, y_f32, s);
  else
    launch_mt<4>(g, o, grid, x_f32, y_f32, s);
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
