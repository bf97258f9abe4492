// Skinny GEMM for a decode step's few rows: Y[M, N] = X[M, K] . W[N, K]^T
// with bf16 weights, bf16 (or fp32, rounded to bf16 as loaded) activations
// and fp32 accumulation, as device functions shared by the cache append
// (append_splitk.h), the query projection and the output projection
// (gemm.hip).
//
// Decode-step products have M <= 64 rows and weights of MBs to 100s of MBs,
// so they are bound by the weight stream.  The product is split over K into
// S chunks so that every compute unit streams a share of W: workgroup
// (16 output columns, chunk kc, 16*MT rows), 4 waves (quarters of the
// chunk, every operand load of a batch issued before its MFMAs,
// v_mfma_f32_16x16x32_bf16 with A = 16 rows of X, B = 16 rows of W).  With
// S = 1 the workgroup's sums are final and go straight to an epilogue.
// Otherwise the chunk sums go to part[kc][m][N] in fp32 and the S chunks of an
// output element are added in the fixed order kc = 0 .. S-1 and handed to the
// epilogue, either by a second launch over all elements or, in the same
// launch, by the last of the S workgroups of a (column, row) tile to finish,
// found with a counter.  Both orders of events give the same bits.
//
// Operand layouts.  ROWS: row-major with a row stride.  PACKED: the matrix
// cut into blocks of 16 rows x 32 columns, block (rb, ks) stored at element
// ((rb * K/32) + ks) * 512 in the lane order of the MFMA operand -- lane l's 8
// elements (row 16rb + l%16, columns 32ks + 8(l/16) .. +7) at l*8 -- so that
// one wave reads a block as one contiguous 1 KB run.  Row-major loads of an
// MFMA operand touch 16 rows x 64 B per instruction; packed loads read whole
// cache lines, which roughly doubles the stream a compute unit sustains.
// Weights are packed once (mla_pack_weight); activations with more than a
// few rows are packed per call (rows padded to a multiple of 64).
//
// W may be up to GK_SEG matrices stacked by rows (the cache append's W^DKV and
// W^KR; the query's W^DQ and W^QR): output columns [seg_end[s-1], seg_end[s])
// come from W[s].  Segment sizes are multiples of 16, so a tile never
// straddles two.
#pragma once

#include "mla_common.h"

namespace mla {

constexpr int GK_TOK = 32;                  // rows of X per workgroup of the cache append (MT = 2)
constexpr int GK_KB = 5;                    // K-steps of operand loads issued per batch
constexpr int GK_SEG = 4;                   // most stacked weight matrices
constexpr int GK_S_MAX = 16;                // most K chunks of one product
constexpr int64_t GK_TARGET_WG = 1024;      // workgroups that fill the GPU: 4 per CU of 256
// Products with at least this many tiles (two per CU) are not split: the
// chunk sums and the in-launch finish cost more than the finer balance gains
// (measured on the query products, 608 and 1024 tiles).
constexpr int64_t GK_UNSPLIT_TILES = 512;
// LDS of the cross-wave reduction for 16*MT rows
__host__ __device__ constexpr int gk_red_floats(int MT) { return 4 * 16 * MT * 17; }
constexpr int GK_RED_FLOATS = gk_red_floats(2);

// Activation operand modes.
enum { GK_X_ROWS = 0, GK_X_ROWS_F32 = 1, GK_X_PACKED = 2 };

// Element offset of (r, c) in the packed layout of a matrix with K columns.
__host__ __device__ __forceinline__ int64_t packed_index(int64_t r, int64_t c, int64_t K) {
  return ((r >> 4) * (K >> 5) + (c >> 5)) * 512 + ((c & 31) >> 3) * 128 + (r & 15) * 8 + (c & 7);
}

struct GemmArgs {
  const void* X;      // ROWS: [M, K] bf16 / fp32, row stride ldx; PACKED: bf16, rows padded to 64
  int64_t ldx;
  const bf16* W[GK_SEG];      // segment s: [seg_end[s] - seg_end[s-1], K], row-major or packed
  int32_t seg_end[GK_SEG];    // cumulative column ends; unused segments end at N
  int32_t M, N, K;
  int32_t S;          // K chunks, <= GK_S_MAX; K % (S * 128) == 0
  float* part;        // [S, M, N] fp32 chunk sums (S > 1)
  int32_t* counters;  // [ceil(M / (16 MT)), N / 16], zero before the first in-launch finish
  int32_t x_rows;     // wide kernel: bf16 X read row-major (row stride ldx) although M > 8
};

// Segment of output column n: its first column and its weight matrix.
__device__ __forceinline__ int gemm_segment(const GemmArgs& g, int n, int* beg) {
  int s = 0, b = 0;
  if (n >= g.seg_end[0]) { s = 1; b = g.seg_end[0]; }
  if (n >= g.seg_end[1]) { s = 2; b = g.seg_end[1]; }
  if (n >= g.seg_end[2]) { s = 3; b = g.seg_end[2]; }
  *beg = b;
  return s;
}

__device__ __forceinline__ const bf16* gemm_weight(const GemmArgs& g, int s) {
  return s == 0 ? g.W[0] : s == 1 ? g.W[1] : s == 2 ? g.W[2] : g.W[3];
}

// 8 consecutive activations as MFMA operand (fp32 rounded to nearest even).
template <bool XF32>
struct XFrag;
template <>
struct XFrag<false> {
  bf16x8 v;
  __device__ __forceinline__ void load(const void* p) { v = *(const bf16x8*)p; }
  __device__ __forceinline__ bf16x8 get() const { return v; }
};
template <>
struct XFrag<true> {
  f32x4 lo, hi;
  __device__ __forceinline__ void load(const void* p) {
    lo = ((const f32x4*)p)[0];
    hi = ((const f32x4*)p)[1];
  }
  __device__ __forceinline__ bf16x8 get() const {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = (bf16)lo[i];
      r[4 + i] = (bf16)hi[i];
    }
    return r;
  }
};

// Products of workgroup (n_blk, kc, m_blk) over rows 16*MT*m_blk .. +16*MT-1,
// left per wave in red (gk_red_floats(MT) floats of LDS):
// red[(wave * 16MT + row) * 17 + column].  KB: K-steps per load batch.
template <int MT, int XM, bool WPACKED, int KB = GK_KB>
__device__ __forceinline__ void gemm_accumulate(int n_blk, int kc, int m_blk, const GemmArgs& g, float* red) {
  constexpr bool XF32 = XM == GK_X_ROWS_F32;
  constexpr int XB = XF32 ? 4 : 2;
  constexpr int ROWS = 16 * MT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n0 = n_blk * 16, m0 = m_blk * ROWS;
  const int K = g.K;
  int beg;
  const int seg = gemm_segment(g, n0, &beg);
  const int kchunk = K / g.S, kw = kchunk / 4, nks = kw / 32;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int64_t kbase = (int64_t)kc * kchunk + wave * kw;   // this wave's first k
  const bf16* wp;
  int wstep;
  if (WPACKED) {
    wp = gemm_weight(g, seg) + ((int64_t)((n0 - beg) >> 4) * (K >> 5) + (kbase >> 5)) * 512 + lane * 8;
    wstep = 512;
  } else {
    wp = gemm_weight(g, seg) + (int64_t)(n0 - beg + r16) * K + kbase + kq;
    wstep = 32;
  }
  const char* xp[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    if (XM == GK_X_PACKED)
      xp[t] = (const char*)g.X + (((int64_t)(m_blk * MT + t) * (K >> 5) + (kbase >> 5)) * 512 + lane * 8) * 2;
    else   // rows past M repeat row M-1
      xp[t] = (const char*)g.X + ((int64_t)min(m0 + 16 * t + r16, g.M - 1) * g.ldx + kbase + kq) * XB;
  }
  constexpr int xstep = XM == GK_X_PACKED ? 1024 : 32 * XB;   // bytes per K-step
  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0, 0, 0, 0};
  for (int b0 = 0; b0 < nks; b0 += KB) {
    bf16x8 wv[KB];
    XFrag<XF32> xv[MT][KB];
#pragma unroll
    for (int i = 0; i < KB; ++i)
      if (b0 + i < nks) {
        wv[i] = *(const bf16x8*)(wp + wstep * (b0 + i));
#pragma unroll
        for (int t = 0; t < MT; ++t) xv[t][i].load(xp[t] + xstep * (b0 + i));
      }
#pragma unroll
    for (int i = 0; i < KB; ++i)
      if (b0 + i < nks) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv[t][i].get(), wv[i], acc[t], 0, 0, 0);
      }
  }
  // C layout: lane holds output column lane%16, rows 4*(lane/16) + i of its tile
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * ROWS + 16 * t + 4 * (lane >> 4) + i) * 17 + r16] = acc[t][i];
  __syncthreads();
}

// Chunk sums of workgroup (n_blk, kc, m_blk) into part (the 4 waves added as
// (w0 + w1) + (w2 + w3)).  COHERENT (in-launch finish): the sums are stored
// at system scope, written through every cache level, so that a workgroup on
// another XCD can read them in the same launch without a cache write-back
// fence.
template <bool COHERENT, int MT = 2, int XM = GK_X_ROWS, bool WPACKED = false, int KB = GK_KB>
__device__ __forceinline__ void gemm_chunk(int n_blk, int kc, int m_blk, const GemmArgs& g, float* red) {
  constexpr int ROWS = 16 * MT;
  gemm_accumulate<MT, XM, WPACKED, KB>(n_blk, kc, m_blk, g, red);
  const int tid = threadIdx.x;
  const int n0 = n_blk * 16, m0 = m_blk * ROWS;
  const int c = tid & 15;
#pragma unroll
  for (int half = 0; half < MT; ++half) {
    const int r = (tid >> 4) + 16 * half;
    const int m = m0 + r;
    auto rd = [&](int w) { return red[(w * ROWS + r) * 17 + c]; };
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

// S == 1: the workgroup's sums are final; each column pair (2cp, 2cp+1) of
// row m goes to epi(m, cp, x0, x1) (waves added as in gemm_chunk).
template <int MT, int XM, bool WPACKED, int KB, class Epi>
__device__ __forceinline__ void gemm_tile_direct(int n_blk, int m_blk, const GemmArgs& g, float* red, Epi&& epi) {
  constexpr int ROWS = 16 * MT;
  gemm_accumulate<MT, XM, WPACKED, KB>(n_blk, 0, m_blk, g, red);
  const int tid = threadIdx.x;
  const int cp = tid & 7;   // 32 rows x 8 column pairs per pass
#pragma unroll
  for (int r = tid >> 3; r < ROWS; r += 32) {
    const int m = m_blk * ROWS + r;
    if (m < g.M) {
      auto rd = [&](int w, int c) { return red[(w * ROWS + r) * 17 + c]; };
      const float x0 = (rd(0, 2 * cp) + rd(1, 2 * cp)) + (rd(2, 2 * cp) + rd(3, 2 * cp));
      const float x1 = (rd(0, 2 * cp + 1) + rd(1, 2 * cp + 1)) + (rd(2, 2 * cp + 1) + rd(3, 2 * cp + 1));
      epi(m, n_blk * 8 + cp, x0, x1);
    }
  }
}

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

// In-launch finish of tile (n_blk, m_blk) of 16*MT rows, called by each of its
// S workgroups right after gemm_chunk<true>: every workgroup waits until its
// chunk-sum stores have completed and counts itself in with a device-scope
// atomic; the one that brings the count to S adds the chunks (system-scope
// loads) and hands each column pair to epi(m, cp, x0, x1), then puts the
// counter back to zero for the next launch.
//
// Ordering.  The hand-off is ordered by the hardware, not by release/acquire
// operations (an agent-scope release or acquire on gfx950 writes back or
// invalidates the whole L2 of the XCD, which made this launch several times
// slower):
//  1. the chunk sums are system-scope stores (global_store ... sc0 sc1), which
//     write through every cache level and are acknowledged by the memory
//     side, not by the XCD's L2;
//  2. s_waitcnt vmcnt(0) waits for those acknowledgements (vmcnt counts
//     stores on gfx9), and the barrier that follows makes every thread's
//     stores complete before thread 0's counter update;
//  3. the counter update is an atomic with a returned value; thread 0 uses
//     that value, through LDS and a second barrier, to decide whether the
//     workgroup finishes the tile, so no finishing load can issue before the
//     count that includes all S chunks has been read;
//  4. the finisher reads the sums with system-scope loads
//     (global_load ... sc0 sc1), which miss in the L2 and read the memory side
//     where step 1 left the values.
// The bitwise tests of the fused decode step against the two-launch path
// (whose kernel boundary orders everything) check this on the hardware.
template <int MT = 2, class Epi>
__device__ __forceinline__ void gemm_finish_tile(int n_blk, int m_blk, const GemmArgs& g, Epi&& epi,
                                                 int* lds_flag) {
  constexpr int ROWS = 16 * MT;
  const int tid = threadIdx.x;
  __builtin_amdgcn_s_waitcnt(0);   // this thread's sum stores are complete
  __syncthreads();
  int32_t* cnt = g.counters + (int64_t)m_blk * (g.N / 16) + n_blk;
  if (tid == 0) *lds_flag = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g.S - 1;
  __syncthreads();
  if (!*lds_flag) return;
  const int cp = tid & 7;   // 32 rows x 8 column pairs per pass
#pragma unroll
  for (int r = tid >> 3; r < ROWS; r += 32) {
    const int m = m_blk * ROWS + r;
    if (m < g.M) {
      const float2 x = gemm_sum_pair<true>(m, n_blk * 8 + cp, g);
      epi(m, n_blk * 8 + cp, x.x, x.y);
    }
  }
  if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- host side (gemm.hip)
// Where finished columns go: those of segment s to Y[s], at column
// n - seg_end[s-1] of a row-major output with ldy[s] elements per row
// (bf16 outputs need even ldy), or, for ldy[s] < 0 (bf16 only), of a packed
// output with K = -ldy[s] columns (an activation for the next product).
struct GemmOut {
  void* Y[GK_SEG];
  int64_t ldy[GK_SEG];
};

// Rows per workgroup (16 * MT) of a product with M rows.
inline int gemm_mt(int32_t M) { return M <= 16 ? 1 : M <= 32 ? 2 : 4; }
// 16-column tiles per wave (wide kernel above 16 rows, gemm.hip).
constexpr int GW_NT = 4;
constexpr int GW_KB = 2;
inline int gemm_nt(int32_t M) { return gemm_mt(M) == 1 ? 1 : GW_NT; }
// Activations are read row-major (each row broadcast to the lanes of a
// tile) up to this many rows and packed above it.
constexpr int GK_ROWS_MAX = 8;
inline bool gemm_x_packed(int32_t M) { return M > GK_ROWS_MAX; }
// bf16 activations of 17..32 rows are read row-major by the wide kernel
// (measured on the query product at 32 rows: 3 us less than packing them in a
// launch of its own; above 32 rows the packed layout wins).
inline bool gemm_x_rows_wide(int32_t M) { return M > 16 && M <= 32; }
// Rows of a packed activation buffer.
inline int64_t gemm_rows_padded(int32_t M) { return ((int64_t)M + 63) / 64 * 64; }

// K chunks for an [M, N, K] product, counted in 16-column tile units
// (workgroups x 16-column tiles per wave): 1 from GK_UNSPLIT_TILES units on,
// else the least power of two that reaches GK_TARGET_WG units (twice that for
// the wide kernel), at most GK_S_MAX, with K % (S * 128) == 0.  A split
// product must have at most SPLITK_COUNTERS (16*NT)-column tiles.
int gemm_pick_splits(int32_t M, int32_t N, int32_t K);
// Bytes of the chunk sums of a split product (0 when S == 1).
size_t gemm_part_bytes(int32_t M, int32_t N, int32_t S);
// The product with packed weights.  f32_weights: fp32 X (rows), W (packed
// fp32) and Y (VALU kernel; g.S is ignored).  Otherwise bf16 W; X packed bf16
// when gemm_x_packed(M), else rows of fp32 (x_f32) or bf16; Y fp32 (y_f32) or
// bf16; with g.S > 1, g.part holds gemm_part_bytes(M, N, S) bytes, and up to
// 16 rows (one launch, in-launch finish) g.counters SPLITK_COUNTERS zeros
// (every completed launch leaves them at zero; at most SPLITK_COUNTERS tiles);
// above 16 rows a second launch adds the chunks.
hipError_t launch_gemm(const GemmArgs& g, const GemmOut& o, bool f32_weights, bool x_f32, bool y_f32, hipStream_t s);
// Packs rows x K of a row-major matrix (row stride ld elements) into dst
// (packed layout, rows_padded rows; rows past `rows` are zero).  Element
// types: bf16 -> bf16, fp32 -> fp32, or fp32 -> bf16 (to_bf16).
hipError_t launch_pack(const void* src, int64_t ld, int32_t rows, int64_t rows_padded, int32_t K, bool src_f32,
                       bool to_bf16, void* dst, hipStream_t s);

}  // namespace mla
