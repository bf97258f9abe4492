// Split-KV flash decode over the paged latent cache, bf16 MFMA (gfx950).
//
// What it computes ("DeepSeek-V2：在“大力出奇迹”的AI军备竞赛中，四两拨千斤",
// liang.world, ch.2 §1-§3): for one decode query per sequence and every head
// i, scores s_j = q~_i . c_j + q^R_i . k^R_j over the sequence's cached rows
// [c_j ; k^R_j] (576 wide), softmax over j, and O~_i = sum_j p_j c_j.  W^UK
// is already folded into q~ (absorb kernel) and W^UV is applied after the
// split combine (combine kernel), so K and V are never built (ch.2 §2,
// absorption paragraph).
//
// One workgroup = NW waves (one per SIMD, occupancy 1) and one contiguous
// range of the batch's tokens (see split_begin).  All n_h = 32*NW heads of a
// sequence share each staged tile:
//  * Within each sequence piece the tiles are visited from a per-split
//    starting tile on, wrapping around (tile_phase, mla_common.h), so that
//    the workgroups' concurrent reads do not march through the pool in
//    lockstep at fixed distances, which crowds HBM channels.
//  * Tiles of TT = 32 cached rows (36 KB) are copied HBM -> LDS with
//    global_load_lds (16 B per lane, 1 KB per wave instruction), three
//    buffers deep: two tiles are in flight while one is computed.  A row is
//    9 lines of 128 B (8 of c^KV, 1 of k^R); copy instruction (g, j) fetches
//    line j of the 8 rows of row group g, i.e. 8 whole cache lines, into a
//    1 KB LDS window: the 16-byte chunk c of row r = 8g + m sits in window
//    9g + c/8 at granule 8*(m ^ (g&1)) + ((c%8) ^ sw(m)), sw swapping the
//    two low bits of m.  That places the score fragments (16 rows, one
//    chunk) and the V^T transposed reads (4 rows x 4 chunks) on distinct
//    LDS banks.  Wave w copies row group w, so a lane resolves one pool row
//    per tile.  The two page ids a tile can touch (pages hold >= 32 rows)
//    are copied into LDS one iteration ahead the same way, so they travel in
//    the same in-order queue as the tiles: no scalar load is pending while
//    LDS reads are waited for.
//  * Scores: wave w owns heads 32w..32w+31.  S^T (16 tokens x 16 heads
//    blocks) = K_tile . Q^T with v_mfma_f32_16x16x32_bf16.  The wave's query
//    block (32 heads x 576 bf16) is split: latent dims 0..447 in 112 VGPRs,
//    dims 448..575 (incl. the RoPE part) staged once per sequence in LDS.
//  * Online softmax in the wave that owns the heads, in log2 units (q~
//    carries softmax_scale*log2(e)).  The running reference max only moves
//    when a tile's max exceeds it by more than RESCALE_T (so p <=
//    2^RESCALE_T), which makes the O rescale rare; the accumulators are
//    zeroed when a segment ends.  Row reductions use v_permlane16/32_swap.
//  * P.V: the same wave owns those 32 heads' O over all 512 latent columns
//    (O^T blocks of 32 latent columns x 32 heads, v_mfma_f32_32x32x16_bf16,
//    256 fp32 accumulators kept in AGPRs).  P never leaves the wave: one
//    v_permlane16_swap per dword turns the score accumulators (bf16) into
//    the P^T operand, so no wave waits for another between the scores and
//    P.V, and the tile-top barrier is the only one per tile.  Block dblk =
//    2g + p holds the columns of chunks 8g + p + {0, 2, 4, 6}; its V^T
//    fragments are read from the staged tile with ds_read_b64_tr_b16.
//  * At the end of each (sequence, range) segment the unnormalised O~ (bf16),
//    the reference max m and the sum l (fp32) go to the segment's partial slot;
//    O~ is transposed through the wave's staged-query LDS area so that every
//    store writes whole 256-byte row pieces.
#include "mla_common.h"

namespace mla {
namespace {

constexpr int TT = DECODE_TT;           // cached rows per tile (32)
constexpr int NINSTR = TT * 72 / 64;    // 36 copy instructions (blocks of 1 KB) per tile
constexpr int TILEB = NINSTR * 1024;    // 36,864 bytes per tile buffer (36 windows of 1 KB)
constexpr int PGOFF = TILEB;            // the tile's two page ids follow its windows
constexpr float RESCALE_T = 24.0f;      // log2 headroom before the reference max moves
constexpr int KS = D_K / 32;            // 18 K-steps of 32 for the score MFMA
constexpr int KS_REG = 14;              // K-steps of the query block kept in VGPRs
constexpr int KS_LDS = KS - KS_REG;     // K-steps staged in LDS (query dims 448..575)
constexpr int QLB = KS_LDS * 64;        // LDS bytes per head of the staged query part

// s_waitcnt immediate waiting until at most n vector-memory operations are
// outstanding (expcnt and lgkmcnt left alone).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// HBM -> LDS copies (global_load_lds).  m0 holds the LDS base of a copy; the
// instruction reads it when it leaves the wave's memory queue, so an m0 write
// right behind a copy waits for that.  m0 is therefore written before each
// copy and not restored after it (declared clobbered: the compiler sets it
// again where it needs it), with the one wait state required between an m0
// write and an LDS-DMA load.  Issued through asm so that the compiler's
// wait-count pass does not see an LDS write in flight: with one visible it
// drains every LDS wait to zero, which would serialise the fragment reads
// below.  The instructions have no result register; their completion is
// awaited explicitly (vmcnt(0) + barrier before the tile is read), and the
// memory clobber keeps LDS accesses on their side of them.
//
// m0 is a register the compiler reserves, and clang warns that a clobber of
// it is not preserved for the compiler; nothing the compiler emits in this
// file reads m0 (tests/test_isa_m0.py checks the built code for that), so
// the warning is silenced for these three helpers.
//
// 16 bytes per lane: lane i's chunk lands at LDS byte lds_base + 16*i.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "s"(lds_base)
               : "memory", "m0");
}
// 4 bytes per active lane (lane i -> lds_base + 4*i).
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(gptr), "s"(lds_base)
               : "memory", "m0");
}
// dma16 of line j of a row group: the copy reads gptr + 128*j (j < 8: the
// offset is the instruction's immediate) or gptr (j = 8), so one address
// register pair serves all nine lines.  The immediate offset is added to the
// LDS address as well, so m0 is set that much lower.
__device__ __forceinline__ void dma16_line(const char* gptr, int j, uint32_t lds_base) {
#define MLA_DMA_LINE(OFF)                                                                                 \
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:" #OFF : : "v"(gptr), \
               "s"(lds_base - (OFF))                                                                     \
               : "memory", "m0")
  switch (j) {
    case 1: MLA_DMA_LINE(128); break;
    case 2: MLA_DMA_LINE(256); break;
    case 3: MLA_DMA_LINE(384); break;
    case 4: MLA_DMA_LINE(512); break;
    case 5: MLA_DMA_LINE(640); break;
    case 6: MLA_DMA_LINE(768); break;
    case 7: MLA_DMA_LINE(896); break;
    default: MLA_DMA_LINE(0); break;
  }
#undef MLA_DMA_LINE
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(lds_void*)p;
}

// Column swizzle of row m (0..7) inside an 8x8 window: swaps bits 0 and 1.
__device__ __forceinline__ int swz(int m) { return (m & 4) | ((m & 1) << 1) | ((m >> 1) & 1); }

// Split handled by workgroup bid: XCD x = bid % 8 receives the x-th of 8
// contiguous runs of splits (run sizes differ by at most one).
__device__ __forceinline__ int32_t xcd_split(int32_t bid, int32_t G) {
  const int32_t x = bid & 7, q = G >> 3, r = G & 7;
  return x * q + (x < r ? x : r) + (bid >> 3);
}

// Max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float wave_rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The O accumulators stay in AGPRs for the whole kernel; these macros touch
// one accumulator through an "a" operand so that the register allocator never
// moves the 256 of them into VGPRs.
#define ACC_SCALE(x, a)                                                                        \
  do {                                                                                         \
    float acc_tmp_;                                                                            \
    asm volatile("v_accvgpr_read_b32 %0, %1\n\tv_mul_f32 %0, %0, %2\n\tv_accvgpr_write_b32 %1, %0" \
                 : "=&v"(acc_tmp_), "+a"(x)                                                    \
                 : "v"(a));                                                                    \
  } while (0)
#define ACC_READ(dst, x) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(dst) : "a"(x))
#define ACC_ZERO(x) asm volatile("v_accvgpr_write_b32 %0, 0" : "=a"(x))
// O^T block += A B on the matrix cores, accumulating in place in AGPRs.  The
// compiler does not see this as an MFMA, so the wait states it would insert
// are written here: two ahead of the MFMA (a VALU write of a source operand
// needs them), and ACC_DRAIN before accumulators are read back.
#define ACC_MFMA(acc, a, b) \
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b))
#define ACC_DRAIN() asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7")

struct TileDesc {
  int32_t b, t0, n;    // sequence, first token in the sequence, rows (0 = none)
  int32_t p0, rem;     // page index of t0 within the sequence, t0 % page_size
  int32_t first, last;
};

// Read-only device arrays (plan records, prefix sums, page table) are read
// through the constant address space so that uniform reads are scalar loads.
typedef const __attribute__((address_space(4))) int32_t* cint_t;

// Cursor over the tiles of one workgroup's token range [P0, P1) (split
// `split`).  The range is cut at sequence ends into segments; a segment
// [sx, se) is cut into K tiles of TT rows from sx on (only tile K-1 can be
// shorter) and visited from tile tile_phase(split, K) on, wrapping around to
// tile 0 (mla_common.h).  Tiles never straddle two sequences.  From one tile
// to the next within a segment the page index and offset advance by TT
// (pages hold at least TT rows); the wrap goes back to the segment's start.
struct Cursor {
  int32_t P1, B, page_size, split;
  int32_t b, s_beg, s_end;   // sequence of the current segment, its tokens [s_beg, s_end)
  int32_t sx, se, K, j, k;   // segment [sx, se) of K tiles, j of them handed out, k the next one
  int32_t pidx, prem;        // page index (in the sequence) and offset of tile k's first row
  int32_t p_sx, r_sx;        // the same for tile 0
  bool done;
  __device__ void segment(int32_t x) {
    sx = x;
    se = s_end < P1 ? s_end : P1;
    K = (se - sx + TT - 1) / TT;
    j = 0;
    k = tile_phase(split, K);
    const int32_t t0 = sx - s_beg, tk = t0 + TT * k;
    p_sx = t0 / page_size;
    r_sx = t0 - p_sx * page_size;
    pidx = tk / page_size;
    prem = tk - pidx * page_size;
  }
  __device__ void init(cint_t rec, int32_t B_, int32_t P0, int32_t P1_, int32_t ps, int32_t w) {
    B = B_;
    P1 = P1_;
    page_size = ps;
    split = w;
    b = rec[0];
    s_beg = rec[1];
    s_end = rec[2];
    done = P0 >= P1;
    if (!done) segment(P0);
  }
  __device__ TileDesc next(cint_t prefix) {
    TileDesc t;
    if (done) {
      t.b = 0; t.t0 = 0; t.n = 0; t.p0 = 0; t.rem = 0; t.first = 0; t.last = 0;
      return t;
    }
    const int32_t x0 = sx + TT * k;
    t.b = b;
    t.t0 = x0 - s_beg;
    t.n = (se - x0) < TT ? (se - x0) : TT;
    t.p0 = pidx;
    t.rem = prem;
    t.first = (j == 0);
    ++j;
    t.last = (j == K);
    if (t.last) {
      if (se < P1) {
        // move to the next sequence holding tokens (skip empty ones)
        do {
          ++b;
          s_beg = s_end;
          s_end = prefix[b + 1];
        } while (s_end <= se && b < B - 1);
        segment(se);
      } else {
        done = true;
      }
    } else if (++k == K) {
      k = 0;
      pidx = p_sx;
      prem = r_sx;
    } else {
      prem += TT;
      if (prem >= page_size) {
        prem -= page_size;
        ++pidx;
      }
    }
    return t;
  }
};

// GATHER: the sparse decode.  A sequence's "tokens" are then the positions
// of its kept list, and position i lives in pool row rows[b * rows_stride +
// i] (rows checked by the selection); a tile's 32 row ids travel like the
// page ids (into the tile buffer's pad, one iteration ahead).
template <int NW, bool GATHER>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_mfma_kernel(const bf16* __restrict__ qabs, const bf16* __restrict__ c_KV, const bf16* __restrict__ k_R,
                   int64_t row_stride, int32_t num_pages, const int32_t* __restrict__ page_table,
                   int32_t max_pages, int32_t page_size, const int32_t* __restrict__ prefix,
                   const int32_t* __restrict__ split_rec, int32_t B, int32_t G, float* __restrict__ part_ml,
                   bf16* __restrict__ part_o, int32_t* __restrict__ flags, const int32_t* __restrict__ rows,
                   int32_t rows_stride) {
  constexpr int NH = 32 * NW;
  constexpr int IPW = NINSTR / NW;              // DMA instructions per wave (NW divides 36)
  constexpr int DB = 16;                        // 32-wide latent blocks of a wave's O (all 512 columns)
  __shared__ __attribute__((aligned(1024))) char kt0[TILEB + 4 * TT];
  __shared__ __attribute__((aligned(1024))) char kt1[TILEB + 4 * TT];
  __shared__ __attribute__((aligned(1024))) char kt2[TILEB + 4 * TT];
  __shared__ __attribute__((aligned(1024))) char ql[NH * QLB];   // query dims 448..575, swizzled

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const cint_t cpre = (cint_t)prefix;
  const cint_t cpt = (cint_t)page_table;
  const int64_t N = cpre[B];
  // Workgroups are handed to the 8 XCDs round-robin; splits are mapped so
  // that each XCD runs a contiguous run of splits, whose sequences' queries,
  // page-table rows and plan records then stay in that XCD's L2.
  const int32_t split = xcd_split(blockIdx.x, G);
  const int32_t P0 = (int32_t)split_begin(split, N, G), P1 = (int32_t)split_begin(split + 1, N, G);
  if (P0 >= P1) return;

  // ---- per-lane constant offsets (see the tile layout in the header)
  // score A fragment (16x16x32): row 16tb + (lane&15), chunk 4ks + (lane>>4);
  // a_off[ks&1] + 18432*tb + 1024*(ks/2) is its byte in the tile
  int a_off[2];
  {
    const int m = lane & 7, h = (lane >> 3) & 1, q4 = lane >> 4;
#pragma unroll
    for (int par = 0; par < 2; ++par) a_off[par] = 16 * (576 * h + 8 * (m ^ h) + ((q4 ^ swz(m)) ^ (4 * par)));
  }
  // staged query fragment: head 32w + 16hb + (lane&15), chunk 4(ks-KS_REG) + (lane>>4),
  // stored at chunk position c ^ (head & 15)
  const int q_off = (32 * wave + (lane & 15)) * QLB;
  // V^T fragment (ds_read_b64_tr_b16) of block dblk = 2g + p, rows kc*16 + 4rr + ...:
  // source lane s reads row 8*(s>>5) + ((s&15)>>2) (plus kc*16 + 4rr), chunk 8g + p + 2y with
  // y = 2*((s>>4)&1) + ((s&3)>>1), bytes 8*(s&1) .. +7 of that chunk
  // v_off[p][hi] + 1024*g + 18432*kc is that byte in the tile (rows m + 4*hi of the 8-row group)
  int v_off[2][2];
  {
    const int rgb = lane >> 5, y = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int m = ((lane & 15) >> 2) + 4 * hi;
        v_off[p][hi] = 16 * (576 * rgb + 8 * (m ^ rgb) + ((p + 2 * y) ^ swz(m))) + 8 * (lane & 1);
      }
  }

  Cursor cur;
  const cint_t rec = (cint_t)split_rec + SPLIT_REC * split;
  cur.init(rec, B, P0, P1, page_size, split);
  TileDesc t_now = cur.next(cpre);   // tile being computed
  TileDesc t_n1 = cur.next(cpre);    // tile in flight
  TileDesc t_n2 = cur.next(cpre);    // tile whose copy is issued this iteration

  // Page-table index of the first (which = 0) or last (which = 1) page a tile touches.
  auto page_index = [&](const TileDesc& td, int which) __attribute__((always_inline)) -> int64_t {
    const int32_t p = (which && td.rem + td.n > page_size) ? td.p0 + 1 : td.p0;
    return (int64_t)td.b * max_pages + p;
  };
  // Pool row of tile row r (rows past the tile's end repeat its last row).
  auto resolve_row = [&](const TileDesc& td, int r, int32_t pg0, int32_t pg1) __attribute__((always_inline)) -> int32_t {
    r = min(r, td.n - 1);
    const int off = td.rem + r;
    const bool cross = off >= page_size;
    int32_t pg = cross ? pg1 : pg0;
    if (pg < 0 || pg >= num_pages) {
      atomicOr(flags, MLA_FLAG_BAD_PAGE);
      pg = pg < 0 ? 0 : num_pages - 1;
    }
    return pg * page_size + (cross ? off - page_size : off);
  };
  // The two page ids of a tile (GATHER: its 32 row ids, positions past the
  // tile's end repeating its last) go to the pad after the windows of a tile
  // buffer (never written by tile copies, never read by the math).
  auto issue_page_ids = [&](char* kt, const TileDesc& td) __attribute__((always_inline)) {
    if (GATHER) {
      if (wave == 0 && td.n > 0 && lane < TT)
        dma4(rows + (int64_t)td.b * rows_stride + td.t0 + min(lane, td.n - 1),
             __builtin_amdgcn_readfirstlane(lds_addr(kt + PGOFF)));
    } else {
      if (wave == 0 && td.n > 0 && lane < 2)
        dma4(page_table + page_index(td, lane), __builtin_amdgcn_readfirstlane(lds_addr(kt + PGOFF)));
    }
  };
  const int64_t stride_b = row_stride * 2;
  // Copy of a tile: wave w fetches row groups w, w + NW, ...; in row group g
  // lane l fetches row 8g + m, m = (l>>3) ^ (g&1), and chunk 8j + ((l&7) ^
  // sw(m)) of it for the 9 lines j (line 8 is k^R), into window 9g + j.
  // dma_src() forms a lane's source offset for the wave's gi-th row group
  // from the scalar bases (nothing is kept live across the loop); copy
  // instruction I = 9*gi + j of the wave is issued by dma_one().
  auto dma_src = [&](const TileDesc& td, int gi, int32_t pg0, int32_t pg1, const char* ids)
                     __attribute__((always_inline)) -> int64_t {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int g = wave + NW * gi;
    const int m = (ln >> 3) ^ (g & 1);
    // GATHER: the ids come from the selection, which only lists checked
    // rows; the clamp keeps the copy inside the pool whatever they hold
    const int64_t row = GATHER ? min(max(*(const int32_t*)(ids + 4 * (8 * g + m)), 0), num_pages * page_size - 1)
                               : resolve_row(td, 8 * g + m, pg0, pg1);
    return row * stride_b + 16 * ((ln & 7) ^ swz(m));
  };
  auto dma_one = [&](char* kt, int I, const char* pc, const char* pk) __attribute__((always_inline)) {
    const int gi = I / 9, j = I % 9, g = wave + NW * gi;
    dma16_line(j < 8 ? pc : pk, j, __builtin_amdgcn_readfirstlane(lds_addr(kt) + (9 * g + j) * 1024));
  };
  auto issue_dma = [&](char* kt, const TileDesc& td, int32_t pg0, int32_t pg1) __attribute__((always_inline)) {
#pragma unroll
    for (int gi = 0; gi < 4 / NW; ++gi) {
      const int64_t off = dma_src(td, gi, pg0, pg1, kt + PGOFF);
      const char* pc = (const char*)c_KV + off;
      const char* pk = (const char*)k_R + off;
#pragma unroll
      for (int j = 0; j < 9; ++j) dma_one(kt, 9 * gi + j, pc, pk);
    }
  };

  // ---- state
  bf16x8 q[2][KS_REG];
  f32x16 o[DB];
  // Softmax state of the lane's heads 32w + 16hb + (lane&15): the reference
  // max (the same in the four lanes that hold a head) and this lane's part of
  // the sum (its tokens only; the four parts are added when the segment ends).
  float m_ref[2], l_sum[2];

  // q~ is grouped for these loads (qabs_offset): the 14 register fragments of
  // 16 heads are 14 consecutive 1 KB blocks, and the staged dims 448..575 are
  // 256 B per head, head after head, so every load below covers one whole
  // 1 KB run.  ql keeps chunk c of head h at chunk position c ^ (h & 15).
  static_assert(KS_REG == 14 && QLB == 256, "the q~ layout of qabs_offset");
  auto load_q = [&](int32_t b) __attribute__((always_inline)) {
    int ln = lane;   // hidden from loop-invariant hoisting
    asm volatile("" : "+v"(ln));
    const bf16* qb = qabs + (int64_t)b * NH * D_K;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const bf16* qp = qb + (2 * wave + hb) * KS_REG * 512 + (ln & 15) * 32 + 8 * (ln >> 4);
#pragma unroll
      for (int ks = 0; ks < KS_REG; ++ks) q[hb][ks] = *(const bf16x8*)(qp + 512 * ks);
    }
#pragma unroll
    for (int j = 0; j < 32 * QLB / 1024; ++j) {
      const int sigma = 64 * j + ln;
      const int hl = sigma / (QLB / 16), c = (sigma % (QLB / 16)) ^ (hl & 15);
      const bf16* src = qb + NH * 32 * KS_REG + (32 * wave + hl) * (QLB / 2) + 8 * c;
      dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(ql + wave * 32 * QLB + j * 1024)));
    }
  };

  // The query registers are loaded once per segment.  Their loads are waited
  // for right away (vmcnt(0)) and the registers then pass through an empty
  // asm, so the compiler sees no load of them pending across the loop and
  // puts no wait in the score loop (a wait there would also hold up the
  // tiles in flight).
  auto settle_q = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int ks = 0; ks < KS_REG; ++ks) asm volatile("" : "+v"(q[hb][ks]));
  };

  // ---- prologue: tiles 0 and 1 in flight, page ids of tile 2 in flight
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) ACC_ZERO(o[db][r]);
  m_ref[0] = m_ref[1] = -INFINITY;
  l_sum[0] = l_sum[1] = 0.f;
  // The query loads go first; the pages of the first two tiles come with the
  // split's plan record when both lie in its first segment, so both copies
  // start one memory latency after the record.
  if (GATHER) {
    // the row ids of the first two tiles, then the query and the copies
    issue_page_ids(kt0, t_now);
    issue_page_ids(kt1, t_n1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    load_q(t_now.b);
    issue_dma(kt0, t_now, 0, 0);
    if (t_n1.n > 0) issue_dma(kt1, t_n1, 0, 0);
  } else {
    load_q(t_now.b);
    const int32_t a0 = rec[3], a1 = rec[4];
    int32_t b0 = 0, b1 = 0;
    if (t_n1.n > 0) {
      if (!t_now.last) {
        b0 = rec[5];
        b1 = rec[6];
      } else {
        b0 = cpt[page_index(t_n1, 0)];
        b1 = cpt[page_index(t_n1, 1)];
      }
    }
    issue_dma(kt0, t_now, a0, a1);
    if (t_n1.n > 0) issue_dma(kt1, t_n1, b0, b1);
  }
  issue_page_ids(kt2, t_n2);
  settle_q();

  auto process = [&](char* kt, char* kt_issue) __attribute__((always_inline)) {
    // Tile t_now was copied into kt two iterations ago; t_n1's copy (issued
    // last iteration, after the page ids of t_n2) may stay in flight.
    if (t_n1.n <= 0)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(IPW));
    __syncthreads();   // copies and page ids landed; P.V of the previous tile done everywhere
    const TileDesc t_n3 = cur.next(cpre);
    // page ids of t_n3 (its buffer is kt) before the copy of t_n2, so that
    // next iteration's wait covers them
    issue_page_ids(kt, t_n3);
    // t_n2's copy instructions are spread over the score K-steps below, so
    // that the four waves do not queue them all at once
    const bool copy = t_n2.n > 0;
    const char* dpc[4 / NW];
    const char* dpk[4 / NW];
    {
      const int2 pg = *(const int2*)(kt_issue + PGOFF);
#pragma unroll
      for (int gi = 0; gi < 4 / NW; ++gi) {
        const int64_t off = copy ? dma_src(t_n2, gi, pg.x, pg.y, kt_issue + PGOFF) : 0;
        dpc[gi] = (const char*)c_KV + off;
        dpk[gi] = (const char*)k_R + off;
      }
    }

    // ---- scores S^T[token][head] for this wave's 32 heads (2 x 2 blocks of 16x16)
    // Software pipelined by hand: the fragments of K-step ks+2 are read before
    // the MFMAs of K-step ks issue; sched_barrier keeps that order.
    f32x4 s[2][2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) s[tb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 af[3][2], qf[3][2];
    auto load_ks = [&](int ks, int st) __attribute__((always_inline)) {
      const int off = a_off[ks & 1] + 1024 * (ks >> 1);
      af[st][0] = *(const bf16x8*)(kt + off);
      af[st][1] = *(const bf16x8*)(kt + off + 18432);
      if (ks >= KS_REG) {
        const int qc = ((4 * (ks - KS_REG) + (lane >> 4)) ^ (lane & 15)) << 4;
        qf[st][0] = *(const bf16x8*)(ql + q_off + qc);
        qf[st][1] = *(const bf16x8*)(ql + q_off + 16 * QLB + qc);
      }
    };
    load_ks(0, 0);
    load_ks(1, 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 2 < KS) load_ks(ks + 2, (ks + 2) % 3);
      __builtin_amdgcn_sched_barrier(0);
      const int st = ks % 3;
      const bf16x8 qb0 = ks < KS_REG ? q[0][ks] : qf[st][0];
      const bf16x8 qb1 = ks < KS_REG ? q[1][ks] : qf[st][1];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        s[tb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[st][tb], qb0, s[tb][0], 0, 0, 0);
        s[tb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[st][tb], qb1, s[tb][1], 0, 0, 0);
      }
      if (copy) {
#pragma unroll
        for (int I = ks * IPW / KS; I < (ks + 1) * IPW / KS; ++I) dma_one(kt_issue, I, dpc[I / 9], dpk[I / 9]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- online softmax (owner wave), lane holds heads 32w + 16hb + (lane&15),
    // tokens 16tb + 4(lane>>4) + i.  The cross-lane max is only formed when
    // a segment starts or when some lane's own max exceeds the reference by
    // more than RESCALE_T (rare); otherwise every lane checks its own values.
    const int n_valid = t_now.n;
    if (n_valid < TT) {   // a segment's last tile may be partial
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * tb + 4 * (lane >> 4) + i >= n_valid) s[tb][hb][i] = -INFINITY;
    }
    float lmax[2];
    int over = 0;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      lmax[hb] = fmaxf(fmaxf(fmaxf(s[0][hb][0], s[0][hb][1]), fmaxf(s[0][hb][2], s[0][hb][3])),
                       fmaxf(fmaxf(s[1][hb][0], s[1][hb][1]), fmaxf(s[1][hb][2], s[1][hb][3])));
      over |= lmax[hb] > m_ref[hb] + RESCALE_T ? 1 : 0;
    }
    float alpha[2] = {1.f, 1.f};
    int any_resc = 0;
    if (t_now.first || __builtin_amdgcn_readfirstlane(__any(over) ? 1 : 0)) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const float mx = wave_rows_max(lmax[hb]);
        if (t_now.first) {
          // a new segment: the accumulators were zeroed at the previous segment's end
          m_ref[hb] = mx;
        } else if (mx > m_ref[hb] + RESCALE_T) {
          alpha[hb] = __builtin_amdgcn_exp2f(m_ref[hb] - mx);
          any_resc = 1;
          m_ref[hb] = mx;
        }
      }
      any_resc = __builtin_amdgcn_readfirstlane(__any(any_resc) ? 1 : 0);
    }
    // P in bf16, and the B fragments of P^T for the two 16-token chunks.
    // Lane (g, c) = (lane>>4, lane&15) holds P of tokens 16tb + 4g + i for
    // heads c (x[0]) and 16 + c (x[1]); the 32x32x16 B operand wants, in lane
    // (g, c), head 16(g&1) + c and tokens 16tb + 8(g>>1) + 0..7.  Rows g and
    // g^1 trade x[0] of the odd row for x[1] of the even row
    // (v_permlane16_swap), after which (x[0], x[1]) is that fragment.
    bf16x8 pf[2];
    float sum[2] = {0.f, 0.f};
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      bf16x4 x[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(s[tb][hb][i] - m_ref[hb]);
          x[hb][i] = (bf16)p;
          sum[hb] += p;
        }
      const u32x2 x0 = __builtin_bit_cast(u32x2, x[0]), x1 = __builtin_bit_cast(u32x2, x[1]);
      const auto w0 = __builtin_amdgcn_permlane16_swap(x0[0], x1[0], false, false);
      const auto w1 = __builtin_amdgcn_permlane16_swap(x0[1], x1[1], false, false);
      pf[tb] = __builtin_bit_cast(bf16x8, u32x4{w0[0], w1[0], w0[1], w1[1]});
    }
    l_sum[0] = l_sum[0] * alpha[0] + sum[0];
    l_sum[1] = l_sum[1] * alpha[1] + sum[1];

    // ---- rescale O where the reference max moved (rare): the lane's
    // accumulators all belong to head lane&31 = 16((lane>>4)&1) + (lane&15)
    if (any_resc) {
      const float a = (lane & 16) ? alpha[1] : alpha[0];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) ACC_SCALE(o[db][r], a);
    }

    // ---- O^T[d][head] += V^T[d][tok] P^T[tok][head] for the wave's 32 heads
    // and all 512 latent columns: 2 chunks x 16 blocks, V^T fragments read
    // from the staged tile VR steps ahead of their MFMA.
    constexpr int VR = 4;
    constexpr int NSTEP = 2 * DB;
    bf16x8 vf[VR];
    auto load_v = [&](int step) __attribute__((always_inline)) {
      const int kc = step / DB, dblk = step % DB;
      const int base = 1024 * (dblk >> 1) + 18432 * kc;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kt + base + v_off[dblk & 1][0]));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kt + base + v_off[dblk & 1][1]));
      const bf16x4 lob = __builtin_bit_cast(bf16x4, lo), hib = __builtin_bit_cast(bf16x4, hi);
      bf16x8& v = vf[step % VR];
      v[0] = lob[0]; v[1] = lob[1]; v[2] = lob[2]; v[3] = lob[3];
      v[4] = hib[0]; v[5] = hib[1]; v[6] = hib[2]; v[7] = hib[3];
    };
#pragma unroll
    for (int st = 0; st < VR - 1; ++st) load_v(st);
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      if (st + VR - 1 < NSTEP) load_v(st + VR - 1);
      __builtin_amdgcn_sched_barrier(0);
      ACC_MFMA(o[st % DB], vf[st % VR], pf[st / DB]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- segment end: write the partial (O~ unnormalised, m, l)
    if (t_now.last) {
      ACC_DRAIN();   // the last MFMAs' results are read back below
      const int64_t slot = (int64_t)split + t_now.b;
      // O~ goes out through the wave's staged-query area (32 heads x 128
      // latent columns of bf16 at a time, 16-byte chunk c of head row h at
      // chunk position c ^ (h & 15)), so that each store covers 4 heads x 256
      // contiguous bytes.  The area is reloaded with the next query below.
      char* stg = ql + wave * 32 * QLB;
      int ln = lane;   // hidden from loop-invariant hoisting (the addresses below stay local)
      asm volatile("" : "+v"(ln));
      const int wh = ln & 31;                                   // head row written by this lane
      char* const wrow = stg + wh * 256 + (ln >> 5) * 8;
      const int rh = ln >> 4, rc = ln & 15;                     // head (mod 4) and chunk read
      {
#pragma unroll
        for (int pc = 0; pc < DB / 4; ++pc) {
#pragma unroll
          for (int dq = 0; dq < 4; ++dq) {
            const int db = 4 * pc + dq;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              // accumulator row m = 8*r4 + 4*(lane>>5) + r%4 of block dblk = 2g + p is
              // latent column 8*(8g + p + 2*r4) + 4*(lane>>5) + r%4: chunk
              // 8*(dq>>1) + (dq&1) + 2*r4 of this 128-column piece, half lane>>5
              float v0, v1, v2, v3;
              ACC_READ(v0, o[db][4 * r4]);
              ACC_READ(v1, o[db][4 * r4 + 1]);
              ACC_READ(v2, o[db][4 * r4 + 2]);
              ACC_READ(v3, o[db][4 * r4 + 3]);
              bf16x4 v;
              v[0] = (bf16)v0;
              v[1] = (bf16)v1;
              v[2] = (bf16)v2;
              v[3] = (bf16)v3;
              const int chunk = 8 * (dq >> 1) + (dq & 1) + 2 * r4;
              *(bf16x4*)(wrow + ((chunk ^ (wh & 15)) << 4)) = v;
            }
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int h = 4 * k + rh;
            const bf16x8 v = *(const bf16x8*)(stg + h * 256 + ((rc ^ (h & 15)) << 4));
            bf16* dst = part_o + (slot * NH + 32 * wave + h) * D_C + 128 * pc + 8 * rc;
            *(bf16x8*)dst = v;
          }
        }
      }
      const float lt0 = wave_rows_sum(l_sum[0]), lt1 = wave_rows_sum(l_sum[1]);
      if (lane < 16) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int head = 32 * wave + 16 * hb + lane;
          part_ml[(slot * NH + head) * 2 + 0] = m_ref[hb];
          part_ml[(slot * NH + head) * 2 + 1] = hb ? lt1 : lt0;
        }
      }
      m_ref[0] = m_ref[1] = -INFINITY;
      l_sum[0] = l_sum[1] = 0.f;
      // the next segment accumulates from zero
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) ACC_ZERO(o[db][r]);
      // the next segment's query, loaded and waited for here (once per
      // segment) so that no query load is in flight during a later tile
      if (t_n1.n > 0) {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // staged reads done before the copies overwrite the area
        load_q(t_n1.b);
        settle_q();
      }
    }
    t_now = t_n1;
    t_n1 = t_n2;
    t_n2 = t_n3;
  };

  // three iterations per loop so that the buffer roles stay compile-time:
  // tile i is computed from buffer i%3 while tile i+2 is copied into (i+2)%3
  while (true) {
    process(kt0, kt2);
    if (t_now.n <= 0) break;
    process(kt1, kt0);
    if (t_now.n <= 0) break;
    process(kt2, kt1);
    if (t_now.n <= 0) break;
  }
}

}  // namespace

template <int NW, bool GATHER>
static void launch_nw(dim3 grid, hipStream_t s, const bf16* qabs, const bf16* c_KV, const bf16* k_R,
                      int64_t row_stride, int32_t num_pages, const int32_t* page_table, int32_t max_pages,
                      int32_t page_size, const int32_t* prefix, const int32_t* split_rec, int32_t B, int32_t G,
                      float* part_ml, bf16* part_o, int32_t* flags, const int32_t* rows, int32_t rows_stride) {
  decode_mfma_kernel<NW, GATHER><<<grid, 64 * NW, 0, s>>>(qabs, c_KV, k_R, row_stride, num_pages, page_table,
                                                          max_pages, page_size, prefix, split_rec, B, G, part_ml,
                                                          part_o, flags, rows, rows_stride);
}

hipError_t launch_decode_mfma(const mla_dims& d, int32_t B, const void* qabs, const void* c_KV,
                              const void* k_R, int64_t row_stride, int32_t num_pages,
                              const int32_t* page_table, int32_t max_pages, const int32_t* prefix,
                              const int32_t* split_rec, int32_t n_splits, float* part_ml, void* part_o_v,
                              int32_t* flags, hipStream_t s, const int32_t* rows, int32_t rows_stride) {
  const dim3 grid(n_splits);
  const bool g = rows != nullptr;
  const auto q = (const bf16*)qabs;
  const auto c = (const bf16*)c_KV;
  const auto k = (const bf16*)k_R;
  bf16* po = (bf16*)part_o_v;
#define MLA_LAUNCH_NW(NW, G)                                                                                  \
  launch_nw<NW, G>(grid, s, q, c, k, row_stride, num_pages, page_table, max_pages, d.page_size, prefix,      \
                   split_rec, B, n_splits, part_ml, po, flags, rows, rows_stride)
  switch (d.n_h / 32) {
    case 1: if (g) MLA_LAUNCH_NW(1, true); else MLA_LAUNCH_NW(1, false); break;
    case 2: if (g) MLA_LAUNCH_NW(2, true); else MLA_LAUNCH_NW(2, false); break;
    case 4: if (g) MLA_LAUNCH_NW(4, true); else MLA_LAUNCH_NW(4, false); break;
    default: return hipErrorInvalidValue;
  }
#undef MLA_LAUNCH_NW
  return hipGetLastError();
}

}  // namespace mla
