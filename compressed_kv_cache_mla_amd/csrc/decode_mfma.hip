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
// One workgroup = 4 waves (one per SIMD, occupancy 1) and one contiguous range
// of the batch's tokens (see split_begin).  All n_h heads of a sequence share
// each staged tile:
//  * Tiles of TT = 48 cached rows (54 KB) are copied HBM -> LDS with
//    global_load_lds (16 B per lane, 1 KB per wave instruction, coalesced),
//    double buffered.  Row r keeps its 72 16-byte chunks in row-major order
//    with chunk c stored at slot c ^ swz(r), which makes both LDS read
//    patterns below bank-conflict free.
//  * Scores: wave w owns heads 32w..32w+31.  S^T (16 tokens x 16 heads
//    blocks) = K_tile . Q^T with v_mfma_f32_16x16x32_bf16; the wave's Q block
//    (32 heads x 576, bf16) lives in 144 VGPRs, K fragments come from LDS.
//  * Online softmax in the owner wave, in log2 units (q~ carries
//    softmax_scale*log2(e)).  The running reference max only moves when a
//    tile's max exceeds it by more than 8 (so p <= 2^8), which makes the
//    O rescale rare.  P (bf16) and the rescale factors go to LDS.
//  * P.V: wave w owns latent columns [128w, 128w+128) for all heads
//    (O^T blocks of 32 d x 32 heads, v_mfma_f32_32x32x16_bf16, 256 fp32
//    accumulators).  V^T fragments are read from the staged tile with
//    ds_read_b64_tr_b16; P^T fragments with ds_read_b128.
//  * At the end of each (sequence, range) segment the unnormalised O~, the
//    reference max m and the sum l go to the segment's partial slot.
#include "mla_common.h"

namespace mla {
namespace {

constexpr int TT = 48;                  // cached rows per tile
constexpr int ROWB = D_K * 2;           // 1152 bytes per row (bf16)
constexpr int TILEB = TT * ROWB;        // 55,296 bytes
constexpr int NINSTR = TT * 72 / 64;    // 54 DMA instructions of 1 KB per tile
constexpr int PSTR = 112;               // bytes per head row of P in LDS (48 bf16 + pad)
constexpr float RESCALE_T = 8.0f;       // log2 headroom before the reference max moves
constexpr int KS = D_K / 32;            // 18 K-steps of 32 for the score MFMA
constexpr int KS_REG = 14;              // K-steps of the query block kept in VGPRs;
                                        // the last 4 (latent dims 448..511 and the
                                        // RoPE dims) are staged in LDS

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Slot permutation of row r: chunk c lives at slot c ^ swz(r) (swz < 8).
__device__ __forceinline__ int swz(int r) {
  const int t = r >> 1;
  return ((t & 1) << 2) | ((t >> 1) & 3);
}

// The O accumulators are meant to stay in AGPRs for the whole kernel; these
// helpers touch one accumulator through an "a" operand so that the register
// allocator never moves the 256 of them into VGPRs.
#define ACC_SCALE(x, a)                                                                        \
  do {                                                                                         \
    float acc_tmp_;                                                                            \
    asm volatile("v_accvgpr_read_b32 %0, %1\n\tv_mul_f32 %0, %0, %2\n\tv_accvgpr_write_b32 %1, %0" \
                 : "=&v"(acc_tmp_), "+a"(x)                                                    \
                 : "v"(a));                                                                    \
  } while (0)
#define ACC_READ(dst, x) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(dst) : "a"(x))
#define ACC_ZERO(x) asm volatile("v_accvgpr_write_b32 %0, 0" : "=a"(x))

struct TileDesc {
  int32_t b, t0, n;   // sequence, first token in the sequence, rows (0 = none)
  int32_t first, last;
};

// The prefix sums are written by the plan kernel and only read here, so they
// are read through the constant address space (uniform scalar loads).
typedef const __attribute__((address_space(4))) int32_t* cprefix_t;

// Cursor over the tiles of one workgroup's token range [x, P1).
struct Cursor {
  int32_t x, P1, s_beg, s_end, seg_beg;
  int32_t b, B;
  __device__ void init(cprefix_t prefix, int32_t B_, int32_t P0, int32_t P1_) {
    B = B_;
    P1 = P1_;
    x = P0;
    if (x < P1) {
      int32_t lo = 0, hi = B - 1;   // last b with prefix[b] <= x
      while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= x) lo = mid; else hi = mid - 1;
      }
      b = lo;
      s_beg = prefix[b];
      s_end = prefix[b + 1];
    } else {
      b = 0;
      s_beg = s_end = 0;
    }
    seg_beg = x;
  }
  __device__ TileDesc next(cprefix_t prefix) {
    TileDesc t;
    if (x >= P1) {
      t.b = 0; t.t0 = 0; t.n = 0; t.first = 0; t.last = 0;
      return t;
    }
    const int32_t seg_end = s_end < P1 ? s_end : P1;
    t.b = b;
    t.t0 = x - s_beg;
    t.n = (seg_end - x) < TT ? (seg_end - x) : TT;
    t.first = (x == seg_beg);
    x += t.n;
    t.last = (x == seg_end);
    if (t.last && x < P1) {
      // move to the next sequence holding tokens (skip empty ones)
      do {
        ++b;
        s_beg = s_end;
        s_end = prefix[b + 1];
      } while (s_end <= x && b < B - 1);
      seg_beg = x;
    }
    return t;
  }
};

template <int NW>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_mfma_kernel(const bf16* __restrict__ qabs, const bf16* __restrict__ c_KV, const bf16* __restrict__ k_R,
                   int64_t row_stride, int32_t num_pages, const int32_t* __restrict__ page_table,
                   int32_t max_pages, int32_t page_size, const int32_t* __restrict__ prefix, int32_t B,
                   int32_t G, float* __restrict__ part_ml, float* __restrict__ part_o,
                   int32_t* __restrict__ flags) {
  constexpr int NH = 32 * NW;
  constexpr int IPW = (NINSTR + NW - 1) / NW;   // DMA instructions per wave
  constexpr int DB = 16 / NW;                   // 32-wide latent blocks per wave in P.V
  __shared__ __attribute__((aligned(1024))) char kt0[TILEB];
  __shared__ __attribute__((aligned(1024))) char kt1[TILEB];
  __shared__ __attribute__((aligned(16))) char pl[NH * PSTR];
  __shared__ __attribute__((aligned(1024))) char ql[NH * 256];   // query dims 448..575, swizzled
  __shared__ float alpha_l[NH];
  __shared__ int resc_l[NW];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t N = ((cprefix_t)prefix)[B];
  const int32_t P0 = (int32_t)split_begin(blockIdx.x, N, G), P1 = (int32_t)split_begin(blockIdx.x + 1, N, G);
  if (P0 >= P1) return;

  // ---- per-lane constant offsets
  // score A fragment (16x16x32): row 16tb + (lane&15), chunk 4ks + (lane>>4)
  const int a_row = lane & 15, a_g = lane >> 4;
  const int a_sw = swz(a_row);
  // slot of chunk 4ks + g is 8*(ks>>1) + 4*((ks&1) ^ (sw>>2)) + (g ^ (sw&3))
  const int a_off_even = a_row * ROWB + (4 * (a_sw >> 2) + (a_g ^ (a_sw & 3))) * 16;
  const int a_off_odd = a_row * ROWB + (4 * (1 - (a_sw >> 2)) + (a_g ^ (a_sw & 3))) * 16;
  // V^T fragment (ds_read_b64_tr_b16): source lane s reads row kc*16 + 8*(s>>5) + 4rr + ((s&15)>>2),
  // columns 32*dblk + 16*((s>>4)&1) + 4*(s&3) .. +3
  const int v_row = 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int v_colc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);   // chunk within the 32-column block
  const int v_half = (lane & 1) * 8;                                // byte within the chunk
  int v_off[2][2];  // [rr][dblk parity]
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int r = v_row + 4 * rr;     // kc*16 adds a multiple of 16: same swizzle
    const int sw = swz(r);
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      // chunk (4*dblk + v_colc) ^ sw, dblk parity par; the dblk-dependent part
      // 4*dblk ^ 4*(sw>>2) is 4*(dblk ^ (sw>>2)): for parity par this is
      // 4*dblk + 4*((par ^ (sw>>2)) - par)
      const int dpar = 4 * ((par ^ (sw >> 2)) - par);
      v_off[rr][par] = r * ROWB + (dpar + (v_colc ^ (sw & 3))) * 16 + v_half;
    }
  }
  // P^T fragment: head 32hb + (lane&31), tokens kc*16 + 8*(lane>>5)
  const int p_off = (lane & 31) * PSTR + (lane >> 5) * 16;

  const cprefix_t cpre = (cprefix_t)prefix;
  Cursor cur;
  cur.init(cpre, B, P0, P1);
  TileDesc t_now = cur.next(cpre);     // tile being computed
  TileDesc t_nxt = cur.next(cpre);     // tile whose rows are in flight

  // Row lookup for a tile in two halves: fetch() issues the page-table load
  // (lane r < TT handles tile row r) and its result is only consumed by
  // resolve() one tile later, so no wait on it lands inside a tile's compute.
  struct RowFetch {
    int32_t page, slot;
  };
  auto fetch_rows = [&](const TileDesc& td) -> RowFetch {
    RowFetch f;
    if (td.n <= 0) {
      f.page = 0;
      f.slot = 0;
      return f;
    }
    int r = lane < TT ? lane : TT - 1;
    if (r >= td.n) r = td.n - 1;
    const int t = td.t0 + r;
    f.page = page_table[(int64_t)td.b * max_pages + t / page_size];
    f.slot = t % page_size;
    return f;
  };
  auto resolve_rows = [&](const RowFetch& f) -> int32_t {
    int32_t pg = f.page;
    if (pg < 0 || pg >= num_pages) {
      atomicOr(flags, MLA_FLAG_BAD_PAGE);
      pg = pg < 0 ? 0 : num_pages - 1;
    }
    return pg * page_size + f.slot;
  };
  const char* cbase = (const char*)c_KV;
  const char* kbase = (const char*)k_R;
  const int64_t stride_b = row_stride * 2;
  auto issue_dma = [&](char* kt, int32_t ridx) {
    // Recomputed for every tile (the empty asm hides the lane id from loop
    // invariant hoisting, which would otherwise keep 14 addresses live).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    int wv = __builtin_amdgcn_readfirstlane(wave);
    asm volatile("" : "+s"(wv));
#pragma unroll
    for (int k = 0; k < IPW; ++k) {
      const int I = wv * IPW + k;
      if (I < NINSTR) {
        const int sigma = I * 64 + ln;
        const int row = sigma / 72;
        const int posn = sigma - row * 72;
        const int chunk = posn ^ swz(row);
        const int ra = (I * 64) / 72;
        const int rb = ra + 1 < TT ? ra + 1 : TT - 1;
        const int rid_a = __builtin_amdgcn_readlane(ridx, ra);
        const int rid_b = __builtin_amdgcn_readlane(ridx, rb);
        const int64_t rid = row == ra ? rid_a : rid_b;
        const char* src = (chunk < 64 ? cbase : kbase) + rid * stride_b + (chunk & 63) * 16;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(kt + I * 1024), 16, 0, 0);
      }
    }
  };

  // ---- state
  bf16x8 q[2][KS_REG];
  f32x16 o[NW][DB];
  float m_ref[2], l_sum[2];

  auto load_q = [&](int32_t b) {
    int ln = lane;   // hidden from hoisting, as in issue_dma
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const bf16* qp = qabs + ((int64_t)b * NH + 32 * wave + 16 * hb + (ln & 15)) * D_K + 8 * (ln >> 4);
#pragma unroll
      for (int ks = 0; ks < KS_REG; ++ks) q[hb][ks] = *(const bf16x8*)(qp + 32 * ks);
    }
    // dims 448..575 of this wave's 32 heads -> ql, 16-byte chunk c of head h
    // at position c ^ (h & 15)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sigma = 64 * j + ln;
      const int hl = sigma >> 4, c = (sigma & 15) ^ (hl & 15);
      const bf16* src = qabs + ((int64_t)b * NH + 32 * wave + hl) * D_K + 32 * KS_REG + 8 * c;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(ql + wave * 8192 + j * 1024), 16, 0, 0);
    }
  };
  auto reset_state = [&]() {
#pragma unroll
    for (int hb = 0; hb < NW; ++hb)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) ACC_ZERO(o[hb][db][r]);
    m_ref[0] = m_ref[1] = -INFINITY;
    l_sum[0] = l_sum[1] = 0.f;
  };

  // ---- prologue: rows of tile 0 -> kt0, row indices of tile 1 ready
  {
    issue_dma(kt0, resolve_rows(fetch_rows(t_now)));
  }
  RowFetch rows_next = fetch_rows(t_nxt);
  load_q(t_now.b);
  reset_state();

  auto process = [&](char* kt, char* kt_other) {
    // tile t_now is (being) loaded into kt; t_nxt goes to kt_other
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of t_now (and q) have landed
    __syncthreads();                 // everyone's copies landed; P.V of the previous tile done
    if (t_nxt.n > 0) issue_dma(kt_other, resolve_rows(rows_next));
    TileDesc t_after = cur.next(cpre);
    rows_next = fetch_rows(t_after);

    // ---- scores S^T[token][head] for this wave's 32 heads
    f32x4 s[3][2];
#pragma unroll
    for (int tb = 0; tb < 3; ++tb)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) s[tb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = (ks & 1 ? a_off_odd : a_off_even) + 128 * (ks >> 1);
      bf16x8 qb0, qb1;
      if (ks < KS_REG) {
        qb0 = q[0][ks];
        qb1 = q[1][ks];
      } else {
        const int c = 4 * (ks - KS_REG) + (lane >> 4);
        const int qo = (32 * wave + (lane & 15)) * 256 + ((c ^ (lane & 15)) << 4);
        qb0 = *(const bf16x8*)(ql + qo);
        qb1 = *(const bf16x8*)(ql + qo + 16 * 256);
      }
#pragma unroll
      for (int tb = 0; tb < 3; ++tb) {
        const bf16x8 a = *(const bf16x8*)(kt + off + tb * 16 * ROWB);
        s[tb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb0, s[tb][0], 0, 0, 0);
        s[tb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb1, s[tb][1], 0, 0, 0);
      }
    }
    // the next sequence's query can be loaded once this segment's scores are done
    if (t_now.last && t_nxt.n > 0) load_q(t_nxt.b);

    // ---- online softmax (owner wave), lane holds heads 32w + 16hb + (lane&15)
    const int n_valid = t_now.n;
    int any_resc = 0;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float mx = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 3; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 16 * tb + 4 * (lane >> 4) + i;
          if (tok >= n_valid) s[tb][hb][i] = -INFINITY;
          mx = fmaxf(mx, s[tb][hb][i]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      float alpha = 1.f;
      if (t_now.first) {
        // a new segment: the accumulators restart from zero (alpha = 0)
        alpha = 0.f;
        any_resc = 1;
        m_ref[hb] = mx;
      } else if (mx > m_ref[hb] + RESCALE_T) {
        if (m_ref[hb] != -INFINITY) {
          alpha = __builtin_amdgcn_exp2f(m_ref[hb] - mx);
          any_resc = 1;
        }
        m_ref[hb] = mx;
      }
      float sum = 0.f;
#pragma unroll
      for (int tb = 0; tb < 3; ++tb) {
        bf16x4 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(s[tb][hb][i] - m_ref[hb]);
          pb[i] = (bf16)p;
          sum += (float)pb[i];
        }
        const int head = 32 * wave + 16 * hb + (lane & 15);
        *(bf16x4*)(pl + head * PSTR + (16 * tb + 4 * (lane >> 4)) * 2) = pb;
      }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      l_sum[hb] = l_sum[hb] * alpha + sum;
      if (lane < 16) alpha_l[32 * wave + 16 * hb + lane] = alpha;
    }
    const int wave_resc = __builtin_amdgcn_readfirstlane(__any(any_resc) ? 1 : 0);
    if (lane == 0) resc_l[wave] = wave_resc;
    // P, alpha visible to all waves.  Only LDS traffic is waited for: a plain
    // __syncthreads would also wait for the next tile's copies in flight.
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt untouched
    __builtin_amdgcn_s_barrier();

    // ---- rescale O if any owner moved its reference max
    int resc = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) resc |= resc_l[w];
    if (resc) {
#pragma unroll
      for (int hb = 0; hb < NW; ++hb) {
        const float a = alpha_l[32 * hb + (lane & 31)];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) ACC_SCALE(o[hb][db][r], a);
      }
    }

    // ---- O^T[d][head] += V^T[d][tok] P^T[tok][head]
#pragma unroll
    for (int kc = 0; kc < 3; ++kc) {
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 pf[NW];
#pragma unroll
      for (int hb = 0; hb < NW; ++hb)
        pf[hb] = *(const bf16x8*)(pl + 32 * hb * PSTR + p_off + kc * 32);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int dblk = DB * wave + db;
        const int par = db & 1;   // DB is even, so dblk parity == db parity
        const int base = kc * 16 * ROWB;
        const int c0 = 64 * dblk;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(kt + base + v_off[0][par] + c0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(kt + base + v_off[1][par] + c0));
        bf16x8 vf;
        const bf16x4 lob = __builtin_bit_cast(bf16x4, lo), hib = __builtin_bit_cast(bf16x4, hi);
        vf[0] = lob[0]; vf[1] = lob[1]; vf[2] = lob[2]; vf[3] = lob[3];
        vf[4] = hib[0]; vf[5] = hib[1]; vf[6] = hib[2]; vf[7] = hib[3];
#pragma unroll
        for (int hb = 0; hb < NW; ++hb)
          o[hb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[hb], o[hb][db], 0, 0, 0);
      }
    }

    // ---- segment end: write the partial (O~ unnormalised, m, l)
    if (t_now.last) {
      const int64_t slot = (int64_t)blockIdx.x + t_now.b;
#pragma unroll
      for (int hb = 0; hb < NW; ++hb) {
        const int head = 32 * hb + (lane & 31);
        float* dst = part_o + (slot * NH + head) * D_C;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d0 = 32 * (DB * wave + db) + 4 * (lane >> 5);
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            f32x4 v;
            ACC_READ(v[0], o[hb][db][4 * r4]);
            ACC_READ(v[1], o[hb][db][4 * r4 + 1]);
            ACC_READ(v[2], o[hb][db][4 * r4 + 2]);
            ACC_READ(v[3], o[hb][db][4 * r4 + 3]);
            *(f32x4*)(dst + d0 + 8 * r4) = v;
          }
        }
      }
      if (lane < 16) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int head = 32 * wave + 16 * hb + lane;
          part_ml[(slot * NH + head) * 2 + 0] = m_ref[hb];
          part_ml[(slot * NH + head) * 2 + 1] = l_sum[hb];
        }
      }
      m_ref[0] = m_ref[1] = -INFINITY;
      l_sum[0] = l_sum[1] = 0.f;
    }
    t_now = t_nxt;
    t_nxt = t_after;
  };

  while (true) {
    process(kt0, kt1);
    if (t_now.n <= 0) break;
    process(kt1, kt0);
    if (t_now.n <= 0) break;
  }
}

}  // namespace

hipError_t launch_decode_mfma(const mla_dims& d, int32_t B, const void* qabs, const void* c_KV,
                              const void* k_R, int64_t row_stride, int32_t num_pages,
                              const int32_t* page_table, int32_t max_pages, const int32_t* prefix,
                              int32_t n_splits, float* part_ml, float* part_o, int32_t* flags,
                              hipStream_t s) {
  const int nw = d.n_h / 32;
  dim3 grid(n_splits);
  switch (nw) {
    case 1:
      decode_mfma_kernel<1><<<grid, 64, 0, s>>>((const bf16*)qabs, (const bf16*)c_KV, (const bf16*)k_R,
                                               row_stride, num_pages, page_table, max_pages, d.page_size,
                                               prefix, B, n_splits, part_ml, part_o, flags);
      break;
    case 2:
      decode_mfma_kernel<2><<<grid, 128, 0, s>>>((const bf16*)qabs, (const bf16*)c_KV, (const bf16*)k_R,
                                                row_stride, num_pages, page_table, max_pages, d.page_size,
                                                prefix, B, n_splits, part_ml, part_o, flags);
      break;
    case 4:
      decode_mfma_kernel<4><<<grid, 256, 0, s>>>((const bf16*)qabs, (const bf16*)c_KV, (const bf16*)k_R,
                                                row_stride, num_pages, page_table, max_pages, d.page_size,
                                                prefix, B, n_splits, part_ml, part_o, flags);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
