// Sparse top-k decode, selection half: the indexer's relevance scores and the
// choice of the k most relevant cached tokens of every sequence (gfx950).
//
// What it computes (reading of "DeepSeek 架构精讲：从 V3 到 V4" (cyco.top),
// §4 V3.2 bullet and §6 question 7, which say only that a light indexer
// picks the few most relevant tokens before attention): every cached token j
// carries an indexer key k^I_j (d_I = 128 bf16, in a paged pool that shares
// the latent cache's page table); a decode query carries H_I indexer heads
// q^I_h and weights w_h; the relevance is
//   I_j = sum_h w_h * max(0, q^I_h . k^I_j)                      (fp32)
// and the kept set is the k largest I_j, equal scores going to the smaller
// token index (every token when n <= k), listed in ascending token order.
//
//  * indexer_kernel: S[token][head] = K^I . Q^I^T on the matrix cores
//    (v_mfma_f32_16x16x32_bf16), then ReLU, the head weights and the sum
//    over heads (in registers, then across the 16 lanes of a row).  A wave
//    takes 32 blocks of 16 tokens; each block's 4 KB of keys is copied HBM
//    -> LDS by 4 global_load_lds instructions of one whole KB each (chunk c
//    of row r at position c ^ r, so the fragment reads hit 16 distinct bank
//    groups), IDX_PF blocks ahead of the one computed.  Bound by HBM: 256 B
//    of keys per token against 2 H_I d_I flops.
//  * Selection: a radix select on order-preserving 32-bit keys of the fp32
//    scores, three passes of 11, 11 and 10 bits (the first one's histogram
//    inside the indexer kernel, on the scores it has just formed).  Each
//    pass histograms the keys that match the bits fixed so far (LDS
//    atomics, then integer atomics into a per-sequence histogram when a
//    sequence spans several workgroups); a pick kernel (or the sequence's
//    only workgroup) then finds the bin where the count of keys from the top
//    reaches k and fixes those bits.  After three passes the threshold key T
//    and the number r of ties at T to keep are known.  A count pass (several
//    chunks only) and a write pass then list, in token order, every token
//    with key > T and the first r tokens with key == T, with their pool rows
//    (page-table lookups) for the gather attention.  When every sequence fits
//    one chunk, select_local_kernel does passes 1 and 2, the picks and the
//    listing in one launch, a workgroup per sequence with its scores in LDS.
//    Integer work only: the result is exact and deterministic.
#include <type_traits>

#include "mla_common.h"

namespace mla {
namespace {

constexpr int IDX_D = 128;                 // indexer key width d_I
constexpr int IDX_KS = IDX_D / 32;         // K-steps of the 16x16x32 MFMA
constexpr int IDX_BPW = 16;                // 16-token blocks per wave
constexpr int IDX_PF = 2;                  // blocks whose keys are in flight ahead of the one computed
constexpr int IDX_TOK_WG = 4 * IDX_BPW * 16;   // 1024 tokens per workgroup (4 waves)
constexpr int SEL_NT = 1024;               // threads of a selection pass workgroup
constexpr int SEL_RT = 4 * SEL_NT;         // tokens per round of a selection pass: a float4 per thread
constexpr int SEL_MAXR = SEL_CH / SEL_RT;  // rounds per chunk
constexpr int SEL_RB = 8;                  // rounds whose loads are issued together
static_assert(SEL_CH % SEL_RT == 0 && SEL_MAXR * (SEL_NT / 64) <= SEL_NT, "one scan entry per (round, wave)");

// Order-preserving key of an fp32 score: a larger score has a larger key;
// -0 is taken as +0 so that the two zeros tie, as they compare equal.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int32_t clamp_len(int32_t n, int32_t max_tokens) {
  return n < 1 ? 0 : (n > max_tokens ? max_tokens : n);
}

// Adds 1 to h[bin] for every active lane, one LDS atomic per distinct bin
// of the wave (scores cluster, so most lanes of a wave share a few bins).
__device__ __forceinline__ void wave_hist_add(int32_t* h, bool active, uint32_t bin) {
  const int lane = threadIdx.x & 63;
  uint64_t m = __ballot(active);
  while (m) {
    const int leader = __ffsll((unsigned long long)m) - 1;
    const uint32_t lb = (uint32_t)__shfl((int)bin, leader);
    const uint64_t same = __ballot(active && bin == lb);
    if (lane == leader) atomicAdd(&h[lb], (int32_t)__popcll(same));
    active = active && bin != lb;
    m &= ~same;
  }
}

// Radix digit of pass PASS: bits 31..21, 20..10, 9..0 of the key; the bits
// above them must equal those fixed by the earlier passes.
template <int PASS> struct Digit {
  static constexpr int SHIFT = PASS == 0 ? 21 : (PASS == 1 ? 10 : 0);
  static constexpr uint32_t HIMASK = PASS == 0 ? 0u : (PASS == 1 ? 0xFFE00000u : 0xFFFFFC00u);
  static constexpr uint32_t BMASK = PASS == 2 ? 0x3FFu : 0x7FFu;
};

// HBM -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane i's
// chunk lands at LDS byte lds_base + 16 i.  Issued through asm, so the
// compiler does not track the LDS write: the reader waits with wait_vm.  m0
// (the LDS base) is written before the copy and not restored: an m0 write
// right behind a copy waits until the copy has left the wave's memory queue.
// m0 is a register the compiler reserves, and clang warns that a clobber of
// it is not preserved for the compiler; nothing the compiler emits in this
// file reads m0 (tests/test_isa_m0.py checks the built code), so the warning
// is silenced here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "s"(lds_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ uint32_t lds_addr(const char* p) { return (uint32_t)(uintptr_t)(lds_void*)p; }
// Waits until at most N vector memory instructions of this wave are in
// flight; also a compiler barrier for memory accesses.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// The same for blocks: at most 4 nb copy instructions (nb blocks) in flight;
// nb is a constant once the caller's loop is unrolled.
__device__ __forceinline__ void wait_blocks(int nb) {
  static_assert(IDX_PF <= 4, "cases below");
  switch (nb) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<4>(); break;
    case 2: wait_vm<8>(); break;
    default: wait_vm<12>(); break;
  }
}

// The digit of pass PASS for sequence b from its histogram `bins` (LDS or,
// from_global, the global one read with agent-scope loads, which the L1 and
// the XCD's L2 do not serve): the bin where the count of keys from the top
// reaches the number still to keep.  st_b: {key bits fixed so far, ties
// still to take, every token kept}.  NT threads; part: NT ints of LDS.
template <int PASS, int NT>
__device__ void pick_digit(const int32_t* bins, bool from_global, int32_t* st_b, int32_t top_k, int32_t* part) {
  constexpr int BPT = SEL_BINS / NT;   // bins per thread
  const int tid = threadIdx.x;
  const uint32_t fixed = PASS == 0 ? 0u : (uint32_t)st_b[0];
  const int32_t rem = PASS == 0 ? top_k : st_b[1];
  int32_t c[BPT], tot = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    c[j] = from_global ? __hip_atomic_load(&bins[BPT * tid + j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                       : bins[BPT * tid + j];
    tot += c[j];
  }
  part[tid] = tot;   // suffix sums over the thread totals
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const int32_t v = tid + off < NT ? part[tid + off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t above = part[tid] - tot;   // keys in the bins above this thread's
#pragma unroll
  for (int j = BPT - 1; j >= 0; --j) {
    if (above < rem && rem <= above + c[j]) {
      st_b[0] = (int32_t)(fixed | ((uint32_t)(BPT * tid + j) << Digit<PASS>::SHIFT));
      st_b[1] = rem - above;
      st_b[2] = 0;
    }
    above += c[j];
  }
}

// Clears every sequence's three global histograms (one per radix pass)
// before the first pass.
__global__ void __launch_bounds__(256) select_clear_kernel(int32_t* __restrict__ hist, int32_t B) {
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    int4* h = (int4*)(hist + ((int64_t)pass * B + blockIdx.x) * SEL_BINS);
    for (int i = threadIdx.x; i < SEL_BINS / 4; i += 256) h[i] = int4{0, 0, 0, 0};
  }
}

// Relevance scores of one 1024-token range of one sequence (blockIdx.y), and
// the histogram of the first radix digit of its scores (added to the
// sequence's pass-0 global histogram, which select_hist_kernel<1> reads).
template <int HB>
__global__ void __launch_bounds__(256) indexer_kernel(const bf16* __restrict__ q_I, const float* __restrict__ w_I,
                                                      const bf16* __restrict__ k_I, int64_t idx_stride,
                                                      int32_t num_pages, const int32_t* __restrict__ page_table,
                                                      int32_t max_pages, int32_t page_size,
                                                      const int32_t* __restrict__ seq_lens, int32_t max_tokens,
                                                      int32_t top_k, float* __restrict__ scores,
                                                      int32_t* __restrict__ hist, int32_t* __restrict__ flags) {
  __shared__ int32_t h[SEL_BINS];
  __shared__ __attribute__((aligned(1024))) char ring[4][IDX_PF][16 * IDX_D * 2];
  const int32_t b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int i = threadIdx.x; i < SEL_BINS; i += 256) h[i] = 0;
  __syncthreads();
  const int32_t n = clamp_len(seq_lens[b], max_tokens);
  const bool all = n <= top_k;
  const int32_t t_wave = blockIdx.x * IDX_TOK_WG + wave * IDX_BPW * 16;
  if (t_wave < n) {
    // S^T[head][token] = Q^I . K^I^T: A operands (query) head 16hb +
    // (lane&15), dims 32ks + 8(lane>>4) .. +7; the result block leaves heads
    // 16hb + 4(lane>>4) + r, r = 0..3, of token t0 + (lane&15) in the lane,
    // so the sum over heads is in-lane plus a 4-lane exchange.
    bf16x8 qf[HB][IDX_KS];
    float wv[HB][4];
    const bf16* qb = q_I + (int64_t)b * HB * 16 * IDX_D;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) wv[hb][r] = w_I[(int64_t)b * HB * 16 + 16 * hb + 4 * (lane >> 4) + r];
#pragma unroll
      for (int ks = 0; ks < IDX_KS; ++ks)
        qf[hb][ks] = *(const bf16x8*)(qb + (16 * hb + (lane & 15)) * IDX_D + 32 * ks + 8 * (lane >> 4));
    }
    // page id of block i in lane i (a block of 16 tokens lies in one page:
    // page_size is a multiple of 16)
    const int32_t* pt = page_table + (int64_t)b * max_pages;
    int32_t pgv = 0;
    {
      const int32_t t0 = min(t_wave + 16 * lane, n - 1);
      if (lane < IDX_BPW) {
        pgv = pt[t0 / page_size];
        if (pgv < 0 || pgv >= num_pages) {
          atomicOr(flags, MLA_FLAG_BAD_PAGE);
          pgv = pgv < 0 ? 0 : num_pages - 1;
        }
      }
    }
    // Copy of block i into ring slot i % IDX_PF: instruction j fetches rows
    // 4j .. 4j+3 (lane l: row 4j + (l>>4), chunk (l&15) ^ row), one whole
    // KB of the pool.  Rows past the sequence's end repeat its last row;
    // every block of the wave is copied (past n too), so that the counts
    // of instructions in flight stay fixed.
    char* rw = ring[wave][0];
    auto dma_blk = [&](int i) __attribute__((always_inline)) {
      const int32_t t0 = min(t_wave + 16 * i, n - 1) & ~15;
      const int32_t p = t0 / page_size;
      const int32_t pg = __builtin_amdgcn_readlane(pgv, min(i, (n - 1 - t_wave) >> 4));
      char* slot = rw + (i % IDX_PF) * (16 * IDX_D * 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * j + (lane >> 4);
        const int32_t t = min(t0 + r, n - 1);
        const char* src = (const char*)(k_I + ((int64_t)pg * page_size + (t - p * page_size)) * idx_stride) +
                          16 * ((lane & 15) ^ r);
        dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(slot + 1024 * j)));
      }
    };
#pragma unroll
    for (int i = 0; i < IDX_PF; ++i) dma_blk(i);
    float sc[IDX_BPW];   // the score of token t0 + (lane&15) of block i
#pragma unroll
    for (int i = 0; i < IDX_BPW; ++i) {
      const int32_t t0 = t_wave + 16 * i;
      if (t0 >= n) break;
      wait_blocks(min(IDX_PF - 1, IDX_BPW - 1 - i));   // block i landed
      // B operands: token t0 + (lane&15) (row lane&15 of the slot), chunk 4ks + (lane>>4)
      const char* slot = rw + (i % IDX_PF) * (16 * IDX_D * 2);
      const int r = lane & 15;
      bf16x8 af[IDX_KS];
#pragma unroll
      for (int ks = 0; ks < IDX_KS; ++ks)
        af[ks] = *(const bf16x8*)(slot + r * (IDX_D * 2) + 16 * ((4 * ks + (lane >> 4)) ^ r));
      f32x4 acc[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < IDX_KS; ++ks)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
          acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[hb][ks], af[ks], acc[hb], 0, 0, 0);
      // the slot's reads are done (the MFMAs consumed them): refill it
      if (i + IDX_PF < IDX_BPW) dma_blk(i + IDX_PF);
      // this lane's heads, then the four lanes l, l^16, l^32, l^48 of the token
      float x = 0.f;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int r = 0; r < 4; ++r) x += wv[hb][r] * fmaxf(acc[hb][r], 0.f);
      const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      x = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
      const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      x = __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
      sc[i] = x;
      wave_hist_add(h, lane < 16 && t0 + lane < n && !all, score_key(x) >> Digit<0>::SHIFT);
    }
    wait_vm<0>();   // no copy still writing the ring when the wave leaves
    float* sb = scores + (int64_t)b * max_tokens;
#pragma unroll
    for (int i = 0; i < IDX_BPW; ++i) {
      const int32_t t = t_wave + 16 * i + lane;
      if (lane < 16 && t < n) sb[t] = sc[i];
    }
  }
  __syncthreads();
  if (!all) {
    int32_t* hb = hist + (int64_t)b * SEL_BINS;
    for (int i = threadIdx.x; i < SEL_BINS; i += 256)
      if (h[i]) atomicAdd(&hb[i], h[i]);
  }
}

// Radix pass PASS (1 or 2) over one SEL_CH-token chunk of one sequence.
// The digit of the pass before comes from that pass's global histogram,
// picked by every workgroup of the sequence (they all find the same); with a
// single chunk per sequence (local) pass 2 instead starts from the state
// pass 1 left.  local: the workgroup then picks this pass's digit from its
// own histogram and stores the resulting state; otherwise it adds its
// histogram to the sequence's global one of this pass (the next kernel picks
// from it), and chunk 0 stores the state before this pass.
// State planes (st, {key bits fixed, ties still to take, every token kept}
// per sequence): 0 after pass 0, 1 after pass 1, 2 final.  Sequences that
// keep every token get {0, 0, 1} in plane 2 here.
template <int PASS>
__global__ void __launch_bounds__(SEL_NT) select_hist_kernel(const float* __restrict__ scores, int32_t max_tokens,
                                                          const int32_t* __restrict__ seq_lens, int32_t top_k,
                                                          int32_t* __restrict__ hist, int32_t B,
                                                          int32_t* __restrict__ st, bool local) {
  using D = Digit<PASS>;
  __shared__ int32_t h[SEL_BINS];
  __shared__ int32_t part[SEL_NT];
  __shared__ int32_t st_l[4];
  const int32_t b = blockIdx.y;
  const int tid = threadIdx.x;
  const int32_t n = clamp_len(seq_lens[b], max_tokens);
  if (n <= top_k) {   // every token kept
    if (PASS == 1 && blockIdx.x == 0 && tid < 3) st[(2 * B + b) * 4 + tid] = tid == 2 ? 1 : 0;
    return;
  }
  if (tid < 3) st_l[tid] = PASS == 1 || !local ? (PASS == 1 ? 0 : st[b * 4 + tid]) : st[(B + b) * 4 + tid];
  __syncthreads();
  if (PASS == 1 || !local) {
    pick_digit<PASS - 1, SEL_NT>(hist + ((int64_t)(PASS - 1) * B + b) * SEL_BINS, true, st_l, top_k, part);
    __syncthreads();
  }
  const uint32_t fixed = (uint32_t)st_l[0];
  for (int i = tid; i < SEL_BINS; i += SEL_NT) h[i] = 0;
  __syncthreads();
  const int32_t c0 = blockIdx.x * SEL_CH, c1 = min(c0 + SEL_CH, n);
  const float* sb = scores + (int64_t)b * max_tokens;
  // a float4 per thread and round (coalesced); the bins below the fixed
  // bits are spread, so plain LDS atomics (distinct addresses) serve best
  for (int32_t rb = c0; rb < c1; rb += SEL_RB * SEL_RT) {
    float4 v[SEL_RB];   // SEL_RB rounds' loads in flight together
#pragma unroll
    for (int j = 0; j < SEL_RB; ++j) {
      const int32_t t = rb + j * SEL_RT + 4 * tid;
      v[j] = t < c1 ? *(const float4*)(sb + t) : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < SEL_RB; ++j) {
      const int32_t t = rb + j * SEL_RT + 4 * tid;
      const float x[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = score_key(x[e]);
        if (t + e < c1 && (key & D::HIMASK) == fixed) atomicAdd(&h[(key >> D::SHIFT) & D::BMASK], 1);
      }
    }
  }
  __syncthreads();
  if (local) {
    pick_digit<PASS, SEL_NT>(h, false, st_l, top_k, part);
    __syncthreads();
    if (tid < 3) st[((PASS == 1 ? 1 : 2) * B + b) * 4 + tid] = st_l[tid];
  } else {
    int32_t* hb = hist + ((int64_t)PASS * B + b) * SEL_BINS;
    for (int i = tid; i < SEL_BINS; i += SEL_NT)
      if (h[i]) atomicAdd(&hb[i], h[i]);
    if (blockIdx.x == 0 && tid < 3) st[((PASS - 1) * B + b) * 4 + tid] = st_l[tid];
  }
}

// Block-wide (SEL_NT threads) exclusive prefix sum of v and the block total.
// wsum: SEL_NT / 64 ints of LDS; the caller syncs before reusing it.
__device__ __forceinline__ int32_t block_excl_sum(int32_t v, int32_t* wsum, int32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t x = v;   // inclusive scan within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int32_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < SEL_NT / 64; ++w) {
    const int32_t c = wsum[w];
    before += w < wave ? c : 0;
    total += c;
  }
  return before + x - v;
}

// Kept tokens of one chunk: {key > T, key == T}, or {all, 0}.
// Several chunks per sequence only: the last digit is first picked from the
// pass-2 global histogram (by every workgroup of the sequence), and chunk 0
// stores the final state (plane 2) for select_write_kernel.
__global__ void __launch_bounds__(SEL_NT) select_count_kernel(const float* __restrict__ scores, int32_t max_tokens,
                                                           const int32_t* __restrict__ seq_lens, int32_t top_k,
                                                           const int32_t* __restrict__ hist, int32_t B,
                                                           int32_t* __restrict__ st, int32_t* __restrict__ cnt,
                                                           int32_t nchunks) {
  __shared__ int32_t wsum[2][SEL_NT / 64];
  __shared__ int32_t part[SEL_NT];
  __shared__ int32_t st_l[4];
  const int32_t b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t n = clamp_len(seq_lens[b], max_tokens);
  const bool all = n <= top_k;
  if (!all) {
    if (tid < 3) st_l[tid] = st[(B + b) * 4 + tid];
    __syncthreads();
    pick_digit<2, SEL_NT>(hist + ((int64_t)2 * B + b) * SEL_BINS, true, st_l, top_k, part);
    __syncthreads();
    if (blockIdx.x == 0 && tid < 3) st[(2 * B + b) * 4 + tid] = st_l[tid];
  }
  const uint32_t T = all ? 0u : (uint32_t)st_l[0];
  const int32_t c0 = blockIdx.x * SEL_CH, c1 = min(c0 + SEL_CH, n);
  int32_t gt = 0, eq = 0;
  const float* sb = scores + (int64_t)b * max_tokens;
  for (int32_t rb = c0; rb < c1; rb += SEL_RB * SEL_RT) {
    float4 v[SEL_RB];
#pragma unroll
    for (int j = 0; j < SEL_RB; ++j) {
      const int32_t t = rb + j * SEL_RT + 4 * tid;
      v[j] = t < c1 && !all ? *(const float4*)(sb + t) : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < SEL_RB; ++j) {
      const int32_t t = rb + j * SEL_RT + 4 * tid;
      const float x[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (t + e < c1) {
          const uint32_t key = score_key(x[e]);
          gt += all || key > T;
          eq += !all && key == T;
        }
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    gt += __shfl_xor(gt, off);
    eq += __shfl_xor(eq, off);
  }
  if (lane == 0) {
    wsum[0][wave] = gt;
    wsum[1][wave] = eq;
  }
  __syncthreads();
  if (tid == 0) {
    int32_t g = 0, e = 0;
#pragma unroll
    for (int w = 0; w < SEL_NT / 64; ++w) {
      g += wsum[0][w];
      e += wsum[1][w];
    }
    int32_t* o = cnt + ((int64_t)b * nchunks + blockIdx.x) * 2;
    o[0] = g;
    o[1] = e;
  }
}

// Exclusive prefix sum of v over the lanes of a wave.
__device__ __forceinline__ int32_t wave_excl_sum(int32_t v) {
  const int lane = threadIdx.x & 63;
  int32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x - v;
}

// Lists the kept tokens of one chunk, in token order, with their pool rows.
// The chunk is read in rounds of SEL_RT tokens, wave w of round r taking 256
// consecutive tokens, 4 per lane (coalesced float4 loads).  A first pass
// counts, per (round, wave), the tokens above T and at T; one block scan
// over those entries (in token order) gives each its first rank among the
// ties at T and its first output position; a second pass re-reads the
// scores and places each lane's kept tokens with wave-level prefix sums.
__global__ void __launch_bounds__(SEL_NT) select_write_kernel(const float* __restrict__ scores, int32_t max_tokens,
                                                           const int32_t* __restrict__ seq_lens, int32_t top_k,
                                                           const int32_t* __restrict__ st,
                                                           const int32_t* __restrict__ cnt, int32_t nchunks,
                                                           const int32_t* __restrict__ page_table, int32_t max_pages,
                                                           int32_t page_size, int32_t num_pages,
                                                           int32_t* __restrict__ sel_tok, int32_t* __restrict__ sel_row,
                                                           int32_t* __restrict__ flags) {
  constexpr int NWV = SEL_NT / 64;
  __shared__ int32_t wsum[2][NWV];
  __shared__ int32_t base[2];
  __shared__ int32_t ent_gt[SEL_NT], ent_eq[SEL_NT];   // per (round, wave); then first tie rank / position
  const int32_t b = blockIdx.y, c = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t n = clamp_len(seq_lens[b], max_tokens);
  const int32_t c0 = c * SEL_CH, c1 = min(c0 + SEL_CH, n);
  if (c0 >= c1) return;
  const bool all = st[4 * b + 2] != 0;
  const uint32_t T = (uint32_t)st[4 * b];
  const int32_t rem = st[4 * b + 1];
  // kept-above-T and tied counts of the chunks before this one
  if (tid < 64) {
    int32_t g = 0, e = 0;
    for (int32_t j = tid; j < c; j += 64) {
      g += cnt[((int64_t)b * nchunks + j) * 2];
      e += cnt[((int64_t)b * nchunks + j) * 2 + 1];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      g += __shfl_xor(g, off);
      e += __shfl_xor(e, off);
    }
    if (tid == 0) {
      base[0] = g;
      base[1] = e;
    }
  }
  const float* sb = scores + (int64_t)b * max_tokens;
  const int32_t nr = (c1 - c0 + SEL_RT - 1) / SEL_RT;
  // this lane's first token of round r, and its 4 scores
  auto lane_tok = [&](int32_t r) __attribute__((always_inline)) { return c0 + r * SEL_RT + 256 * wave + 4 * lane; };
  auto load4 = [&](int32_t r) __attribute__((always_inline)) {
    const int32_t t = lane_tok(r);
    return r < nr && t < c1 && !all ? *(const float4*)(sb + t) : float4{0.f, 0.f, 0.f, 0.f};
  };
  // bits e of gtm / eqm: token t + e above T / at T
  auto classify = [&](int32_t t, float4 v, uint32_t& gtm, uint32_t& eqm) __attribute__((always_inline)) {
    gtm = eqm = 0;
    const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = score_key(x[e]);
      const uint32_t in = t + e < c1 ? 1u : 0u;
      gtm |= (in & (all || key > T ? 1u : 0u)) << e;
      eqm |= (in & (!all && key == T ? 1u : 0u)) << e;
    }
  };
  for (int32_t rb = 0; rb < SEL_MAXR; rb += SEL_RB) {   // pass 1: counts per (round, wave)
    float4 v[SEL_RB];
#pragma unroll
    for (int j = 0; j < SEL_RB; ++j) v[j] = load4(rb + j);
#pragma unroll
    for (int j = 0; j < SEL_RB; ++j) {
      const int32_t r = rb + j;
      int32_t g = 0, e = 0;
      if (r < nr) {
        uint32_t gtm, eqm;
        classify(lane_tok(r), v[j], gtm, eqm);
        g = __popc(gtm);
        e = __popc(eqm);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          g += __shfl_xor(g, off);
          e += __shfl_xor(e, off);
        }
      }
      if (lane == 0) {
        ent_gt[r * NWV + wave] = g;
        ent_eq[r * NWV + wave] = e;
      }
    }
  }
  __syncthreads();   // entries and base[] ready
  {
    const bool ent = tid < SEL_MAXR * NWV;   // the rest of the arrays holds no entry
    const int32_t g = ent ? ent_gt[tid] : 0, e = ent ? ent_eq[tid] : 0;
    int32_t tot;
    const int32_t eq_first = base[1] + block_excl_sum(e, wsum[0], tot);
    const int32_t keep = all ? 0 : max(0, min(e, rem - eq_first));   // ties of this entry that are kept
    const int32_t pos_first = base[0] + (all ? 0 : min(base[1], rem)) + block_excl_sum(g + keep, wsum[1], tot);
    __syncthreads();
    ent_eq[tid] = eq_first;
    ent_gt[tid] = pos_first;
  }
  __syncthreads();
  const int32_t* pt = page_table + (int64_t)b * max_pages;
  for (int32_t rb = 0; rb < nr; rb += SEL_RB) {   // pass 2: place the kept tokens
   float4 v[SEL_RB];
   int32_t pgs[SEL_RB];   // page of the lane's 4 tokens (one page: t is a multiple of 4, page_size of 16)
#pragma unroll
   for (int j = 0; j < SEL_RB; ++j) {
     v[j] = load4(rb + j);
     const int32_t t = lane_tok(rb + j);
     pgs[j] = rb + j < nr && t < c1 ? pt[t / page_size] : 0;
   }
#pragma unroll
   for (int j = 0; j < SEL_RB; ++j) {
    const int32_t r = rb + j;
    if (r >= nr) break;
    const int32_t t = lane_tok(r);
    uint32_t gtm, eqm;
    classify(t, v[j], gtm, eqm);
    const int32_t rank = ent_eq[r * NWV + wave] + wave_excl_sum(__popc(eqm));   // of this lane's first tie
    uint32_t keep_eq = 0;
    int32_t k = rank;
    for (uint32_t m = eqm; m; m &= m - 1, ++k)
      if (k < rem) keep_eq |= m & (~m + 1u);
    const uint32_t selm = gtm | keep_eq;
    int32_t pos = ent_gt[r * NWV + wave] + wave_excl_sum(__popc(selm));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if ((selm >> e) & 1u) {
        if (pos < top_k) {   // always below top_k when the passes agree; guards the writes
          const int32_t te = t + e;
          const int32_t p = te / page_size;
          int32_t pg = pgs[j];
          if (pg < 0 || pg >= num_pages) {
            atomicOr(flags, MLA_FLAG_BAD_PAGE);
            pg = pg < 0 ? 0 : num_pages - 1;
          }
          sel_tok[(int64_t)b * top_k + pos] = te;
          sel_row[(int64_t)b * top_k + pos] = pg * page_size + (te - p * page_size);
        }
        ++pos;
      }
    }
   }
  }
}

// Every sequence within one SEL_CH chunk: the radix passes after the
// indexer's, the final threshold and the listing, in one workgroup per
// sequence with the sequence's scores held in LDS (instead of
// select_hist_kernel<1>, <2> and select_write_kernel, three launches).  The
// pass-0 digit is picked from the indexer's histogram; passes 1 and 2
// histogram the keys that match the bits fixed so far (LDS atomics) and pick
// their digit; then each thread takes a contiguous run of tokens, and two
// block scans of its counts above T and at T give, for every token in order,
// its position in the list: the tokens above T before it plus the ties at T
// before it, at most r of them.  The same list as the three-launch path.
__global__ void __launch_bounds__(SEL_NT) select_local_kernel(const float* __restrict__ scores, int32_t max_tokens,
                                                           const int32_t* __restrict__ seq_lens, int32_t top_k,
                                                           const int32_t* __restrict__ hist, int32_t B,
                                                           int32_t* __restrict__ st,
                                                           const int32_t* __restrict__ page_table, int32_t max_pages,
                                                           int32_t page_size, int32_t num_pages,
                                                           int32_t* __restrict__ sel_tok, int32_t* __restrict__ sel_row,
                                                           int32_t* __restrict__ flags) {
  __shared__ __attribute__((aligned(16))) float sc[SEL_CH];
  __shared__ int32_t h[SEL_BINS];
  __shared__ int32_t part[SEL_NT];
  __shared__ int32_t wsum[2][SEL_NT / 64];
  __shared__ int32_t st_l[4];
  const int32_t b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t n = clamp_len(seq_lens[b], max_tokens);
  const bool all = n <= top_k;
  if (!all) {
    const float* sb = scores + (int64_t)b * max_tokens;
    for (int32_t t = 4 * tid; t < n; t += 4 * SEL_NT) {
      const float4 v = *(const float4*)(sb + t);
      const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (t + e < n) sc[t + e] = x[e];
    }
    if (tid < 3) st_l[tid] = 0;
    __syncthreads();
    pick_digit<0, SEL_NT>(hist + (int64_t)b * SEL_BINS, true, st_l, top_k, part);
    __syncthreads();
    auto pass = [&](auto P) __attribute__((always_inline)) {
      using D = Digit<decltype(P)::value>;
      for (int i = tid; i < SEL_BINS; i += SEL_NT) h[i] = 0;
      __syncthreads();
      const uint32_t fixed = (uint32_t)st_l[0];
      for (int32_t t = tid; t < n; t += SEL_NT) {
        const uint32_t key = score_key(sc[t]);
        if ((key & D::HIMASK) == fixed) atomicAdd(&h[(key >> D::SHIFT) & D::BMASK], 1);
      }
      __syncthreads();
      pick_digit<decltype(P)::value, SEL_NT>(h, false, st_l, top_k, part);
      __syncthreads();
    };
    pass(std::integral_constant<int, 1>{});
    pass(std::integral_constant<int, 2>{});
  }
  const uint32_t T = all ? 0u : (uint32_t)st_l[0];
  const int32_t rem = all ? 0 : st_l[1];
  if (tid < 3) st[(2 * B + b) * 4 + tid] = all ? (tid == 2 ? 1 : 0) : (tid == 2 ? 0 : (int32_t)(tid ? rem : T));
  const int32_t per = (n + SEL_NT - 1) / SEL_NT;
  const int32_t t0 = min(n, tid * per), t1 = min(n, t0 + per);
  int32_t g = 0, e = 0;
  for (int32_t t = t0; t < t1; ++t) {
    const uint32_t key = all ? 0u : score_key(sc[t]);
    g += all || key > T;
    e += !all && key == T;
  }
  int32_t tot;
  int32_t er = block_excl_sum(e, wsum[0], tot);
  int32_t gr = block_excl_sum(g, wsum[1], tot);
  const int32_t* pt = page_table + (int64_t)b * max_pages;
  for (int32_t t = t0; t < t1; ++t) {
    const uint32_t key = all ? 0u : score_key(sc[t]);
    int32_t pos = -1;
    if (all || key > T) {
      pos = gr + min(er, rem);
      ++gr;
    } else if (key == T) {
      if (er < rem) pos = gr + er;
      ++er;
    }
    if (pos >= 0 && pos < top_k) {   // always below top_k when the passes agree; guards the writes
      const int32_t p = t / page_size;
      int32_t pg = pt[p];
      if (pg < 0 || pg >= num_pages) {
        atomicOr(flags, MLA_FLAG_BAD_PAGE);
        pg = pg < 0 ? 0 : num_pages - 1;
      }
      sel_tok[(int64_t)b * top_k + pos] = t;
      sel_row[(int64_t)b * top_k + pos] = pg * page_size + (t - p * page_size);
    }
  }
}

}  // namespace

SelectWs select_ws_layout(int32_t B, int32_t max_tokens, int32_t top_k, bool outputs) {
  SelectWs w;
  w.nchunks = (int32_t)(((int64_t)max_tokens + SEL_CH - 1) / SEL_CH);
  size_t off = 0;
  w.hist = off;    off += align256((size_t)3 * B * SEL_BINS * 4);   // one histogram per radix pass
  w.st = off;      off += align256((size_t)3 * B * 16);             // one state per pass
  w.cnt = off;     off += align256((size_t)B * w.nchunks * 8);
  w.scores = w.sel_tok = w.sel_row = 0;
  if (outputs) {
    w.scores = off;  off += align256((size_t)B * max_tokens * 4);
    w.sel_tok = off; off += align256((size_t)B * top_k * 4);
    w.sel_row = off; off += align256((size_t)B * top_k * 4);
  }
  w.total = off;
  return w;
}

hipError_t launch_indexer_select(int32_t B, int32_t H_I, const void* q_I, const float* w_I, const void* k_I,
                                 int64_t idx_stride, int32_t num_pages, const int32_t* page_table, int32_t max_pages,
                                 int32_t page_size, const int32_t* seq_lens, int32_t top_k, char* ws,
                                 const SelectWs& L, float* scores, int32_t* sel_tok, int32_t* sel_row,
                                 int32_t* flags, hipStream_t s) {
  const int32_t max_tokens = max_pages * page_size;
  int32_t* hist = (int32_t*)(ws + L.hist);
  int32_t* st = (int32_t*)(ws + L.st);
  int32_t* cnt = (int32_t*)(ws + L.cnt);
  select_clear_kernel<<<B, 256, 0, s>>>(hist, B);
  const dim3 gi((uint32_t)(((int64_t)max_tokens + IDX_TOK_WG - 1) / IDX_TOK_WG), B);
  const bf16* q = (const bf16*)q_I;
  const bf16* k = (const bf16*)k_I;
#define MLA_INDEXER(HB)                                                                                       \
  indexer_kernel<HB><<<gi, 256, 0, s>>>(q, w_I, k, idx_stride, num_pages, page_table, max_pages, page_size,    \
                                        seq_lens, max_tokens, top_k, scores, hist, flags)
  switch (H_I / 16) {
    case 1: MLA_INDEXER(1); break;
    case 2: MLA_INDEXER(2); break;
    case 4: MLA_INDEXER(4); break;
    default: return hipErrorInvalidValue;
  }
#undef MLA_INDEXER
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 gs(L.nchunks, B);
  if (L.nchunks == 1) {   // one workgroup per sequence does the whole selection
    select_local_kernel<<<B, SEL_NT, 0, s>>>(scores, max_tokens, seq_lens, top_k, hist, B, st, page_table, max_pages,
                                             page_size, num_pages, sel_tok, sel_row, flags);
    return hipGetLastError();
  }
  const bool local = false;
  select_hist_kernel<1><<<gs, SEL_NT, 0, s>>>(scores, max_tokens, seq_lens, top_k, hist, B, st, local);
  select_hist_kernel<2><<<gs, SEL_NT, 0, s>>>(scores, max_tokens, seq_lens, top_k, hist, B, st, local);
  if (!local)
    select_count_kernel<<<gs, SEL_NT, 0, s>>>(scores, max_tokens, seq_lens, top_k, hist, B, st, cnt, L.nchunks);
  select_write_kernel<<<gs, SEL_NT, 0, s>>>(scores, max_tokens, seq_lens, top_k, st + 2 * B * 4, cnt, L.nchunks, page_table,
                                            max_pages, page_size, num_pages, sel_tok, sel_row, flags);
  return hipGetLastError();
}

}  // namespace mla
