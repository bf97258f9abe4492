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
//    (v_mfma_f32_16x16x32_bf16; a wave takes 16-token blocks, its query
//    fragments stay in registers), then ReLU, the head weights and the sum
//    over heads (in registers, then across the 16 lanes of a row).  Bound by
//    HBM: 256 B of keys per token against 2 H_I d_I flops.
//  * Selection: a radix select on order-preserving 32-bit keys of the fp32
//    scores, three passes of 11, 11 and 10 bits.  Each pass histograms the
//    keys that match the bits fixed so far (LDS, then integer atomics into a
//    per-sequence histogram); the last workgroup of a sequence to finish
//    (counted by an atomic ticket) finds the bin where the running count
//    from the top reaches k and fixes those bits.  After three passes the
//    threshold key T and the number r of ties at T to keep are known.  A
//    count pass and a write pass then list, in token order, every token
//    with key > T and the first r tokens with key == T, with their pool rows
//    (page-table lookups) for the gather attention.  Integer work only: the
//    result is exact and deterministic.
#include "mla_common.h"

namespace mla {
namespace {

constexpr int IDX_D = 128;                 // indexer key width d_I
constexpr int IDX_KS = IDX_D / 32;         // K-steps of the 16x16x32 MFMA
constexpr int IDX_BPW = 8;                 // 16-token blocks per wave
constexpr int IDX_TOK_WG = 4 * IDX_BPW * 16;   // 512 tokens per workgroup (4 waves)

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

// Relevance scores of one 512-token range of one sequence (blockIdx.y).
// Workgroup x = 0 of each sequence also clears that sequence's selection
// histogram and ticket (the selection passes come after this launch).
template <int HB>
__global__ void __launch_bounds__(256) indexer_kernel(const bf16* __restrict__ q_I, const float* __restrict__ w_I,
                                                      const bf16* __restrict__ k_I, int64_t idx_stride,
                                                      int32_t num_pages, const int32_t* __restrict__ page_table,
                                                      int32_t max_pages, int32_t page_size,
                                                      const int32_t* __restrict__ seq_lens, int32_t max_tokens,
                                                      float* __restrict__ scores, int32_t* __restrict__ hist,
                                                      int32_t* __restrict__ ticket, int32_t* __restrict__ flags) {
  const int32_t b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < SEL_BINS; i += 256) hist[(int64_t)b * SEL_BINS + i] = 0;
    if (threadIdx.x == 0) ticket[b] = 0;
  }
  const int32_t n = clamp_len(seq_lens[b], max_tokens);
  const int32_t t_wave = blockIdx.x * IDX_TOK_WG + wave * IDX_BPW * 16;
  if (t_wave >= n) return;

  // B operands: head 16hb + (lane&15), dims 32ks + 8(lane>>4) .. +7
  bf16x8 qf[HB][IDX_KS];
  float wv[HB];
  const bf16* qb = q_I + (int64_t)b * HB * 16 * IDX_D;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    wv[hb] = w_I[(int64_t)b * HB * 16 + 16 * hb + (lane & 15)];
#pragma unroll
    for (int ks = 0; ks < IDX_KS; ++ks)
      qf[hb][ks] = *(const bf16x8*)(qb + (16 * hb + (lane & 15)) * IDX_D + 32 * ks + 8 * (lane >> 4));
  }
  // A operands of the wave's blocks: token t0 + (lane&15), same dims.  A
  // block of 16 tokens lies in one page (page_size is a multiple of 16);
  // rows past the sequence's end repeat its last row.
  const int32_t* pt = page_table + (int64_t)b * max_pages;
  bf16x8 af[IDX_BPW][IDX_KS];
#pragma unroll
  for (int i = 0; i < IDX_BPW; ++i) {
    const int32_t t0 = t_wave + 16 * i;
    if (t0 < n) {
      const int32_t p = t0 / page_size;
      int32_t pg = pt[p];
      if (pg < 0 || pg >= num_pages) {
        atomicOr(flags, MLA_FLAG_BAD_PAGE);
        pg = pg < 0 ? 0 : num_pages - 1;
      }
      const int32_t t = min(t0 + (lane & 15), n - 1);
      const bf16* kr = k_I + ((int64_t)pg * page_size + (t - p * page_size)) * idx_stride + 8 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < IDX_KS; ++ks) af[i][ks] = *(const bf16x8*)(kr + 32 * ks);
    }
  }
  float* sb = scores + (int64_t)b * max_tokens;
#pragma unroll
  for (int i = 0; i < IDX_BPW; ++i) {
    const int32_t t0 = t_wave + 16 * i;
    if (t0 >= n) break;
    f32x4 acc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < IDX_KS; ++ks)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
        acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i][ks], qf[hb][ks], acc[hb], 0, 0, 0);
    // lane holds tokens t0 + 4(lane>>4) + r, head 16hb + (lane&15)
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = 0.f;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) x += wv[hb] * fmaxf(acc[hb][r], 0.f);
      v[r] = x;
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] += __shfl_xor(v[r], off);
    const int r = lane & 3;
    const int32_t t = t0 + 4 * (lane >> 4) + r;
    const float val = r == 0 ? v[0] : (r == 1 ? v[1] : (r == 2 ? v[2] : v[3]));
    if ((lane & 15) < 4 && t < n) sb[t] = val;
  }
}

// Block-wide (256 threads) exclusive count of `flag` below this thread and
// the block total.  wsum: 4 ints of LDS; the caller syncs before reusing it.
__device__ __forceinline__ int32_t block_excl(bool flag, int32_t* wsum, int32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const int32_t below = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[wave] = __popcll(m);
  __syncthreads();
  int32_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int32_t c = wsum[w];
    before += w < wave ? c : 0;
    total += c;
  }
  return before + below;
}

// Radix pass PASS (bits 31..21, 20..10, 9..0) over one 4096-token chunk of
// one sequence; the sequence's last workgroup fixes the pass's bits.
// st[4b..]: {key bits fixed so far, ties still to take, every token kept}.
template <int PASS>
__global__ void __launch_bounds__(256) select_hist_kernel(const float* __restrict__ scores, int32_t max_tokens,
                                                          const int32_t* __restrict__ seq_lens, int32_t top_k,
                                                          int32_t* __restrict__ hist, int32_t* __restrict__ ticket,
                                                          int32_t* __restrict__ st, int32_t nchunks) {
  constexpr int SHIFT = PASS == 0 ? 21 : (PASS == 1 ? 10 : 0);
  constexpr uint32_t HIMASK = PASS == 0 ? 0u : (PASS == 1 ? 0xFFE00000u : 0xFFFFFC00u);
  constexpr uint32_t BMASK = PASS == 2 ? 0x3FFu : 0x7FFu;
  __shared__ int32_t h[SEL_BINS];
  __shared__ int32_t part[256];
  __shared__ int32_t is_last;
  const int32_t b = blockIdx.y;
  const int tid = threadIdx.x;
  const int32_t n = clamp_len(seq_lens[b], max_tokens);
  const bool all = n <= top_k;
  const uint32_t fixed = PASS == 0 ? 0u : (uint32_t)st[4 * b];
  int32_t* hb = hist + (int64_t)b * SEL_BINS;
  if (!all) {
    for (int i = tid; i < SEL_BINS; i += 256) h[i] = 0;
    __syncthreads();
    const int32_t c0 = blockIdx.x * SEL_CH, c1 = min(c0 + SEL_CH, n);
    const float* sb = scores + (int64_t)b * max_tokens;
    for (int32_t t = c0 + tid; t < c1; t += 256) {
      const uint32_t key = score_key(sb[t]);
      if ((key & HIMASK) == fixed) atomicAdd(&h[(key >> SHIFT) & BMASK], 1);
    }
    __syncthreads();
    for (int i = tid; i < SEL_BINS; i += 256)
      if (h[i]) atomicAdd(&hb[i], h[i]);
  }
  // Ticket: the histogram atomics of this workgroup are ordered before its
  // ticket (release fence); the last one to take a ticket sees them all
  // (acquire fence, then agent-scope loads that skip the L1).
  __threadfence();
  __syncthreads();
  if (tid == 0) is_last = atomicAdd(&ticket[b], 1) == nchunks - 1;
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  if (tid == 0) ticket[b] = 0;
  if (all) {
    if (tid == 0 && PASS == 0) {
      st[4 * b + 0] = 0;
      st[4 * b + 1] = 0;
      st[4 * b + 2] = 1;
    }
    return;
  }
  const int32_t rem = PASS == 0 ? top_k : st[4 * b + 1];
  // thread tid owns bins 8 tid .. 8 tid + 7
  int32_t c[8], tot = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    c[j] = __hip_atomic_load(&hb[8 * tid + j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    tot += c[j];
  }
  // count in the bins above this thread's: suffix sum over thread totals
  part[tid] = tot;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int32_t v = tid + off < 256 ? part[tid + off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t above = part[tid] - tot;   // keys in bins > 8 tid + 7
#pragma unroll
  for (int j = 7; j >= 0; --j) {
    if (above < rem && rem <= above + c[j]) {
      st[4 * b + 0] = (int32_t)(fixed | ((uint32_t)(8 * tid + j) << SHIFT));
      st[4 * b + 1] = rem - above;
      st[4 * b + 2] = 0;
    }
    above += c[j];
  }
  for (int i = tid; i < SEL_BINS; i += 256) hb[i] = 0;
}

// Kept tokens of one chunk: {key > T, key == T}, or {all, 0}.
__global__ void __launch_bounds__(256) select_count_kernel(const float* __restrict__ scores, int32_t max_tokens,
                                                           const int32_t* __restrict__ seq_lens,
                                                           const int32_t* __restrict__ st, int32_t* __restrict__ cnt,
                                                           int32_t nchunks) {
  __shared__ int32_t wsum[2][4];
  const int32_t b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t n = clamp_len(seq_lens[b], max_tokens);
  const bool all = st[4 * b + 2] != 0;
  const uint32_t T = (uint32_t)st[4 * b];
  const int32_t c0 = blockIdx.x * SEL_CH, c1 = min(c0 + SEL_CH, n);
  int32_t gt = 0, eq = 0;
  const float* sb = scores + (int64_t)b * max_tokens;
  for (int32_t t = c0 + tid; t < c1; t += 256) {
    if (all) {
      ++gt;
    } else {
      const uint32_t key = score_key(sb[t]);
      gt += key > T;
      eq += key == T;
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
    int32_t* o = cnt + ((int64_t)b * nchunks + blockIdx.x) * 2;
    o[0] = wsum[0][0] + wsum[0][1] + wsum[0][2] + wsum[0][3];
    o[1] = wsum[1][0] + wsum[1][1] + wsum[1][2] + wsum[1][3];
  }
}

// Lists the kept tokens of one chunk, in token order, with their pool rows.
__global__ void __launch_bounds__(256) select_write_kernel(const float* __restrict__ scores, int32_t max_tokens,
                                                           const int32_t* __restrict__ seq_lens, int32_t top_k,
                                                           const int32_t* __restrict__ st,
                                                           const int32_t* __restrict__ cnt, int32_t nchunks,
                                                           const int32_t* __restrict__ page_table, int32_t max_pages,
                                                           int32_t page_size, int32_t num_pages,
                                                           int32_t* __restrict__ sel_tok, int32_t* __restrict__ sel_row,
                                                           int32_t* __restrict__ flags) {
  __shared__ int32_t wsum[2][4];
  __shared__ int32_t base[2];
  const int32_t b = blockIdx.y, c = blockIdx.x;
  const int tid = threadIdx.x;
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
  __syncthreads();
  int32_t run_eq = base[1];
  int32_t run_sel = base[0] + (all ? 0 : min(base[1], rem));
  const float* sb = scores + (int64_t)b * max_tokens;
  const int32_t* pt = page_table + (int64_t)b * max_pages;
  for (int32_t r0 = c0; r0 < c1; r0 += 256) {
    const int32_t t = r0 + tid;
    const bool valid = t < c1;
    bool gt = false, eq = false;
    if (valid) {
      if (all) {
        gt = true;
      } else {
        const uint32_t key = score_key(sb[t]);
        gt = key > T;
        eq = key == T;
      }
    }
    int32_t tot_eq, tot_sel;
    const int32_t eq_rank = run_eq + block_excl(eq, wsum[0], tot_eq);
    const bool sel = gt || (eq && eq_rank < rem);
    const int32_t pos = run_sel + block_excl(sel, wsum[1], tot_sel);
    if (sel && pos < top_k) {   // always true when the passes above agree; guards the writes
      const int32_t p = t / page_size;
      int32_t pg = pt[p];
      if (pg < 0 || pg >= num_pages) {
        atomicOr(flags, MLA_FLAG_BAD_PAGE);
        pg = pg < 0 ? 0 : num_pages - 1;
      }
      sel_tok[(int64_t)b * top_k + pos] = t;
      sel_row[(int64_t)b * top_k + pos] = pg * page_size + (t - p * page_size);
    }
    run_eq += tot_eq;
    run_sel += tot_sel;
    __syncthreads();   // wsum is reused next round
  }
}

}  // namespace

SelectWs select_ws_layout(int32_t B, int32_t max_tokens, int32_t top_k, bool outputs) {
  SelectWs w;
  w.nchunks = (max_tokens + SEL_CH - 1) / SEL_CH;
  size_t off = 0;
  w.hist = off;    off += align256((size_t)B * SEL_BINS * 4);
  w.ticket = off;  off += align256((size_t)B * 4);
  w.st = off;      off += align256((size_t)B * 16);
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
  int32_t* ticket = (int32_t*)(ws + L.ticket);
  int32_t* st = (int32_t*)(ws + L.st);
  int32_t* cnt = (int32_t*)(ws + L.cnt);
  const dim3 gi((max_tokens + IDX_TOK_WG - 1) / IDX_TOK_WG, B);
  const bf16* q = (const bf16*)q_I;
  const bf16* k = (const bf16*)k_I;
  switch (H_I / 16) {
    case 1: indexer_kernel<1><<<gi, 256, 0, s>>>(q, w_I, k, idx_stride, num_pages, page_table, max_pages, page_size,
                                                 seq_lens, max_tokens, scores, hist, ticket, flags); break;
    case 2: indexer_kernel<2><<<gi, 256, 0, s>>>(q, w_I, k, idx_stride, num_pages, page_table, max_pages, page_size,
                                                 seq_lens, max_tokens, scores, hist, ticket, flags); break;
    case 4: indexer_kernel<4><<<gi, 256, 0, s>>>(q, w_I, k, idx_stride, num_pages, page_table, max_pages, page_size,
                                                 seq_lens, max_tokens, scores, hist, ticket, flags); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 gs(L.nchunks, B);
  select_hist_kernel<0><<<gs, 256, 0, s>>>(scores, max_tokens, seq_lens, top_k, hist, ticket, st, L.nchunks);
  select_hist_kernel<1><<<gs, 256, 0, s>>>(scores, max_tokens, seq_lens, top_k, hist, ticket, st, L.nchunks);
  select_hist_kernel<2><<<gs, 256, 0, s>>>(scores, max_tokens, seq_lens, top_k, hist, ticket, st, L.nchunks);
  select_count_kernel<<<gs, 256, 0, s>>>(scores, max_tokens, seq_lens, st, cnt, L.nchunks);
  select_write_kernel<<<gs, 256, 0, s>>>(scores, max_tokens, seq_lens, top_k, st, cnt, L.nchunks, page_table,
                                         max_pages, page_size, num_pages, sel_tok, sel_row, flags);
  return hipGetLastError();
}

}  // namespace mla
