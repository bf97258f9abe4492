// Shared device/host definitions of the gfx950 MLA kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "../../include/mla.h"

namespace mla {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

// Fixed MLA widths the kernels are built for (DeepSeek-V2).
constexpr int D_C = 512;          // latent c^KV
constexpr int D_R = 64;           // decoupled RoPE key k^R
constexpr int D_K = D_C + D_R;    // 576: one cached row
constexpr int D_H = 128;          // per-head q^C / v width

constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// Row index of token t of sequence b in the paged pool; out-of-range page ids
// are clamped into the pool and reported through *flags.
__device__ __forceinline__ int64_t pool_row(const int32_t* __restrict__ page_table, int32_t max_pages,
                                            int32_t num_pages, int32_t page_size, int32_t b, int32_t t,
                                            int32_t* flags) {
  int32_t pg = page_table[(int64_t)b * max_pages + t / page_size];
  if (pg < 0 || pg >= num_pages) {
    if (flags) atomicOr(flags, MLA_FLAG_BAD_PAGE);
    pg = pg < 0 ? 0 : num_pages - 1;
  }
  return (int64_t)pg * page_size + t % page_size;
}

// RoPE frequencies theta_k = base^(-2k/d_hR), k = 0..31, formed once on the
// host in fp64 and passed to the kernels by value.
struct RopeTab {
  double theta[D_R / 2];
};
inline RopeTab rope_table(float base) {
  RopeTab t;
  for (int k = 0; k < D_R / 2; ++k) t.theta[k] = std::pow((double)base, -2.0 * k / (double)D_R);
  return t;
}

// cos / sin of the RoPE angle of pair k at position pos: the angle
// pos * theta_k is formed and reduced to [-pi, pi] in fp64 (the angle is
// exact to ~1e-11 for positions below 2^31), then its cosine and sine are
// taken in fp32.
__device__ __forceinline__ void rope_cos_sin(int32_t pos, int k, const RopeTab& rt, float* c, float* s) {
  const double a = (double)pos * rt.theta[k];
  const double n = rint(a * 0.15915494309189535);   // a / (2 pi), rounded
  const float r = (float)fma(-n, 6.283185307179586, a);
  sincosf(r, s, c);
}

// Element offset of (head h, dim d) in one sequence's block of the absorbed
// queries q~ ([n_h x 576] elements).  bf16 with n_h % 32 == 0: grouped so
// that each of the attention kernel's query loads (decode_mfma.hip) covers
// one whole 1 KB run, while each head's dims stay in runs of 64 B or more for
// the absorption's stores:
//  * dims 0..447: for each 16 heads and each 32 dims, a 1 KB block holding
//    the 16 heads' 32 dims head after head (the B operands of one K-step of
//    the 16x16x32 score MFMAs);
//  * dims 448..575, after all heads' first part: 128 dims per head, head
//    after head.
// Otherwise (fp32, or n_h not a multiple of 32) rows of 576 in head order.
__host__ __device__ __forceinline__ int64_t qabs_offset(int32_t n_h, bool frag, int h, int d) {
  if (!frag || n_h % 32 != 0) return (int64_t)h * D_K + d;
  if (d < 448) return (int64_t)(h >> 4) * 7168 + (d >> 5) * 512 + (h & 15) * 32 + (d & 31);
  return (int64_t)n_h * 448 + h * 128 + (d - 448);
}

// Ints per split record (see plan_block).
constexpr int SPLIT_REC = 8;

// Cached rows per tile of the bf16 attention kernel (decode_mfma.hip).
constexpr int DECODE_TT = 32;

// Tile order within a segment (the piece of one sequence that one split
// covers): split w visits the segment's K tiles starting at tile
// tile_phase(w, K) and wrapping around to tile 0.  Walked in lockstep from
// their first rows, the splits' concurrent reads keep fixed distances from
// one another in the cache pool, and for some pool layouts (each sequence's
// pages in order) those distances crowd a few HBM channels: a plain stream
// over such a layout ran at 4.2 TB/s where the same bytes read with spread
// starting tiles ran at 5.8.  The softmax is order-free, so any order gives
// the same result up to fp32 rounding.  w times the golden-ratio constant,
// top 16 bits, modulo K.
__host__ __device__ __forceinline__ int32_t tile_phase(int32_t w, int32_t K) {
  return (int32_t)((((uint32_t)w * 0x9E3779B1u) >> 16) % (uint32_t)K);
}

// d_model chunks of the split-K append (append_splitk.h).
constexpr int APPEND_SK_SPLIT = 8;

// Decode workspace layout (bytes, each part 256-aligned).  flags: word 0 the
// decode's error flags, word 1 (decode step only) the append's; then three
// blocks of split-K tile counters at fixed offsets: the decode step's append
// (app_cnt), and the whole-layer entry point's query and output projections
// (q_cnt, o_cnt).  Everything after them moves with the batch size; the
// counters must not, because a workspace is zero-filled once and then reused
// for any batch size.  The decode step adds the split-K append's chunk sums.
struct DecodeWs {
  size_t flags, prefix, splits, qabs, part_ml, part_o, app_part, app_cnt, q_cnt, o_cnt, total;
  int32_t n_slots;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Tile counters of in-launch split-K reductions.  A product is split only
// while it has fewer tiles than fill the GPU (1024 workgroups), so 1024
// counters serve any product; each block sits at a fixed offset of its
// workspace (right after the flags of a decode workspace, at offset 0 of a
// projection's) and each completed launch leaves them at zero, so a
// workspace zero-filled once stays valid for every batch size and for
// consecutive products.
constexpr int SPLITK_COUNTERS = 1024;
constexpr size_t SPLITK_COUNTER_BYTES = SPLITK_COUNTERS * 4;

inline DecodeWs decode_ws_layout(int32_t B, int32_t n_h, int32_t n_splits, int elt, bool step = false) {
  DecodeWs w;
  w.n_slots = n_splits + B;
  size_t off = 0;
  w.flags = off;   off += 256;
  w.app_cnt = off; off += SPLITK_COUNTER_BYTES;
  w.q_cnt = off;   off += SPLITK_COUNTER_BYTES;
  w.o_cnt = off;   off += SPLITK_COUNTER_BYTES;
  w.prefix = off;  off += align256((size_t)(B + 1) * 4);
  w.splits = off;  off += align256((size_t)n_splits * SPLIT_REC * 4);   // per split: see plan_block
  w.qabs = off;    off += align256((size_t)B * n_h * D_K * elt);
  w.part_ml = off; off += align256((size_t)w.n_slots * n_h * 2 * 4);
  w.part_o = off;  off += align256((size_t)w.n_slots * n_h * D_C * elt);   // partial O~ in the cache type
  w.app_part = off;
  if (step) off += align256((size_t)APPEND_SK_SPLIT * B * D_K * 4);       // fp32 chunk sums
  w.total = off;
  return w;
}

// Work partition: the batch's N cached tokens, laid end to end, are cut into
// n_splits near-equal ranges [P_w, P_w+1), P_w = floor(w*N/n_splits).  Range w
// and sequence b overlap in at most one segment, whose partial result lives in
// slot w + b (distinct for every overlapping pair, and contiguous in w for a
// fixed b).
__device__ __forceinline__ int64_t split_begin(int64_t w, int64_t N, int64_t G) { return (w * N) / G; }
// Split holding global token x (0 <= x < N).
__device__ __forceinline__ int64_t split_of(int64_t x, int64_t N, int64_t G) {
  return ((x + 1) * G + N - 1) / N - 1;
}
// Last b in [0, B) with prefix[b] <= x.
__device__ __forceinline__ int32_t seq_of(const int32_t* __restrict__ prefix, int32_t B, int64_t x) {
  int32_t lo = 0, hi = B - 1;
  while (lo < hi) {
    int32_t mid = (lo + hi + 1) >> 1;
    if ((int64_t)prefix[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Inputs and outputs of the decode plan.
struct PlanArgs {
  const int32_t* seq_lens;
  int32_t B, max_tokens, G;
  int32_t* prefix;
  int32_t* split_rec;
  int32_t* flags;
  const int32_t* page_table;
  int32_t max_pages, page_size;
  // Sparse decode: each sequence keeps at most `keep` tokens (the selection's
  // list positions); the records then carry no page ids (gather = true).
  int32_t keep = 0x7fffffff;
  bool gather = false;
};

// Decode plan, run by one workgroup of NT threads.  part: NT + cap ints of
// LDS (prefix sums are kept there when B + 1 <= cap).  It clears the error
// flags, writes prefix[0..B] = exclusive sum of the clamped sequence lengths,
// and for every split w the record
//   {b, prefix[b], prefix[b+1], a_0, a_1, c_0, c_1, 0}
// of the sequence b holding its first token P_w = floor(w N / G) (the last b
// with prefix[b] <= P_w).  The split's first segment is [P_w, min(prefix[b+1],
// P_{w+1})), cut into K tiles of DECODE_TT rows from P_w on; a_0, a_1 are the
// page-table entries of the first and last page of tile tile_phase(w, K),
// the first tile the attention kernel visits, and c_0, c_1 those of the
// tile after it in that order (tile 0 after tile K - 1; meaningless when
// K = 1).  Page indices past the table's row repeat its last entry.  One
// thread per split, so the page-table reads of all splits are in flight
// together.
template <int NT>
__device__ __forceinline__ void plan_block(const PlanArgs& pa, int32_t* part, int32_t cap) {
  const int tid = threadIdx.x;
  const int32_t B = pa.B, max_tokens = pa.max_tokens, G = pa.G;
  if (tid == 0) pa.flags[0] = 0;   // the flags describe the latest decode on this workspace
  __syncthreads();
  const int per = (B + NT - 1) / NT;
  const int beg = tid * per, end = min(beg + per, B);
  int32_t local = 0;
  for (int b = beg; b < end; ++b) {
    int32_t n = pa.seq_lens[b];
    if (n < 1 || n > max_tokens) {
      atomicOr(pa.flags, MLA_FLAG_BAD_SEQ_LEN);
      n = n < 1 ? 0 : max_tokens;
    }
    local += min(n, pa.keep);
  }
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {   // Hillis-Steele inclusive scan of the thread totals
    const int32_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  const int32_t N = part[NT - 1];
  const bool in_lds = B + 1 <= cap;
  int32_t* pl = part + NT;
  int32_t run = tid > 0 ? part[tid - 1] : 0;
  for (int b = beg; b < end; ++b) {
    int32_t n = pa.seq_lens[b];
    n = n < 1 ? 0 : (n > max_tokens ? max_tokens : n);
    n = min(n, pa.keep);
    pa.prefix[b] = run;
    if (in_lds) pl[b] = run;
    run += n;
  }
  if (tid == NT - 1) {
    pa.prefix[B] = N;
    if (in_lds) pl[B] = N;
  }
  __threadfence_block();
  __syncthreads();
  if (N <= 0) return;
  const int32_t* px = in_lds ? pl : pa.prefix;
  for (int32_t w = tid; w < G; w += NT) {
    const int32_t P = (int32_t)((int64_t)w * N / G);
    int32_t lo = 0, hi = B - 1;   // last b with prefix[b] <= P
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (px[mid] <= P) lo = mid; else hi = mid - 1;
    }
    const int32_t s0 = px[lo], s1 = px[lo + 1];
    const int32_t Pn = (int32_t)((int64_t)(w + 1) * N / G);
    const int32_t se = min(s1, Pn);
    const int32_t K = (se - P + DECODE_TT - 1) / DECODE_TT;   // 0 for an empty split
    const int32_t* pt = pa.page_table + (int64_t)lo * pa.max_pages;
    int32_t pg[4] = {0, 0, 0, 0};
    if (K > 0 && !pa.gather) {
      const int32_t k0 = tile_phase(w, K);
      const int32_t k1 = k0 + 1 == K ? 0 : k0 + 1;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int32_t x0 = P + DECODE_TT * (i ? k1 : k0);
        const int32_t n = min(DECODE_TT, se - x0);
        const int32_t pf = (x0 - s0) / pa.page_size, pl = (x0 - s0 + n - 1) / pa.page_size;
        pg[2 * i] = pt[min(pf, pa.max_pages - 1)];
        pg[2 * i + 1] = pt[min(pl, pa.max_pages - 1)];
      }
    }
    int4* r = (int4*)(pa.split_rec + SPLIT_REC * w);
    r[0] = int4{lo, s0, s1, pg[0]};
    r[1] = int4{pg[1], pg[2], pg[3], 0};
  }
}

}  // namespace mla

// Launchers (host side), one per kernel family.
namespace mla {
// Cache append.  With a workspace of append_workspace_bytes(d, T) bytes (0:
// no workspace path for these sizes) a batch of up to APPEND_WS_MAX_T rows
// (bf16) runs split over d_model in two launches; otherwise one kernel does
// it.  The split path measured faster from 128 to 1024 rows (33 against 53 us
// at 512, 61 against 109 us at 1024 on DeepSeek-V2 sizes, with 16-column
// chunk-sum tiles; the 64 x 64 tiles used from 256 rows bring 512 rows to 25).
constexpr int APPEND_WS_MAX_T = 1024;
size_t append_workspace_bytes(const mla_dims& d, int32_t T);
hipError_t launch_append(const mla_dims& d, int32_t T, const void* h, const void* W_DKV, const void* W_KR,
                         const int32_t* seq_id, const int32_t* pos, const int32_t* page_table,
                         int32_t num_seqs, int32_t max_pages, void* c_KV, void* k_R, int64_t row_stride,
                         int32_t num_pages, int32_t* err_flag, void* ws, size_t ws_bytes, hipStream_t s);
hipError_t launch_plan(const PlanArgs& pa, hipStream_t s);
// Chunked prefill: per-query page-table rows and lengths, and a cleared
// append flag word (prefill.hip).
hipError_t launch_prefill_queries(int32_t T, const int32_t* seq_id, const int32_t* pos, const int32_t* page_table,
                                  int32_t num_seqs, int32_t max_pages, int32_t page_size, int32_t* q_pt,
                                  int32_t* q_len, int32_t* append_flag, hipStream_t s);
// Query absorption; for bf16 the decode plan runs in the same launch (then
// launch_plan is not called).
hipError_t launch_absorb(const mla_dims& d, int32_t B, const void* q_C, const void* q_R, const int32_t* pos_q,
                         const void* W_UK, void* qabs, const PlanArgs& pa, hipStream_t s);
// The decode layer's q^C = W^UQ c^Q and its absorption in one launch (bf16;
// c^Q and W^UQ in the packed layout of the projection kernels, c^Q with its
// rows padded to a multiple of 64).  The plan is not run here.
inline bool absorb_fused_supported(const mla_dims& d, int32_t B, int32_t d_cq) {
  return d.dtype == MLA_BF16 && B >= 1 && d_cq >= 32 && d_cq % 32 == 0;
}
hipError_t launch_absorb_fused(const mla_dims& d, int32_t B, int32_t d_cq, const void* cQ_packed,
                               const void* W_UQ_packed, const void* q_R, const int32_t* pos_q, const void* W_UK,
                               void* qabs, hipStream_t s);
// Decode step, first launch: the split-K append of each sequence's newest
// token (finished in the same launch), the query absorption and the plan, as
// one grid (bf16, d_model a multiple of 1024; step_prep_supported()).
struct AppendDst;
bool step_prep_supported(const mla_dims& d, int32_t B);
// absorb = false: append and plan only (the absorption runs elsewhere).
hipError_t launch_step_prep(const mla_dims& d, int32_t B, const void* h_new, const void* W_DKV, const void* W_KR,
                            const void* q_C, const void* q_R, const int32_t* pos_q, const void* W_UK, void* qabs,
                            const PlanArgs& pa, float* app_part, int32_t* app_cnt, const AppendDst& dst,
                            hipStream_t s, bool absorb = true);
hipError_t launch_decode_simple(const mla_dims& d, int32_t B, const void* qabs, const void* c_KV,
                                const void* k_R, int64_t row_stride, int32_t num_pages,
                                const int32_t* page_table, int32_t max_pages, const int32_t* prefix,
                                int32_t n_splits, float* part_ml, void* part_o, int32_t* flags,
                                hipStream_t s);
// rows: NULL (contiguous tokens through the page table), or the sparse
// decode's kept pool rows, rows[b * rows_stride + i] for list position i
// (the plan then counts list positions, PlanArgs::keep / gather).
hipError_t launch_decode_mfma(const mla_dims& d, int32_t B, const void* qabs, const void* c_KV,
                              const void* k_R, int64_t row_stride, int32_t num_pages,
                              const int32_t* page_table, int32_t max_pages, const int32_t* prefix,
                              const int32_t* split_rec, int32_t n_splits, float* part_ml, void* part_o,
                              int32_t* flags, hipStream_t s, const int32_t* rows = nullptr,
                              int32_t rows_stride = 0);

// Sparse decode selection (sparse.hip): workspace parts, bytes from the
// start of the selection area.  nchunks: SEL_CH-token chunks per sequence.
constexpr int SEL_BINS = 2048;   // radix bins per pass
constexpr int SEL_CH = 16384;    // tokens per selection workgroup (longer sequences: several)
struct SelectWs {
  int32_t nchunks;
  size_t hist, st, cnt, scores, sel_tok, sel_row, total;
};
// outputs: also room for the scores and the kept tokens / rows (else the
// caller provides them).
SelectWs select_ws_layout(int32_t B, int32_t max_tokens, int32_t top_k, bool outputs);
// Indexer scores (into `scores`, [B, max_pages*page_size] fp32) and the kept
// tokens and pool rows ([B, top_k] each; the first min(n_b, top_k) entries of
// row b are written).  ws: the selection area laid out by L.
hipError_t launch_indexer_select(int32_t B, int32_t H_I, const void* q_I, const float* w_I, const void* k_I,
                                 int64_t idx_stride, int32_t num_pages, const int32_t* page_table, int32_t max_pages,
                                 int32_t page_size, const int32_t* seq_lens, int32_t top_k, char* ws,
                                 const SelectWs& L, float* scores, int32_t* sel_tok, int32_t* sel_row,
                                 int32_t* flags, hipStream_t s);
// merge_flags: NULL, or (decode step) the flag area whose word 1 holds the
// append's flags, to be OR-ed into word 0 and cleared; ext_flags (NULL, or a
// caller's device word, with merge_flags given) also receives them.
hipError_t launch_combine(const mla_dims& d, int32_t B, const int32_t* prefix, int32_t n_splits,
                          const float* part_ml, const void* part_o, const void* W_UV, float* out,
                          float* lse, int32_t* merge_flags, void* out_packed, hipStream_t s,
                          int32_t* ext_flags = nullptr);
}  // namespace mla
