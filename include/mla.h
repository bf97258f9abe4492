/*
 * mla.h -- C ABI of the MI355X (gfx950) Multi-head Latent Attention decode
 * library (libmla.so).
 *
 * What is computed (DeepSeek-V2 MLA, notation of the pages):
 *   "DeepSeek-V2：在“大力出奇迹”的AI军备竞赛中，四两拨千斤" (liang.world), ch.2
 *   "侠客甲——MLA": §2 low-rank joint KV compression (c_t^KV = W^DKV h_t,
 *   k_t^C = W^UK c_t^KV, v_t^C = W^UV c_t^KV; W^UK and W^UV absorbed into the
 *   query and output sides), §3 decoupled RoPE (q_{t,i} = [q^C_{t,i}; q^R_{t,i}],
 *   k_{t,i} = [k^C_{t,i}; k^R_t], one k^R shared by all heads); and
 *   "DeepSeek 系列模型技术深度解读" (tuntang.top), MLA section, "RoPE 的兼容性处理"
 *   (k^R_t = RoPE(W^KR h_t)).  Each cached token stores only c^KV (d_c) and k^R
 *   (d_h^R): "Must also cache k_rope" -- pptc.cn DeepSeek note, §6 pitfall 2.
 *
 * Conventions fixed here where the pages are silent:
 *   - RoPE rotates adjacent pairs (x[2k], x[2k+1]) by pos * rope_base^(-2k/d_hR);
 *     angles are formed in fp64, the rotation is done in fp32.
 *   - Scores are (q^C . k^C + q^R . k^R) * softmax_scale (normally
 *     1/sqrt(d_h + d_hR)); softmax over every cached token of the sequence.
 *   - Weights are [out, in] row-major: W^DKV [d_c, d_model], W^KR [d_hR, d_model],
 *     W^UK and W^UV [n_h*d_h, d_c]; head i owns rows i*d_h .. i*d_h+d_h-1.
 *   - The attention output is each head's o_i = W^UV_i O~_i (fp32);
 *     mla_output_project applies W_O to it.
 *
 * Latent cache (paged pool, owned by the caller):
 *   A pool row r holds one token: c^KV at c_KV + r*row_stride (d_c elements)
 *   and k^R at k_R + r*row_stride (d_hR elements, already rotated).  The
 *   interleaved layout k_R = c_KV + d_c, row_stride = d_c + d_hR (576) is the
 *   default; separate pools sharing one stride also work.  Token t of sequence
 *   b lives in row page_table[b*max_pages + t/page_size]*page_size + t%page_size.
 *   Rows are 16-byte aligned (row_stride * element size % 16 == 0).
 *
 * Element type: dims.dtype selects bf16 (MLA_BF16: h, weights, q, cache in
 * bf16; fp32 accumulation) or fp32 (MLA_FP32: everything fp32).  Outputs of
 * mla_decode are fp32 in both cases.
 *
 * Ownership and ordering: every pointer is caller-owned device memory (HBM)
 * unless stated.  Calls enqueue kernels on `stream` (a hipStream_t, or NULL
 * for the default stream) and return after the launch; results are ready when
 * the stream reaches that point.  The library allocates no device memory: the
 * decode scratch is the caller's workspace.  Calls are reentrant; the only
 * state is the thread-local message behind mla_last_error().
 *
 * Errors: host-side checks (null or misaligned pointers, unsupported dims,
 * bad sizes, small workspace) return a status without launching anything.
 * Limits shared by every call: batch rows B or T <= 2^20, n_splits <= 2^20,
 * row strides <= 2^24 elements, tokens addressed by one call (B * max_pages *
 * page_size, and num_pages * page_size) < 2^31; softmax_scale and rope_base
 * positive and finite.  The workspace-size functions return 0 outside these
 * limits.
 * Values that live on the device (positions, sequence lengths, page ids) are
 * checked by the kernels: an out-of-range value is clamped so that no access
 * leaves its buffer, and a flag is raised in the workspace (decode) or in the
 * optional err_flag word (append), readable with mla_read_error_flags().
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,  /* null / misaligned pointer, bad size or count */
  MLA_ERR_UNSUPPORTED = 2,  /* dims the kernels are not built for */
  MLA_ERR_WORKSPACE = 3,    /* workspace smaller than mla_decode_workspace_size() */
  MLA_ERR_HIP = 4           /* a HIP runtime / launch error */
} mla_status;

typedef enum mla_dtype { MLA_BF16 = 0, MLA_FP32 = 1 } mla_dtype;

/* Device-side error flags (bit mask) raised by the kernels. */
enum {
  MLA_FLAG_BAD_SEQ_LEN = 1,   /* seq_len < 1 or > max_pages*page_size (clamped) */
  MLA_FLAG_BAD_PAGE = 2,      /* page id outside [0, num_pages) (clamped) */
  MLA_FLAG_BAD_POSITION = 4,  /* append position outside [0, max_pages*page_size) (row skipped) */
  MLA_FLAG_BAD_SEQ_ID = 8     /* append sequence id outside [0, num_seqs) (row skipped) */
};

typedef struct mla_dims {
  int32_t n_h;        /* attention heads (DeepSeek-V2: 128) */
  int32_t d_h;        /* per-head q^C / k^C / v^C width (must be 128) */
  int32_t d_c;        /* latent width of c^KV (must be 512) */
  int32_t d_hR;       /* decoupled RoPE width of q^R / k^R (must be 64) */
  int32_t d_model;    /* width of h_t (multiple of 64) */
  int32_t page_size;  /* tokens per cache page (>= 1) */
  float softmax_scale;
  float rope_base;
  int32_t dtype;      /* mla_dtype */
} mla_dims;

/*
 * mla_cache_append -- write T new tokens into the latent cache.
 * For each token row t: c^KV = W^DKV h_t and k^R = RoPE(W^KR h_t, pos[t])
 * (liang.world ch.2 §2 eq. for c_t^KV; tuntang.top MLA section, k_t formula),
 * rounded to the cache type and stored at position pos[t] of sequence
 * seq_id[t] (the row of page_table), per the paging rule above.
 *   h_t        [T, d_model]          dtype        device
 *   W_DKV      [d_c, d_model]        dtype        device
 *   W_KR       [d_hR, d_model]       dtype        device
 *   seq_id     [T] int32 or NULL     device       NULL means seq_id[t] = t
 *   pos        [T] int32             device       0 <= pos < max_pages*page_size
 *   page_table [num_seqs, max_pages] int32 device entries in [0, num_pages)
 *   c_KV, k_R  pool base pointers, row_stride elements per row, num_pages pages
 *   err_flag   int32 device word or NULL; bad ids / positions set MLA_FLAG_* bits
 * Rows with a bad seq_id / position are skipped; page ids are clamped.
 */
mla_status mla_cache_append(const mla_dims* dims, int32_t T, const void* h_t, const void* W_DKV,
                            const void* W_KR, const int32_t* seq_id, const int32_t* pos,
                            const int32_t* page_table, int32_t num_seqs, int32_t max_pages,
                            void* c_KV, void* k_R, int64_t row_stride, int32_t num_pages,
                            int32_t* err_flag, void* stream);

/*
 * mla_cache_append_workspace_size -- bytes of device workspace with which
 * mla_cache_append_ws takes its split path for T tokens (bf16, T <= 1024,
 * d_model a multiple of 1024); 0 when that path does not apply.
 *
 * mla_cache_append_ws -- mla_cache_append with a caller workspace
 * (256-byte aligned, device memory, contents need no initialisation).  With
 * at least mla_cache_append_workspace_size() bytes, the batch is
 * computed split over d_model (fp32 partial sums in the workspace, then one
 * pass that adds them in a fixed order, applies RoPE and stores the rows), so
 * the weight stream is spread over the whole GPU; results are the same
 * computation as mla_cache_append up to fp32 summation order.  With a smaller
 * or NULL workspace it behaves exactly as mla_cache_append.  Calls that share
 * one workspace must be ordered (e.g. on one stream).
 */
size_t mla_cache_append_workspace_size(const mla_dims* dims, int32_t T);
mla_status mla_cache_append_ws(const mla_dims* dims, int32_t T, const void* h_t, const void* W_DKV,
                               const void* W_KR, const int32_t* seq_id, const int32_t* pos,
                               const int32_t* page_table, int32_t num_seqs, int32_t max_pages,
                               void* c_KV, void* k_R, int64_t row_stride, int32_t num_pages,
                               int32_t* err_flag, void* workspace, size_t ws_bytes, void* stream);

/*
 * mla_decode_workspace_size -- bytes of device workspace mla_decode needs for
 * batch B with n_splits work partitions (0 = the library's default, one per
 * compute unit).  Returns 0 for invalid dims.
 */
size_t mla_decode_workspace_size(const mla_dims* dims, int32_t B, int32_t n_splits);

/*
 * mla_decode -- one decode query per sequence against its cached tokens.
 * (liang.world ch.2 §1 per-head softmax attention over earlier tokens; §2
 * absorption of W^UK into the query side, q~_i = W^UK_i^T q^C_i, and of W^UV
 * into the output side; §3 score = q^C.k^C + q^R.k^R.)
 * Steps, all in this library's kernels: plan (split the batch's tokens into
 * n_splits near-equal ranges), absorb (q~ and RoPE(q^R) at pos_q), split-KV
 * flash decode over the paged latent (all heads share each staged tile),
 * cross-split log-sum-exp combine, and the W^UV epilogue.
 *   q_C        [B, n_h, d_h]   dtype   device
 *   q_R        [B, n_h, d_hR]  dtype   device, NOT yet rotated
 *   pos_q      [B] int32       device  query positions (normally seq_lens[b]-1)
 *   W_UK, W_UV [n_h*d_h, d_c]  dtype   device
 *   c_KV, k_R, row_stride, num_pages   the pool, as for mla_cache_append
 *   page_table [B, max_pages]  int32   device
 *   seq_lens   [B] int32       device  cached tokens per sequence (>= 1; the
 *                                      query's own token is among them)
 *   out        [B, n_h, d_h]   fp32    device
 *   lse        [B, n_h] fp32 or NULL   natural-log softmax normaliser per head
 *   workspace  ws_bytes >= mla_decode_workspace_size(dims, B, n_splits),
 *              256-byte aligned device memory; it also holds the error flags.
 * Results are deterministic for fixed inputs and n_splits (no float atomics).
 */
mla_status mla_decode(const mla_dims* dims, int32_t B, const void* q_C, const void* q_R,
                      const int32_t* pos_q, const void* W_UK, const void* W_UV,
                      const void* c_KV, const void* k_R, int64_t row_stride, int32_t num_pages,
                      const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens,
                      float* out, float* lse, void* workspace, size_t ws_bytes, int32_t n_splits,
                      void* stream);

/*
 * mla_decode_ex -- mla_decode with options.  opts may be NULL (then it is
 * mla_decode).  ev_start / ev_stop are hipEvent_t handles (or NULL) recorded
 * on `stream` right before and right after the split-KV attention kernel, so
 * a caller can time that kernel alone.  impl selects the attention kernel:
 * 0 = default (bf16 MFMA kernel when dtype is bf16, n_h is 32, 64 or 128 and
 * page_size >= 32; otherwise the VALU kernel), 1 = always the VALU kernel.
 */
typedef struct mla_decode_opts {
  void* ev_start;
  void* ev_stop;
  int32_t impl;
} mla_decode_opts;

mla_status mla_decode_ex(const mla_dims* dims, int32_t B, const void* q_C, const void* q_R,
                         const int32_t* pos_q, const void* W_UK, const void* W_UV,
                         const void* c_KV, const void* k_R, int64_t row_stride, int32_t num_pages,
                         const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens,
                         float* out, float* lse, void* workspace, size_t ws_bytes, int32_t n_splits,
                         const mla_decode_opts* opts, void* stream);

/*
 * mla_decode_step_workspace_size -- bytes of device workspace mla_decode_step
 * needs for batch B and n_splits (0 = default); 0 for invalid dims.
 *
 * mla_decode_step -- one whole decode step: append each sequence's newest
 * token to the latent cache, then mla_decode.  Token b's state h_new[b] is
 * projected and stored exactly as mla_cache_append_ws with T = B, seq_id =
 * NULL (row b is sequence b) and pos = pos_q (liang.world ch.2 §2 eq. for
 * c_t^KV; tuntang.top MLA section, k_t formula), and the decode that follows
 * attends over seq_lens[b] tokens, the new one included (normally seq_lens[b]
 * = pos_q[b] + 1).  Results are bitwise those of mla_cache_append_ws followed
 * by mla_decode_ex with the same arguments.  For bf16 with d_model a multiple
 * of 1024 the append's split-K product (finished inside the same launch by the
 * last workgroup of each output tile), the query absorption and the plan run
 * as one launch, followed by the attention and combine launches; otherwise the
 * append is its own launch before the decode's.
 *   h_new        [B, d_model]  dtype   device
 *   W_DKV, W_KR  as for mla_cache_append
 *   c_KV, k_R    the pool, written (token pos_q[b] of sequence b) and read
 *   the other arguments as for mla_decode_ex (opts may be NULL).
 *   workspace    ws_bytes >= mla_decode_step_workspace_size(dims, B, n_splits),
 *                256-byte aligned device memory, ZERO-FILLED ONCE after
 *                allocation: it holds counters of the in-launch append
 *                reduction, which every completed call leaves at zero again.
 * Error flags: an append position outside [0, max_pages*page_size) skips that
 * row and raises MLA_FLAG_BAD_POSITION; it and the decode's flags are read
 * from the workspace with mla_read_error_flags.  Calls that share one
 * workspace must be ordered (e.g. on one stream).
 */
size_t mla_decode_step_workspace_size(const mla_dims* dims, int32_t B, int32_t n_splits);
mla_status mla_decode_step(const mla_dims* dims, int32_t B, const void* h_new, const void* W_DKV,
                           const void* W_KR, const void* q_C, const void* q_R, const int32_t* pos_q,
                           const void* W_UK, const void* W_UV, void* c_KV, void* k_R, int64_t row_stride,
                           int32_t num_pages, const int32_t* page_table, int32_t max_pages,
                           const int32_t* seq_lens, float* out, float* lse, void* workspace, size_t ws_bytes,
                           int32_t n_splits, const mla_decode_opts* opts, void* stream);

/*
 * mla_decode_step_noalloc -- mla_decode_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): no workspace argument, and nothing is allocated by
 * this call or by the library -- the step's scratch is a file-scope device
 * array of the library, 80 MiB, one copy per GPU, held until the process
 * ends.  Same kernels, same default split count (the device's CU count) and
 * bitwise the same results as mla_decode_step with n_splits = 0 and opts =
 * NULL; the arguments mean what they mean there.
 *   err_flags  NULL, or one int32 of device memory into which the step ORs
 *              its MLA_FLAG_* bits (the caller clears it).
 * Limit: the step's scratch for (B, n_h, CU count) must fit the 80 MiB
 * (mla_decode_step_workspace_size(dims, B, 0) <= 80 MiB: at n_h = 128 and
 * 256 CUs, B <= 167); larger batches return MLA_ERR_WORKSPACE (use
 * mla_decode_step).  The first call on each device looks up the array's
 * address and clears its counters with a small kernel on `stream`; make that
 * call outside graph capture.  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (several streams or threads) race and
 * must be ordered by the caller.
 */
mla_status mla_decode_step_noalloc(const mla_dims* dims, int32_t B, const void* h_new, const void* W_DKV,
                                   const void* W_KR, const void* q_C, const void* q_R, const int32_t* pos_q,
                                   const void* W_UK, const void* W_UV, void* c_KV, void* k_R, int64_t row_stride,
                                   int32_t num_pages, const int32_t* page_table, int32_t max_pages,
                                   const int32_t* seq_lens, float* out, float* lse, int32_t* err_flags,
                                   void* stream);

/*
 * mla_pack_weight -- copy a row-major weight W [rows, K] (dims.dtype) into
 * the packed layout the projection kernels stream (mla_query_project,
 * mla_output_project): blocks of 16 rows x 32 columns, block (rb, ks) at
 * element (rb*K/32 + ks)*512, inside it lane l's 8 elements (row 16rb + l%16,
 * columns 32ks + 8(l/16) .. +7) at l*8 -- the lane order of a 16x16x32 MFMA
 * operand, so that a wave reads each block as one contiguous 1 KB run.  A
 * permutation: W_packed holds rows*K elements.  Done once per weight.
 *   rows: multiple of 16; K: multiple of 32; W, W_packed 16-byte aligned,
 *   device memory, not overlapping.
 */
mla_status mla_pack_weight(const mla_dims* dims, int32_t rows, int32_t K, const void* W, void* W_packed,
                           void* stream);

/*
 * mla_query_project_workspace_size -- bytes of device workspace
 * mla_query_project needs for batch B and query rank d_cq; 0 for invalid
 * arguments.
 *
 * mla_query_project -- the decode queries of B tokens from their states h
 * (liang.world ch.2 §2, closing paragraph: the query has its own low-rank
 * compression c^Q; tuntang.top MLA section, "RoPE 的兼容性处理": q_t =
 * [W^UQ c_t^Q ; W^QR h_t RoPE(t)]):
 *     c^Q = W^DQ h     (d_cq wide; the pages give no formula or width for it:
 *                       this is the analogue of c^KV = W^DKV h)
 *     q^C = W^UQ c^Q   per head,  q^R = W^QR h  per head, NOT rotated
 * so that q_C / q_R feed mla_decode / mla_decode_step directly (they rotate
 * q^R at the query position).  d_cq == 0 means no down-projection (c^Q = h,
 * W_DQ NULL, W_UQ [n_h*d_h, d_model]).
 *   h          [B, d_model]          dtype   device
 *   W_DQ       [d_cq, d_model]       dtype   device, packed (NULL iff d_cq == 0)
 *   W_UQ       [n_h*d_h, d_cq]       dtype   device, packed ([n_h*d_h, d_model] when d_cq == 0)
 *   W_QR       [n_h*d_hR, d_model]   dtype   device, packed
 *   (packed: the weight's row-major form passed through mla_pack_weight)
 *   q_C        [B, n_h, d_h]         dtype   device, written
 *   q_R        [B, n_h, d_hR]        dtype   device, written
 *   workspace  ws_bytes >= mla_query_project_workspace_size(dims, B, d_cq),
 *              256-byte aligned device memory, ZERO-FILLED ONCE after
 *              allocation (it holds counters of in-launch split-K reductions,
 *              which every completed call leaves at zero); it also holds c^Q.
 * d_cq must be 0 or a multiple of 128; for bf16 d_model must be a multiple of
 * 128.  bf16: operands bf16, fp32 accumulation, c^Q rounded to bf16 before
 * the second product; fp32: everything fp32.  Deterministic for fixed inputs.
 * Calls that share one workspace must be ordered (e.g. on one stream).
 */
size_t mla_query_project_workspace_size(const mla_dims* dims, int32_t B, int32_t d_cq);
mla_status mla_query_project(const mla_dims* dims, int32_t B, int32_t d_cq, const void* h, const void* W_DQ,
                             const void* W_UQ, const void* W_QR, void* q_C, void* q_R, void* workspace,
                             size_t ws_bytes, void* stream);

/*
 * mla_output_project_workspace_size -- bytes of device workspace
 * mla_output_project needs for batch B; 0 for invalid arguments.
 *
 * mla_output_project -- u = W^O [o_1; ...; o_{n_h}] per token: the heads'
 * outputs concatenated in head order and multiplied by the output matrix
 * (liang.world ch.2 §1, the attention output step).
 *   o          [B, n_h, d_h]        fp32    device (as mla_decode writes it;
 *                                            rounded to bf16 for the bf16 product)
 *   W_O        [d_model, n_h*d_h]   dtype   device, packed (mla_pack_weight)
 *   u          [B, d_model]         fp32    device, written
 *   workspace  ws_bytes >= mla_output_project_workspace_size(dims, B),
 *              256-byte aligned, ZERO-FILLED ONCE (as for mla_query_project).
 * Deterministic for fixed inputs; calls sharing a workspace must be ordered.
 */
size_t mla_output_project_workspace_size(const mla_dims* dims, int32_t B);
mla_status mla_output_project(const mla_dims* dims, int32_t B, const float* o, const void* W_O, float* u,
                              void* workspace, size_t ws_bytes, void* stream);

/*
 * mla_prefill_workspace_size -- bytes of device workspace mla_prefill needs
 * for a chunk of T tokens, page-table rows of max_pages entries and n_splits
 * (0 = default); 0 for invalid arguments.
 *
 * mla_prefill -- a chunk of T new tokens, any mix of sequences (chunked
 * prefill, or several decode tokens per sequence).  Token t belongs to
 * sequence seq_id[t] at position pos[t]; all T rows are first appended to the
 * latent cache as mla_cache_append would (liang.world ch.2 §2 eq. for c_t^KV;
 * tuntang.top MLA section, k_t formula), through the split path of
 * mla_cache_append_ws when the chunk fits it (up to 1024 rows, chunk sums in
 * part of this workspace; only the fp32 summation order differs); then token t attends causally to rows
 * 0 .. pos[t] of its sequence, earlier tokens of the same chunk included
 * (liang.world ch.2 §1: a token attends to the tokens before it and itself),
 * exactly as mla_decode with one query per new token.
 *   h            [T, d_model]      dtype   device
 *   W_DKV, W_KR  as for mla_cache_append
 *   q_C, q_R     [T, n_h, d_h], [T, n_h, d_hR] dtype device (q_R not rotated)
 *   seq_id, pos  [T] int32         device  sequence and position of each token
 *   W_UK, W_UV   as for mla_decode
 *   c_KV, k_R, row_stride, num_pages, page_table [num_seqs, max_pages]: the pool
 *   out          [T, n_h, d_h] fp32, lse [T, n_h] fp32 or NULL
 *   workspace    ws_bytes >= mla_prefill_workspace_size(dims, T, max_pages, n_splits),
 *                256-byte aligned device memory; holds the error flags.
 * A token with a bad sequence id or position is not appended, its output is
 * empty (out = 0, lse = -inf) and MLA_FLAG_BAD_SEQ_ID / BAD_POSITION /
 * BAD_SEQ_LEN are raised (mla_read_error_flags).  Deterministic for fixed
 * inputs and n_splits.
 */
size_t mla_prefill_workspace_size(const mla_dims* dims, int32_t T, int32_t max_pages, int32_t n_splits);
mla_status mla_prefill(const mla_dims* dims, int32_t T, const void* h, const void* W_DKV, const void* W_KR,
                       const void* q_C, const void* q_R, const int32_t* seq_id, const int32_t* pos, const void* W_UK,
                       const void* W_UV, void* c_KV, void* k_R, int64_t row_stride, int32_t num_pages,
                       const int32_t* page_table, int32_t num_seqs, int32_t max_pages, float* out, float* lse,
                       void* workspace, size_t ws_bytes, int32_t n_splits, void* stream);

/*
 * mla_decode_layer_workspace_size -- bytes of device workspace
 * mla_decode_layer needs for batch B, query rank d_cq and n_splits (0 =
 * default); 0 for invalid arguments.
 *
 * mla_decode_layer -- one MLA attention layer for one decode token per
 * sequence, from the token states h to the layer output u: the query path
 * (mla_query_project), the decode step (mla_decode_step: append of the token's
 * latent row, absorption, attention over the cache, combine + W^UV) and the
 * output projection (mla_output_project), on the same stream and with the
 * same results as those three calls, except in one case.  With bf16, a
 * low-rank query (d_cq > 0), more than 8 sequences and d_model a multiple of
 * 1024, q^C = W^UQ c^Q is formed inside the absorption launch and never stored
 * ("DeepSeek-V2：在“大力出奇迹”的AI军备竞赛中，四两拨千斤" (liang.world), ch.2 §2:
 * the query's low-rank compression c^Q, absorbed with W^UK).  Its fp32 sums
 * then run in another order before the bf16 rounding of q^C, so u and lse
 * agree with the three calls to within that rounding, not bit for bit.
 *   h            [B, d_model]     dtype   device  state of each sequence's new token
 *   W_DKV, W_KR  row-major, as for mla_cache_append
 *   W_DQ, W_UQ, W_QR   packed, as for mla_query_project (W_DQ NULL iff d_cq == 0)
 *   W_UK, W_UV   row-major, as for mla_decode
 *   W_O          packed, as for mla_output_project
 *   pos_q, c_KV, k_R, row_stride, num_pages, page_table, max_pages, seq_lens, opts:
 *                as for mla_decode_step (the new token is written at pos_q[b])
 *   u            [B, d_model] fp32 device, written;  lse [B, n_h] fp32 or NULL
 *   workspace    ws_bytes >= mla_decode_layer_workspace_size(dims, B, d_cq, n_splits),
 *                256-byte aligned, ZERO-FILLED ONCE (split-K counters); its
 *                first word holds the error flags (mla_read_error_flags).
 */
size_t mla_decode_layer_workspace_size(const mla_dims* dims, int32_t B, int32_t d_cq, int32_t n_splits);
mla_status mla_decode_layer(const mla_dims* dims, int32_t B, int32_t d_cq, const void* h, const void* W_DKV,
                            const void* W_KR, const void* W_DQ, const void* W_UQ, const void* W_QR, const void* W_UK,
                            const void* W_UV, const void* W_O, const int32_t* pos_q, void* c_KV, void* k_R,
                            int64_t row_stride, int32_t num_pages, const int32_t* page_table, int32_t max_pages,
                            const int32_t* seq_lens, float* u, float* lse, void* workspace, size_t ws_bytes,
                            int32_t n_splits, const mla_decode_opts* opts, void* stream);

/*
 * Sparse top-k decode (reading of "DeepSeek 架构精讲：从 V3 到 V4",
 * cyco.top, §4 V3.2 bullet and §6 question 7: a light indexer picks the few
 * most relevant cached tokens, and attention then looks at those alone).
 * Every cached token j carries an indexer key k^I_j (d_I bf16) in a paged
 * pool that shares the latent cache's page table; a decode query carries
 * H_I indexer heads q^I_h (bf16) and weights w_h (fp32).  The relevance is
 *   I_j = sum_h w_h * max(0, q^I_h . k^I_j)                  (fp32)
 * and each sequence keeps its top_k tokens of largest I_j, equal scores
 * going to the smaller token index (all tokens when seq_len <= top_k).  The
 * selection is exact integer work on order-preserving keys of the fp32
 * scores, so it is deterministic.  Supported: d_I = 128, H_I in {16, 32,
 * 64}, page_size a multiple of 16 (of 32 for mla_sparse_decode).
 *
 * mla_indexer_select_workspace_size -- bytes of scratch mla_indexer_select
 * needs; 0 for invalid sizes.
 *
 * mla_indexer_select -- scores and selection only.
 *   q_I        [B, H_I, d_I]   bf16    device
 *   w_I        [B, H_I]        fp32    device
 *   k_I        [num_pages*page_size, idx_row_stride] bf16 device, the key of
 *              token t of sequence b at row page_table[b][t/page_size] *
 *              page_size + t % page_size
 *   page_table [B, max_pages] int32, seq_lens [B] int32    device
 *   scores     [B, max_pages*page_size] fp32 device out, 16-byte aligned:
 *              I_j at [b][j] for j < seq_len (the rest untouched)
 *   sel_tok    [B, top_k] int32 device out: the kept tokens, ascending
 *   sel_row    [B, top_k] int32 device out: their pool rows
 *              (entries past min(seq_len, top_k) are left untouched)
 *   err_flags  int32 device word: MLA_FLAG_BAD_PAGE (page clamped) is OR-ed
 *              in; seq_len outside [1, max_pages*page_size] is clamped
 *   workspace  ws_bytes >= mla_indexer_select_workspace_size(), 256-byte
 *              aligned; needs no initialisation.
 *
 * mla_sparse_decode_workspace_size -- bytes of device workspace
 * mla_sparse_decode needs (n_splits 0 = default); 0 for invalid arguments.
 *
 * mla_sparse_decode -- the whole sparse decode: query absorption, indexer
 * scores, selection, split-KV attention over the kept latent rows only
 * (each split copies the rows of its list positions straight from the pool),
 * log-sum-exp combine and the W^UV epilogue.  out / lse are those of
 * mla_decode with the softmax over the kept tokens.  Arguments as for
 * mla_decode_ex (bf16, n_h in {32, 64, 128}) and mla_indexer_select; sel_tok
 * (optional, [B, top_k] int32) receives the kept tokens.  n_splits 0 picks
 * about one split per 128 kept tokens, at most one per CU.  The error flags
 * sit in the workspace's first word, as for mla_decode.  opts: ev_start /
 * ev_stop as for mla_decode_ex; impl must be 0.
 */
size_t mla_indexer_select_workspace_size(int32_t B, int32_t max_pages, int32_t page_size, int32_t top_k);
mla_status mla_indexer_select(int32_t B, int32_t H_I, int32_t d_I, int32_t top_k, const void* q_I,
                              const float* w_I, const void* k_I, int64_t idx_row_stride, int32_t num_pages,
                              int32_t page_size, const int32_t* page_table, int32_t max_pages,
                              const int32_t* seq_lens, float* scores, int32_t* sel_tok, int32_t* sel_row,
                              int32_t* err_flags, void* workspace, size_t ws_bytes, void* stream);
size_t mla_sparse_decode_workspace_size(const mla_dims* dims, int32_t B, int32_t max_pages, int32_t top_k,
                                        int32_t n_splits);
mla_status mla_sparse_decode(const mla_dims* dims, int32_t B, const void* q_C, const void* q_R,
                             const int32_t* pos_q, const void* W_UK, const void* W_UV, const void* c_KV,
                             const void* k_R, int64_t row_stride, int32_t num_pages, const int32_t* page_table,
                             int32_t max_pages, const int32_t* seq_lens, int32_t H_I, int32_t d_I, int32_t top_k,
                             const void* q_I, const float* w_I, const void* k_I, int64_t idx_row_stride,
                             float* out, float* lse, int32_t* sel_tok, void* workspace, size_t ws_bytes,
                             int32_t n_splits, const mla_decode_opts* opts, void* stream);

/*
 * mla_read_error_flags -- wait for `stream`, then copy the device error flags
 * of a decode workspace (or an append err_flag word) to *flags and clear them.
 */
mla_status mla_read_error_flags(void* workspace_or_flag, int32_t* flags, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* mla_last_error(void);

/* Number of compute units of the current device (default n_splits). */
int32_t mla_device_cu_count(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
