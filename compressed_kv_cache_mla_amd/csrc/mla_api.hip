// C ABI entry points of libmla.so: argument checks, workspace layout,
// kernel selection and launch order.  No device memory is allocated here.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <string>
#include <tuple>

#include "append_splitk.h"

namespace {

thread_local std::string g_err;

// Limits every entry point shares: batch rows (B, T), work partitions and
// pool row strides (elements).  Within them every size and offset below fits
// its type.
constexpr int32_t MAX_ROWS = 1 << 20;
constexpr int32_t MAX_SPLITS = 1 << 20;
constexpr int64_t MAX_ROW_STRIDE = (int64_t)1 << 24;

mla_status fail(mla_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mla_status fail(mla_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

mla_status ok() {
  g_err.clear();
  return MLA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int elt_size(const mla_dims* d) { return d->dtype == MLA_FP32 ? 4 : 2; }

// x > 0 and finite, decided on the bits: the library is built with
// -fno-honor-nans, under which a float comparison may treat a NaN as ordered.
bool positive_finite(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  return (u >> 31) == 0 && u != 0 && ((u >> 23) & 0xff) != 0xff;
}

mla_status check_dims(const mla_dims* d) {
  if (!d) return fail(MLA_ERR_INVALID_ARG, "dims is NULL");
  if (d->dtype != MLA_BF16 && d->dtype != MLA_FP32) return fail(MLA_ERR_INVALID_ARG, "bad dtype %d", d->dtype);
  if (d->d_c != mla::D_C || d->d_hR != mla::D_R || d->d_h != mla::D_H)
    return fail(MLA_ERR_UNSUPPORTED, "kernels are built for d_c=512, d_hR=64, d_h=128 (got %d, %d, %d)", d->d_c,
                d->d_hR, d->d_h);
  if (d->n_h < 1 || d->n_h > 1024) return fail(MLA_ERR_INVALID_ARG, "n_h=%d out of range", d->n_h);
  if (d->d_model < 64 || d->d_model % 64 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "d_model=%d must be a positive multiple of 64", d->d_model);
  if (d->page_size < 1) return fail(MLA_ERR_INVALID_ARG, "page_size=%d must be >= 1", d->page_size);
  if (!positive_finite(d->softmax_scale) || !positive_finite(d->rope_base))
    return fail(MLA_ERR_INVALID_ARG, "softmax_scale and rope_base must be positive and finite");
  return MLA_OK;
}

mla_status check_pool(const mla_dims* d, const void* c_KV, const void* k_R, int64_t row_stride, int32_t num_pages) {
  if (!c_KV || !k_R) return fail(MLA_ERR_INVALID_ARG, "c_KV / k_R is NULL");
  if (!aligned16(c_KV) || !aligned16(k_R)) return fail(MLA_ERR_INVALID_ARG, "c_KV / k_R not 16-byte aligned");
  if (row_stride < mla::D_C || row_stride > MAX_ROW_STRIDE || (row_stride * elt_size(d)) % 16 != 0)
    return fail(MLA_ERR_INVALID_ARG, "row_stride=%lld must be in [512, 2^24] and a multiple of 16 bytes",
                (long long)row_stride);
  if (num_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_pages=%d must be >= 1", num_pages);
  if ((int64_t)num_pages * d->page_size >= ((int64_t)1 << 31))
    return fail(MLA_ERR_UNSUPPORTED, "pool holds more than 2^31 rows");
  return MLA_OK;
}

int32_t default_splits();

// n_splits as the calls take it: <= 0 selects the default; -1 when above the limit.
int32_t resolve_splits(int32_t n_splits) {
  if (n_splits <= 0) return default_splits();
  return n_splits > MAX_SPLITS ? -1 : n_splits;
}

int32_t default_splits() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  return cus;
}

}  // namespace

extern "C" {

const char* mla_last_error(void) { return g_err.c_str(); }

int32_t mla_device_cu_count(void) { return default_splits(); }

static mla_status cache_append_impl(const mla_dims* dims, int32_t T, const void* h_t, const void* W_DKV,
                                    const void* W_KR, const int32_t* seq_id, const int32_t* pos,
                                    const int32_t* page_table, int32_t num_seqs, int32_t max_pages, void* c_KV,
                                    void* k_R, int64_t row_stride, int32_t num_pages, int32_t* err_flag,
                                    void* workspace, size_t ws_bytes, void* stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (T < 0 || T > MAX_ROWS) return fail(MLA_ERR_INVALID_ARG, "T=%d out of range [0, 2^20]", T);
  if (T == 0) return ok();
  if (!h_t || !W_DKV || !W_KR || !pos || !page_table)
    return fail(MLA_ERR_INVALID_ARG, "null pointer among h_t, W_DKV, W_KR, pos, page_table");
  if (!aligned16(h_t) || !aligned16(W_DKV) || !aligned16(W_KR))
    return fail(MLA_ERR_INVALID_ARG, "h_t / W_DKV / W_KR not 16-byte aligned");
  if (num_seqs < 1 || max_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_seqs and max_pages must be >= 1");
  if (!seq_id && T > num_seqs) return fail(MLA_ERR_INVALID_ARG, "seq_id NULL needs T <= num_seqs");
  st = check_pool(dims, c_KV, k_R, row_stride, num_pages);
  if (st != MLA_OK) return st;
  if ((int64_t)max_pages * dims->page_size >= ((int64_t)1 << 31))
    return fail(MLA_ERR_UNSUPPORTED, "max_pages*page_size >= 2^31");
  if (workspace && ((uintptr_t)workspace & 255) != 0)
    return fail(MLA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  hipError_t e = mla::launch_append(*dims, T, h_t, W_DKV, W_KR, seq_id, pos, page_table, num_seqs, max_pages, c_KV,
                                    k_R, row_stride, num_pages, err_flag, workspace, ws_bytes, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "append launch: %s", hipGetErrorString(e));
  return ok();
}

mla_status mla_cache_append(const mla_dims* dims, int32_t T, const void* h_t, const void* W_DKV, const void* W_KR,
                            const int32_t* seq_id, const int32_t* pos, const int32_t* page_table,
                            int32_t num_seqs, int32_t max_pages, void* c_KV, void* k_R, int64_t row_stride,
                            int32_t num_pages, int32_t* err_flag, void* stream) {
  return cache_append_impl(dims, T, h_t, W_DKV, W_KR, seq_id, pos, page_table, num_seqs, max_pages, c_KV, k_R,
                           row_stride, num_pages, err_flag, nullptr, 0, stream);
}

size_t mla_cache_append_workspace_size(const mla_dims* dims, int32_t T) {
  if (check_dims(dims) != MLA_OK || T < 1 || T > MAX_ROWS) return 0;
  return mla::append_workspace_bytes(*dims, T);
}

mla_status mla_cache_append_ws(const mla_dims* dims, int32_t T, const void* h_t, const void* W_DKV,
                               const void* W_KR, const int32_t* seq_id, const int32_t* pos,
                               const int32_t* page_table, int32_t num_seqs, int32_t max_pages, void* c_KV,
                               void* k_R, int64_t row_stride, int32_t num_pages, int32_t* err_flag,
                               void* workspace, size_t ws_bytes, void* stream) {
  return cache_append_impl(dims, T, h_t, W_DKV, W_KR, seq_id, pos, page_table, num_seqs, max_pages, c_KV, k_R,
                           row_stride, num_pages, err_flag, workspace, ws_bytes, stream);
}

size_t mla_decode_workspace_size(const mla_dims* dims, int32_t B, int32_t n_splits) {
  if (check_dims(dims) != MLA_OK || B < 1 || B > MAX_ROWS) return 0;
  n_splits = resolve_splits(n_splits);
  if (n_splits < 0) return 0;
  return mla::decode_ws_layout(B, dims->n_h, n_splits, elt_size(dims)).total;
}

mla_status mla_decode(const mla_dims* dims, int32_t B, const void* q_C, const void* q_R, const int32_t* pos_q,
                      const void* W_UK, const void* W_UV, const void* c_KV, const void* k_R, int64_t row_stride,
                      int32_t num_pages, const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens,
                      float* out, float* lse, void* workspace, size_t ws_bytes, int32_t n_splits, void* stream) {
  return mla_decode_ex(dims, B, q_C, q_R, pos_q, W_UK, W_UV, c_KV, k_R, row_stride, num_pages, page_table, max_pages,
                       seq_lens, out, lse, workspace, ws_bytes, n_splits, nullptr, stream);
}

// Inputs of the append half of a decode step.
struct StepAppendIn {
  const void* h_new;
  const void* W_DKV;
  const void* W_KR;
  void* o_packed;   // optional: the combine also writes out as the output projection's packed bf16 activations
};

// The decode layer's query path fused with the absorption: q^C = W^UQ c^Q is
// formed by the absorption launch from the packed c^Q (rows padded to a
// multiple of 64) and the packed W^UQ; q_C is then not read.
struct FusedQuery {
  const void* cQ_packed;
  const void* W_UQ_packed;
  int32_t d_cq;
};

static mla_status decode_impl(const mla_dims* dims, int32_t B, const void* q_C, const void* q_R, const int32_t* pos_q,
                              const void* W_UK, const void* W_UV, const void* c_KV, const void* k_R,
                              int64_t row_stride, int32_t num_pages, const int32_t* page_table, int32_t max_pages,
                              const int32_t* seq_lens, float* out, float* lse, void* workspace, size_t ws_bytes,
                              int32_t n_splits, const mla_decode_opts* opts, const StepAppendIn* step,
                              void* stream, bool merge_append_flags = false, int32_t* ext_flags = nullptr,
                              const FusedQuery* fq = nullptr) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (B < 1 || B > MAX_ROWS) return fail(MLA_ERR_INVALID_ARG, "B=%d out of range [1, 2^20]", B);
  if (!q_C || !q_R || !pos_q || !W_UK || !W_UV || !page_table || !seq_lens || !out || !workspace)
    return fail(MLA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(q_C) || !aligned16(q_R) || !aligned16(W_UK) || !aligned16(W_UV) || !aligned16(out))
    return fail(MLA_ERR_INVALID_ARG, "q_C / q_R / W_UK / W_UV / out not 16-byte aligned");
  if (step) {
    if (!step->h_new || !step->W_DKV || !step->W_KR)
      return fail(MLA_ERR_INVALID_ARG, "null pointer among h_new, W_DKV, W_KR");
    if (!aligned16(step->h_new) || !aligned16(step->W_DKV) || !aligned16(step->W_KR))
      return fail(MLA_ERR_INVALID_ARG, "h_new / W_DKV / W_KR not 16-byte aligned");
  }
  if (((uintptr_t)workspace & 255) != 0) return fail(MLA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  st = check_pool(dims, c_KV, k_R, row_stride, num_pages);
  if (st != MLA_OK) return st;
  if (max_pages < 1 || (int64_t)max_pages * dims->page_size >= ((int64_t)1 << 31))
    return fail(MLA_ERR_INVALID_ARG, "max_pages=%d out of range", max_pages);
  if ((int64_t)B * max_pages * dims->page_size >= ((int64_t)1 << 31))
    return fail(MLA_ERR_UNSUPPORTED, "B*max_pages*page_size >= 2^31 tokens");
  const int32_t n_req = n_splits;
  n_splits = resolve_splits(n_splits);
  if (n_splits < 0) return fail(MLA_ERR_INVALID_ARG, "n_splits=%d above 2^20", n_req);
  const mla::DecodeWs L = mla::decode_ws_layout(B, dims->n_h, n_splits, elt_size(dims), step != nullptr);
  if (ws_bytes < L.total)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total);

  char* ws = (char*)workspace;
  int32_t* flags = (int32_t*)(ws + L.flags);
  int32_t* prefix = (int32_t*)(ws + L.prefix);
  int32_t* split_rec = (int32_t*)(ws + L.splits);
  void* qabs = ws + L.qabs;
  float* part_ml = (float*)(ws + L.part_ml);
  void* part_o = ws + L.part_o;
  hipStream_t s = (hipStream_t)stream;
  const int32_t max_tokens = max_pages * dims->page_size;

  mla::PlanArgs pa;
  pa.seq_lens = seq_lens;
  pa.B = B;
  pa.max_tokens = max_tokens;
  pa.G = n_splits;
  pa.prefix = prefix;
  pa.split_rec = split_rec;
  pa.flags = flags;
  pa.page_table = page_table;
  pa.max_pages = max_pages;
  pa.page_size = dims->page_size;
  if (opts && opts->impl != 0 && opts->impl != 1) return fail(MLA_ERR_INVALID_ARG, "opts->impl=%d", opts->impl);
  if (fq && !(step && mla::step_prep_supported(*dims, B) && mla::absorb_fused_supported(*dims, B, fq->d_cq)))
    return fail(MLA_ERR_UNSUPPORTED, "the fused query absorption needs the one-launch step (bf16, d_model %% 1024 == 0)");
  hipError_t e = hipSuccess;
  if (step && mla::step_prep_supported(*dims, B)) {
    // append (split-K, finished in the same launch), absorption and plan in one launch
    const mla::AppendDst dst{nullptr, pos_q, page_table, B, max_pages, dims->page_size, num_pages,
                             (mla::bf16*)c_KV, (mla::bf16*)k_R, row_stride, mla::rope_table(dims->rope_base),
                             flags + 1};
    e = mla::launch_step_prep(*dims, B, step->h_new, step->W_DKV, step->W_KR, q_C, q_R, pos_q, W_UK, qabs, pa,
                              (float*)(ws + L.app_part), (int32_t*)(ws + L.app_cnt), dst, s, fq == nullptr);
    if (e == hipSuccess && fq)
      e = mla::launch_absorb_fused(*dims, B, fq->d_cq, fq->cQ_packed, fq->W_UQ_packed, q_R, pos_q, W_UK, qabs, s);
  } else {
    if (step)
      e = mla::launch_append(*dims, B, step->h_new, step->W_DKV, step->W_KR, nullptr, pos_q, page_table, B,
                             max_pages, (void*)c_KV, (void*)k_R, row_stride, num_pages, flags + 1, nullptr, 0, s);
    if (e == hipSuccess) e = mla::launch_absorb(*dims, B, q_C, q_R, pos_q, W_UK, qabs, pa, s);
  }
  if (e == hipSuccess && opts && opts->ev_start) e = hipEventRecord((hipEvent_t)opts->ev_start, s);
  if (e == hipSuccess) {
    const bool mfma = dims->dtype == MLA_BF16 && (dims->n_h == 32 || dims->n_h == 64 || dims->n_h == 128) &&
                      dims->page_size >= 32 && !(opts && opts->impl == 1);
    if (mfma)
      e = mla::launch_decode_mfma(*dims, B, qabs, c_KV, k_R, row_stride, num_pages, page_table, max_pages, prefix,
                                  split_rec, n_splits, part_ml, part_o, flags, s);
    else
      e = mla::launch_decode_simple(*dims, B, qabs, c_KV, k_R, row_stride, num_pages, page_table, max_pages,
                                    prefix, n_splits, part_ml, part_o, flags, s);
  }
  if (e == hipSuccess && opts && opts->ev_stop) e = hipEventRecord((hipEvent_t)opts->ev_stop, s);
  if (e == hipSuccess)
    e = mla::launch_combine(*dims, B, prefix, n_splits, part_ml, part_o, W_UV, out, lse,
                            step || merge_append_flags ? flags : nullptr, step ? step->o_packed : nullptr, s,
                            ext_flags);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

mla_status mla_decode_ex(const mla_dims* dims, int32_t B, const void* q_C, const void* q_R, const int32_t* pos_q,
                         const void* W_UK, const void* W_UV, const void* c_KV, const void* k_R, int64_t row_stride,
                         int32_t num_pages, const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens,
                         float* out, float* lse, void* workspace, size_t ws_bytes, int32_t n_splits,
                         const mla_decode_opts* opts, void* stream) {
  return decode_impl(dims, B, q_C, q_R, pos_q, W_UK, W_UV, c_KV, k_R, row_stride, num_pages, page_table, max_pages,
                     seq_lens, out, lse, workspace, ws_bytes, n_splits, opts, nullptr, stream);
}

size_t mla_decode_step_workspace_size(const mla_dims* dims, int32_t B, int32_t n_splits) {
  if (check_dims(dims) != MLA_OK || B < 1 || B > MAX_ROWS) return 0;
  n_splits = resolve_splits(n_splits);
  if (n_splits < 0) return 0;
  return mla::decode_ws_layout(B, dims->n_h, n_splits, elt_size(dims), true).total;
}

mla_status mla_decode_step(const mla_dims* dims, int32_t B, const void* h_new, const void* W_DKV, const void* W_KR,
                           const void* q_C, const void* q_R, const int32_t* pos_q, const void* W_UK,
                           const void* W_UV, void* c_KV, void* k_R, int64_t row_stride, int32_t num_pages,
                           const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens, float* out,
                           float* lse, void* workspace, size_t ws_bytes, int32_t n_splits,
                           const mla_decode_opts* opts, void* stream) {
  const StepAppendIn in{h_new, W_DKV, W_KR, nullptr};
  return decode_impl(dims, B, q_C, q_R, pos_q, W_UK, W_UV, c_KV, k_R, row_stride, num_pages, page_table, max_pages,
                     seq_lens, out, lse, workspace, ws_bytes, n_splits, opts, &in, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- projections
namespace {

// Launch plan of the query projection for batch B.  d_cq > 0: product 1 is
// h . [W^DQ ; W^QR]^T -> (c^Q in the workspace, q^R), product 2 is
// c^Q . W^UQ^T -> q^C.  d_cq == 0 (no down-projection): product 1 is
// h . [W^UQ ; W^QR]^T -> (q^C, q^R).
struct QueryPlan {
  bool lowrank, packed;
  int32_t N1, S1, N2, S2;
  bool pack_h;   // h packed by a launch of its own (else read row-major, or rows <= 8)
  size_t off_h, off_cq, off_part, total;
};

// Workspace: split-K tile counters (fixed offset 0), h packed (bf16, more
// than a few rows, except 17..32 rows, read row-major), c^Q (packed above a
// few rows, else row-major), then the chunk sums
// (shared by the two products, which run one after the other).
QueryPlan query_plan(const mla_dims& d, int32_t B, int32_t d_cq) {
  QueryPlan p{};
  const bool bf = d.dtype == MLA_BF16;
  p.lowrank = d_cq > 0;
  p.packed = bf && mla::gemm_x_packed(B);
  p.pack_h = p.packed && !mla::gemm_x_rows_wide(B);
  const int64_t rows = p.packed ? mla::gemm_rows_padded(B) : B;
  p.N1 = (p.lowrank ? d_cq : d.n_h * mla::D_H) + d.n_h * mla::D_R;
  p.S1 = bf ? mla::gemm_pick_splits(B, p.N1, d.d_model) : 1;
  p.N2 = p.lowrank ? d.n_h * mla::D_H : 0;
  p.S2 = bf && p.lowrank ? mla::gemm_pick_splits(B, p.N2, d_cq) : 1;
  p.off_h = mla::SPLITK_COUNTER_BYTES;
  p.off_cq = p.off_h + (p.pack_h ? mla::align256((size_t)rows * d.d_model * 2) : 0);
  p.off_part = p.off_cq + (p.lowrank ? mla::align256((size_t)rows * d_cq * (bf ? 2 : 4)) : 0);
  const size_t part = std::max(mla::gemm_part_bytes(B, p.N1, p.S1), p.lowrank ? mla::gemm_part_bytes(B, p.N2, p.S2) : 0);
  p.total = p.off_part + (bf ? part : 0);
  return p;
}

// Output projection workspace: counters, o packed (bf16, more than a few
// rows), chunk sums.
struct OutputPlan {
  bool packed;
  int32_t S;
  size_t off_o, off_part, total;
};

OutputPlan output_plan(const mla_dims& d, int32_t B) {
  OutputPlan p{};
  const bool bf = d.dtype == MLA_BF16;
  const int32_t K = d.n_h * mla::D_H;
  p.packed = bf && mla::gemm_x_packed(B);
  p.S = bf ? mla::gemm_pick_splits(B, d.d_model, K) : 1;
  p.off_o = mla::SPLITK_COUNTER_BYTES;
  p.off_part = p.off_o + (p.packed ? mla::align256((size_t)mla::gemm_rows_padded(B) * K * 2) : 0);
  p.total = p.off_part + (bf ? mla::gemm_part_bytes(B, d.d_model, p.S) : 0);
  return p;
}

mla_status check_query_dims(const mla_dims* dims, int32_t B, int32_t d_cq) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (B < 1 || B > MAX_ROWS) return fail(MLA_ERR_INVALID_ARG, "B=%d out of range [1, 2^20]", B);
  if (d_cq < 0 || d_cq > 65536 || d_cq % 128 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "d_cq=%d must be 0 or a positive multiple of 128 up to 65536", d_cq);
  if (dims->dtype == MLA_BF16 && dims->d_model % 128 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "bf16 projections need d_model %% 128 == 0 (got %d)", dims->d_model);
  return MLA_OK;
}

mla::GemmArgs gemm_args(const void* X, int64_t ldx, int32_t M, int32_t K, char* counters) {
  mla::GemmArgs g{};
  g.counters = (int32_t*)counters;
  g.X = X;
  g.ldx = ldx;
  g.M = M;
  g.K = K;
  g.S = 1;
  return g;
}

// Stacks the weight segments (W, rows) of a product; unused segments end at N.
void gemm_segments(mla::GemmArgs& g, mla::GemmOut& o, std::initializer_list<std::tuple<const void*, int32_t, void*, int64_t>> segs) {
  int i = 0, end = 0;
  for (const auto& sg : segs) {
    end += std::get<1>(sg);
    g.W[i] = (const mla::bf16*)std::get<0>(sg);
    g.seg_end[i] = end;
    o.Y[i] = std::get<2>(sg);
    o.ldy[i] = std::get<3>(sg);
    ++i;
  }
  g.N = end;
  for (; i < mla::GK_SEG; ++i) {
    g.W[i] = nullptr;
    g.seg_end[i] = end;
    o.Y[i] = nullptr;
    o.ldy[i] = 0;
  }
}

}  // namespace

extern "C" {

size_t mla_query_project_workspace_size(const mla_dims* dims, int32_t B, int32_t d_cq) {
  if (check_query_dims(dims, B, d_cq) != MLA_OK) return 0;
  return query_plan(*dims, B, d_cq).total;
}

}  // extern "C"

// counters: the split-K tile counters of the two products (SPLITK_COUNTER_BYTES
// of zeros); the public entry point passes the block at offset 0 of its
// workspace, the whole layer a block at a fixed offset of its own.
// first_only (low-rank, bf16, packed c^Q): only c^Q and q^R are formed; c^Q
// stays packed in the workspace for the fused absorption.
static mla_status query_project_impl(const mla_dims* dims, int32_t B, int32_t d_cq, const void* h, const void* W_DQ,
                                     const void* W_UQ, const void* W_QR, void* q_C, void* q_R, void* workspace,
                                     size_t ws_bytes, void* stream, char* counters, bool first_only = false) {
  mla_status st = check_query_dims(dims, B, d_cq);
  if (st != MLA_OK) return st;
  if (!h || !W_UQ || !W_QR || !q_C || !q_R || !workspace)
    return fail(MLA_ERR_INVALID_ARG, "null pointer among h, W_UQ, W_QR, q_C, q_R, workspace");
  if ((d_cq > 0) != (W_DQ != nullptr))
    return fail(MLA_ERR_INVALID_ARG, "W_DQ must be given exactly when d_cq > 0 (d_cq=%d)", d_cq);
  if (!aligned16(h) || !aligned16(W_UQ) || !aligned16(W_QR) || !aligned16(q_C) || !aligned16(q_R) ||
      (W_DQ && !aligned16(W_DQ)))
    return fail(MLA_ERR_INVALID_ARG, "h / weights / q_C / q_R not 16-byte aligned");
  if (((uintptr_t)workspace & 255) != 0) return fail(MLA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  const QueryPlan p = query_plan(*dims, B, d_cq);
  if (ws_bytes < p.total)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, p.total);
  const bool f32 = dims->dtype == MLA_FP32;
  const int32_t nq = dims->n_h * mla::D_H, nr = dims->n_h * mla::D_R;
  char* ws = (char*)workspace;
  void* c_Q = ws + p.off_cq;
  hipStream_t s = (hipStream_t)stream;
  const int64_t rows = mla::gemm_rows_padded(B);
  hipError_t e = hipSuccess;
  const void* X1 = h;
  if (p.pack_h) {
    e = mla::launch_pack(h, dims->d_model, B, rows, dims->d_model, false, false, ws + p.off_h, s);
    X1 = ws + p.off_h;
  }
  mla::GemmArgs g = gemm_args(X1, dims->d_model, B, dims->d_model, counters ? counters : ws);
  g.x_rows = p.packed && !p.pack_h;
  mla::GemmOut o{};
  if (p.lowrank)
    gemm_segments(g, o, {{W_DQ, d_cq, c_Q, p.packed ? -(int64_t)d_cq : d_cq}, {W_QR, nr, q_R, nr}});
  else
    gemm_segments(g, o, {{W_UQ, nq, q_C, nq}, {W_QR, nr, q_R, nr}});
  g.S = p.S1;
  g.part = (float*)(ws + p.off_part);
  if (e == hipSuccess) e = mla::launch_gemm(g, o, f32, f32, f32, s);
  if (e == hipSuccess && p.lowrank && !first_only) {
    mla::GemmArgs g2 = gemm_args(c_Q, d_cq, B, d_cq, counters ? counters : ws);
    mla::GemmOut o2{};
    gemm_segments(g2, o2, {{W_UQ, nq, q_C, nq}});
    g2.S = p.S2;
    g2.part = (float*)(ws + p.off_part);
    e = mla::launch_gemm(g2, o2, f32, f32, f32, s);
  }
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "query projection launch: %s", hipGetErrorString(e));
  return ok();
}

extern "C" {

mla_status mla_query_project(const mla_dims* dims, int32_t B, int32_t d_cq, const void* h, const void* W_DQ,
                             const void* W_UQ, const void* W_QR, void* q_C, void* q_R, void* workspace,
                             size_t ws_bytes, void* stream) {
  return query_project_impl(dims, B, d_cq, h, W_DQ, W_UQ, W_QR, q_C, q_R, workspace, ws_bytes, stream, nullptr);
}

size_t mla_output_project_workspace_size(const mla_dims* dims, int32_t B) {
  if (check_query_dims(dims, B, 0) != MLA_OK) return 0;
  return output_plan(*dims, B).total;
}

}  // extern "C"

// o_prepacked: o's packed bf16 copy is already in the workspace (written by the
// combine of the decode layer), so the pack launch is skipped.  counters: as
// for query_project_impl (NULL: the block at offset 0 of the workspace).
static mla_status output_project_impl(const mla_dims* dims, int32_t B, const float* o, const void* W_O, float* u,
                                      void* workspace, size_t ws_bytes, void* stream, bool o_prepacked,
                                      char* counters = nullptr) {
  mla_status st = check_query_dims(dims, B, 0);
  if (st != MLA_OK) return st;
  if (!o || !W_O || !u || !workspace) return fail(MLA_ERR_INVALID_ARG, "null pointer among o, W_O, u, workspace");
  if (!aligned16(o) || !aligned16(W_O) || !aligned16(u))
    return fail(MLA_ERR_INVALID_ARG, "o / W_O / u not 16-byte aligned");
  if (((uintptr_t)workspace & 255) != 0) return fail(MLA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  const OutputPlan p = output_plan(*dims, B);
  if (ws_bytes < p.total) return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, p.total);
  const bool f32 = dims->dtype == MLA_FP32;
  const int32_t K = dims->n_h * mla::D_H;
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  const void* X = o;
  if (p.packed) {
    if (!o_prepacked) e = mla::launch_pack(o, K, B, mla::gemm_rows_padded(B), K, true, true, ws + p.off_o, s);
    X = ws + p.off_o;
  }
  mla::GemmArgs g = gemm_args(X, K, B, K, counters ? counters : ws);
  mla::GemmOut out{};
  gemm_segments(g, out, {{W_O, dims->d_model, u, dims->d_model}});
  g.S = p.S;
  g.part = (float*)(ws + p.off_part);
  if (e == hipSuccess) e = mla::launch_gemm(g, out, f32, true, true, s);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "output projection launch: %s", hipGetErrorString(e));
  return ok();
}

extern "C" {

mla_status mla_output_project(const mla_dims* dims, int32_t B, const float* o, const void* W_O, float* u,
                              void* workspace, size_t ws_bytes, void* stream) {
  return output_project_impl(dims, B, o, W_O, u, workspace, ws_bytes, stream, false);
}

mla_status mla_pack_weight(const mla_dims* dims, int32_t rows, int32_t K, const void* W, void* W_packed,
                           void* stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (rows < 16 || rows % 16 != 0 || K < 32 || K % 32 != 0)
    return fail(MLA_ERR_INVALID_ARG, "rows=%d must be a positive multiple of 16 and K=%d of 32", rows, K);
  if ((int64_t)rows * K >= ((int64_t)1 << 40)) return fail(MLA_ERR_INVALID_ARG, "matrix too large");
  if (!W || !W_packed) return fail(MLA_ERR_INVALID_ARG, "W / W_packed is NULL");
  if (!aligned16(W) || !aligned16(W_packed)) return fail(MLA_ERR_INVALID_ARG, "W / W_packed not 16-byte aligned");
  const bool f32 = dims->dtype == MLA_FP32;
  hipError_t e = mla::launch_pack(W, K, rows, rows, K, f32, false, W_packed, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "pack launch: %s", hipGetErrorString(e));
  return ok();
}

// Chunked prefill workspace: the decode's for T queries, then the queries'
// page-table rows [T, max_pages] and lengths [T].
struct PrefillWs {
  size_t q_pt, q_len, total;
};

static PrefillWs prefill_ws_layout(const mla_dims& d, int32_t T, int32_t max_pages, int32_t n_splits) {
  PrefillWs w;
  w.q_pt = mla::decode_ws_layout(T, d.n_h, n_splits, elt_size(&d)).total;
  w.q_len = w.q_pt + mla::align256((size_t)T * max_pages * 4);
  w.total = w.q_len + mla::align256((size_t)T * 4);
  return w;
}

size_t mla_prefill_workspace_size(const mla_dims* dims, int32_t T, int32_t max_pages, int32_t n_splits) {
  if (check_dims(dims) != MLA_OK || T < 1 || T > MAX_ROWS || max_pages < 1) return 0;
  n_splits = resolve_splits(n_splits);
  if (n_splits < 0) return 0;
  return prefill_ws_layout(*dims, T, max_pages, n_splits).total;
}

mla_status mla_prefill(const mla_dims* dims, int32_t T, const void* h, const void* W_DKV, const void* W_KR,
                       const void* q_C, const void* q_R, const int32_t* seq_id, const int32_t* pos, const void* W_UK,
                       const void* W_UV, void* c_KV, void* k_R, int64_t row_stride, int32_t num_pages,
                       const int32_t* page_table, int32_t num_seqs, int32_t max_pages, float* out, float* lse,
                       void* workspace, size_t ws_bytes, int32_t n_splits, void* stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (T < 1 || T > MAX_ROWS) return fail(MLA_ERR_INVALID_ARG, "T=%d out of range [1, 2^20]", T);
  // every check of the decode that follows is made here too, before anything is launched
  if (!h || !W_DKV || !W_KR || !seq_id || !pos || !page_table || !workspace || !q_C || !q_R || !W_UK || !W_UV ||
      !out)
    return fail(MLA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(h) || !aligned16(W_DKV) || !aligned16(W_KR) || !aligned16(q_C) || !aligned16(q_R) ||
      !aligned16(W_UK) || !aligned16(W_UV) || !aligned16(out))
    return fail(MLA_ERR_INVALID_ARG, "h / weights / q_C / q_R / out not 16-byte aligned");
  if (num_seqs < 1 || max_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_seqs and max_pages must be >= 1");
  if (((uintptr_t)workspace & 255) != 0) return fail(MLA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  const int32_t n_req = n_splits;
  n_splits = resolve_splits(n_splits);
  if (n_splits < 0) return fail(MLA_ERR_INVALID_ARG, "n_splits=%d above 2^20", n_req);
  st = check_pool(dims, c_KV, k_R, row_stride, num_pages);
  if (st != MLA_OK) return st;
  if ((int64_t)T * max_pages * dims->page_size >= ((int64_t)1 << 31))
    return fail(MLA_ERR_UNSUPPORTED, "T*max_pages*page_size >= 2^31 tokens");
  const PrefillWs L = prefill_ws_layout(*dims, T, max_pages, n_splits);
  if (ws_bytes < L.total) return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  char* ws = (char*)workspace;
  int32_t* q_pt = (int32_t*)(ws + L.q_pt);
  int32_t* q_len = (int32_t*)(ws + L.q_len);
  hipStream_t s = (hipStream_t)stream;
  // append errors go to flag word 1 (cleared first), which the combine folds into word 0
  hipError_t e = mla::launch_prefill_queries(T, seq_id, pos, page_table, num_seqs, max_pages, dims->page_size, q_pt,
                                             q_len, (int32_t*)ws + 1, s);
  // The append's split path keeps its chunk sums in the decode layout's
  // partials region, which the attention fills only after the append.
  const mla::DecodeWs D = mla::decode_ws_layout(T, dims->n_h, n_splits, (int)elt_size(dims));
  const size_t app_need = mla::append_workspace_bytes(*dims, T);
  char* app_ws = app_need > 0 && D.app_part - D.part_o >= app_need ? ws + D.part_o : nullptr;
  if (e == hipSuccess)
    e = mla::launch_append(*dims, T, h, W_DKV, W_KR, seq_id, pos, page_table, num_seqs, max_pages, c_KV, k_R,
                           row_stride, num_pages, (int32_t*)ws + 1, app_ws, app_ws ? app_need : 0, s);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return decode_impl(dims, T, q_C, q_R, pos, W_UK, W_UV, c_KV, k_R, row_stride, num_pages, q_pt, max_pages, q_len,
                     out, lse, workspace, L.q_pt, n_splits, nullptr, nullptr, stream, true);
}

// Whole-layer decode workspace: the decode step's (first, so that its error
// flags sit at offset 0) | query projection | q_C | q_R | o | output projection.
struct LayerWs {
  size_t q, qc, qr, o, out, total;
};

static LayerWs layer_ws_layout(const mla_dims& d, int32_t B, int32_t d_cq, int32_t n_splits) {
  const size_t elt = elt_size(&d);
  LayerWs w;
  size_t off = mla::decode_ws_layout(B, d.n_h, n_splits, (int)elt, true).total;
  w.q = off;   off += mla::align256(query_plan(d, B, d_cq).total);
  w.qc = off;  off += mla::align256((size_t)B * d.n_h * mla::D_H * elt);
  w.qr = off;  off += mla::align256((size_t)B * d.n_h * mla::D_R * elt);
  w.o = off;   off += mla::align256((size_t)B * d.n_h * mla::D_H * 4);
  w.out = off; off += mla::align256(output_plan(d, B).total);
  w.total = off;
  return w;
}

size_t mla_decode_layer_workspace_size(const mla_dims* dims, int32_t B, int32_t d_cq, int32_t n_splits) {
  if (check_query_dims(dims, B, d_cq) != MLA_OK) return 0;
  n_splits = resolve_splits(n_splits);
  if (n_splits < 0) return 0;
  return layer_ws_layout(*dims, B, d_cq, n_splits).total;
}

mla_status mla_decode_layer(const mla_dims* dims, int32_t B, int32_t d_cq, const void* h, const void* W_DKV,
                            const void* W_KR, const void* W_DQ, const void* W_UQ, const void* W_QR, const void* W_UK,
                            const void* W_UV, const void* W_O, const int32_t* pos_q, void* c_KV, void* k_R,
                            int64_t row_stride, int32_t num_pages, const int32_t* page_table, int32_t max_pages,
                            const int32_t* seq_lens, float* u, float* lse, void* workspace, size_t ws_bytes,
                            int32_t n_splits, const mla_decode_opts* opts, void* stream) {
  // every check of the three parts is made here, before anything is launched
  mla_status st = check_query_dims(dims, B, d_cq);
  if (st != MLA_OK) return st;
  if (!h || !W_DKV || !W_KR || !W_UQ || !W_QR || !W_UK || !W_UV || !W_O || !pos_q || !page_table || !seq_lens ||
      !u || !workspace || (d_cq > 0) != (W_DQ != nullptr))
    return fail(MLA_ERR_INVALID_ARG, "null pointer argument (W_DQ must be given exactly when d_cq > 0)");
  if (!aligned16(h) || !aligned16(W_DKV) || !aligned16(W_KR) || (W_DQ && !aligned16(W_DQ)) || !aligned16(W_UQ) ||
      !aligned16(W_QR) || !aligned16(W_UK) || !aligned16(W_UV) || !aligned16(W_O) || !aligned16(u))
    return fail(MLA_ERR_INVALID_ARG, "h / weights / u not 16-byte aligned");
  if (((uintptr_t)workspace & 255) != 0) return fail(MLA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  st = check_pool(dims, c_KV, k_R, row_stride, num_pages);
  if (st != MLA_OK) return st;
  if (max_pages < 1 || (int64_t)B * max_pages * dims->page_size >= ((int64_t)1 << 31))
    return fail(MLA_ERR_INVALID_ARG, "max_pages=%d out of range", max_pages);
  if (opts && opts->impl != 0 && opts->impl != 1) return fail(MLA_ERR_INVALID_ARG, "opts->impl=%d", opts->impl);
  const int32_t n_req = n_splits;
  n_splits = resolve_splits(n_splits);
  if (n_splits < 0) return fail(MLA_ERR_INVALID_ARG, "n_splits=%d above 2^20", n_req);
  const LayerWs L = layer_ws_layout(*dims, B, d_cq, n_splits);
  if (ws_bytes < L.total) return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  char* ws = (char*)workspace;
  // the projections' split-K counters sit at fixed offsets of the step's
  // layout (the rest of the workspace moves with B)
  const mla::DecodeWs D = mla::decode_ws_layout(B, dims->n_h, n_splits, (int)elt_size(dims), true);
  // bf16 with a low-rank query: q^C = W^UQ c^Q is formed inside the
  // absorption launch from the packed c^Q the first product leaves in the
  // query workspace, so the W^UQ product has no launch of its own
  const QueryPlan qp = query_plan(*dims, B, d_cq);
  const bool fuse = d_cq > 0 && qp.packed && mla::step_prep_supported(*dims, B) &&
                    mla::absorb_fused_supported(*dims, B, d_cq);
  const FusedQuery fq{ws + L.q + qp.off_cq, W_UQ, d_cq};
  st = query_project_impl(dims, B, d_cq, h, W_DQ, W_UQ, W_QR, ws + L.qc, ws + L.qr, ws + L.q, L.qc - L.q, stream,
                          ws + D.q_cnt, fuse);
  // the step's combine also leaves o packed (bf16) where the output
  // projection reads it, which saves that projection's pack launch
  const OutputPlan op = output_plan(*dims, B);
  const StepAppendIn in{h, W_DKV, W_KR, op.packed ? ws + L.out + op.off_o : nullptr};
  if (st == MLA_OK)
    st = decode_impl(dims, B, ws + L.qc, ws + L.qr, pos_q, W_UK, W_UV, c_KV, k_R, row_stride, num_pages, page_table,
                     max_pages, seq_lens, (float*)(ws + L.o), lse, workspace, L.q, n_splits, opts, &in, stream, false,
                     nullptr, fuse ? &fq : nullptr);
  if (st == MLA_OK)
    st = output_project_impl(dims, B, (const float*)(ws + L.o), W_O, u, ws + L.out, L.total - L.out, stream,
                             op.packed, ws + D.o_cnt);
  return st;
}

// ---------------------------------------------------------------- sparse top-k decode
namespace {

mla_status check_indexer(int32_t H_I, int32_t d_I, int32_t top_k, const void* q_I, const float* w_I, const void* k_I,
                         int64_t idx_row_stride, int32_t page_size) {
  if (d_I != 128) return fail(MLA_ERR_UNSUPPORTED, "d_I=%d: the indexer kernel is built for 128", d_I);
  if (H_I != 16 && H_I != 32 && H_I != 64) return fail(MLA_ERR_UNSUPPORTED, "H_I=%d not in {16, 32, 64}", H_I);
  if (top_k < 1) return fail(MLA_ERR_INVALID_ARG, "top_k=%d must be >= 1", top_k);
  if (!q_I || !w_I || !k_I) return fail(MLA_ERR_INVALID_ARG, "q_I / w_I / k_I is NULL");
  if (!aligned16(q_I) || !aligned16(k_I) || ((uintptr_t)w_I & 3) != 0)
    return fail(MLA_ERR_INVALID_ARG, "q_I / k_I not 16-byte aligned or w_I not 4-byte aligned");
  if (idx_row_stride < d_I || idx_row_stride > MAX_ROW_STRIDE || idx_row_stride % 8 != 0)
    return fail(MLA_ERR_INVALID_ARG, "idx_row_stride=%lld must be in [d_I, 2^24] and a multiple of 8",
                (long long)idx_row_stride);
  if (page_size < 16 || page_size % 16 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "page_size=%d: the indexer needs a multiple of 16", page_size);
  return MLA_OK;
}

int32_t sparse_default_splits(int32_t B, int32_t top_k) {
  const int64_t want = ((int64_t)B * top_k + 127) / 128;   // about four 32-row tiles per split
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>(want, default_splits()));
}

}  // namespace

size_t mla_indexer_select_workspace_size(int32_t B, int32_t max_pages, int32_t page_size, int32_t top_k) {
  if (B < 1 || B > MAX_ROWS || max_pages < 1 || page_size < 1 || top_k < 1) return 0;
  if ((int64_t)B * max_pages * page_size >= ((int64_t)1 << 31)) return 0;
  return mla::select_ws_layout(B, max_pages * page_size, top_k, false).total;
}

mla_status mla_indexer_select(int32_t B, int32_t H_I, int32_t d_I, int32_t top_k, const void* q_I, const float* w_I,
                              const void* k_I, int64_t idx_row_stride, int32_t num_pages, int32_t page_size,
                              const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens, float* scores,
                              int32_t* sel_tok, int32_t* sel_row, int32_t* err_flags, void* workspace,
                              size_t ws_bytes, void* stream) {
  if (B < 1 || B > MAX_ROWS) return fail(MLA_ERR_INVALID_ARG, "B=%d out of range [1, 2^20]", B);
  mla_status st = check_indexer(H_I, d_I, top_k, q_I, w_I, k_I, idx_row_stride, page_size);
  if (st != MLA_OK) return st;
  if (!page_table || !seq_lens || !scores || !sel_tok || !sel_row || !err_flags || !workspace)
    return fail(MLA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(scores)) return fail(MLA_ERR_INVALID_ARG, "scores not 16-byte aligned");
  if (((uintptr_t)workspace & 255) != 0) return fail(MLA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  if (num_pages < 1 || (int64_t)num_pages * page_size >= ((int64_t)1 << 31))
    return fail(MLA_ERR_INVALID_ARG, "num_pages=%d out of range", num_pages);
  if (max_pages < 1 || (int64_t)B * max_pages * page_size >= ((int64_t)1 << 31))
    return fail(MLA_ERR_INVALID_ARG, "max_pages=%d out of range", max_pages);
  const mla::SelectWs L = mla::select_ws_layout(B, max_pages * page_size, top_k, false);
  if (ws_bytes < L.total) return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  const hipError_t e = mla::launch_indexer_select(B, H_I, q_I, w_I, k_I, idx_row_stride, num_pages, page_table,
                                                  max_pages, page_size, seq_lens, top_k, (char*)workspace, L, scores,
                                                  sel_tok, sel_row, err_flags, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "indexer / selection launch: %s", hipGetErrorString(e));
  return ok();
}

size_t mla_sparse_decode_workspace_size(const mla_dims* dims, int32_t B, int32_t max_pages, int32_t top_k,
                                        int32_t n_splits) {
  if (check_dims(dims) != MLA_OK || B < 1 || B > MAX_ROWS || max_pages < 1 || top_k < 1) return 0;
  if ((int64_t)B * max_pages * dims->page_size >= ((int64_t)1 << 31)) return 0;
  if (n_splits > MAX_SPLITS) return 0;
  if (n_splits <= 0) n_splits = sparse_default_splits(B, top_k);
  const mla::DecodeWs D = mla::decode_ws_layout(B, dims->n_h, n_splits, elt_size(dims));
  return D.total + mla::select_ws_layout(B, max_pages * dims->page_size, top_k, true).total;
}

mla_status mla_sparse_decode(const mla_dims* dims, int32_t B, const void* q_C, const void* q_R, const int32_t* pos_q,
                             const void* W_UK, const void* W_UV, const void* c_KV, const void* k_R,
                             int64_t row_stride, int32_t num_pages, const int32_t* page_table, int32_t max_pages,
                             const int32_t* seq_lens, int32_t H_I, int32_t d_I, int32_t top_k, const void* q_I,
                             const float* w_I, const void* k_I, int64_t idx_row_stride, float* out, float* lse,
                             int32_t* sel_tok, void* workspace, size_t ws_bytes, int32_t n_splits,
                             const mla_decode_opts* opts, void* stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (dims->dtype != MLA_BF16 || (dims->n_h != 32 && dims->n_h != 64 && dims->n_h != 128) || dims->page_size < 32 ||
      dims->page_size % 32 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "sparse decode needs bf16, n_h in {32, 64, 128} and page_size a multiple of 32");
  if (B < 1 || B > MAX_ROWS) return fail(MLA_ERR_INVALID_ARG, "B=%d out of range [1, 2^20]", B);
  st = check_indexer(H_I, d_I, top_k, q_I, w_I, k_I, idx_row_stride, dims->page_size);
  if (st != MLA_OK) return st;
  if (!q_C || !q_R || !pos_q || !W_UK || !W_UV || !page_table || !seq_lens || !out || !workspace)
    return fail(MLA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(q_C) || !aligned16(q_R) || !aligned16(W_UK) || !aligned16(W_UV) || !aligned16(out))
    return fail(MLA_ERR_INVALID_ARG, "q_C / q_R / W_UK / W_UV / out not 16-byte aligned");
  if (((uintptr_t)workspace & 255) != 0) return fail(MLA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  st = check_pool(dims, c_KV, k_R, row_stride, num_pages);
  if (st != MLA_OK) return st;
  if (max_pages < 1 || (int64_t)B * max_pages * dims->page_size >= ((int64_t)1 << 31))
    return fail(MLA_ERR_INVALID_ARG, "max_pages=%d out of range", max_pages);
  if ((int64_t)B * top_k >= ((int64_t)1 << 31)) return fail(MLA_ERR_UNSUPPORTED, "B*top_k >= 2^31");
  if (opts && opts->impl != 0) return fail(MLA_ERR_INVALID_ARG, "opts->impl=%d (sparse decode has one kernel)", opts->impl);
  if (n_splits > MAX_SPLITS) return fail(MLA_ERR_INVALID_ARG, "n_splits=%d above 2^20", n_splits);
  if (n_splits <= 0) n_splits = sparse_default_splits(B, top_k);
  const mla::DecodeWs D = mla::decode_ws_layout(B, dims->n_h, n_splits, elt_size(dims));
  const mla::SelectWs S = mla::select_ws_layout(B, max_pages * dims->page_size, top_k, true);
  if (ws_bytes < D.total + S.total)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, D.total + S.total);

  char* ws = (char*)workspace;
  char* sw = ws + D.total;
  int32_t* flags = (int32_t*)(ws + D.flags);
  int32_t* sel_row = (int32_t*)(sw + S.sel_row);
  hipStream_t s = (hipStream_t)stream;
  mla::PlanArgs pa;
  pa.seq_lens = seq_lens;
  pa.B = B;
  pa.max_tokens = max_pages * dims->page_size;
  pa.G = n_splits;
  pa.prefix = (int32_t*)(ws + D.prefix);
  pa.split_rec = (int32_t*)(ws + D.splits);
  pa.flags = flags;
  pa.page_table = page_table;
  pa.max_pages = max_pages;
  pa.page_size = dims->page_size;
  pa.keep = top_k;
  pa.gather = true;
  // query absorption and the plan over the kept counts (it clears the flags),
  // then the indexer and the selection, the gather attention and the combine
  hipError_t e = mla::launch_absorb(*dims, B, q_C, q_R, pos_q, W_UK, ws + D.qabs, pa, s);
  if (e == hipSuccess)
    e = mla::launch_indexer_select(B, H_I, q_I, w_I, k_I, idx_row_stride, num_pages, page_table, max_pages,
                                   dims->page_size, seq_lens, top_k, sw, S, (float*)(sw + S.scores),
                                   sel_tok ? sel_tok : (int32_t*)(sw + S.sel_tok), sel_row, flags, s);
  if (e == hipSuccess && opts && opts->ev_start) e = hipEventRecord((hipEvent_t)opts->ev_start, s);
  if (e == hipSuccess)
    e = mla::launch_decode_mfma(*dims, B, ws + D.qabs, c_KV, k_R, row_stride, num_pages, page_table, max_pages,
                                pa.prefix, pa.split_rec, n_splits, (float*)(ws + D.part_ml), ws + D.part_o, flags, s,
                                sel_row, top_k);
  if (e == hipSuccess && opts && opts->ev_stop) e = hipEventRecord((hipEvent_t)opts->ev_stop, s);
  if (e == hipSuccess)
    e = mla::launch_combine(*dims, B, pa.prefix, n_splits, (float*)(ws + D.part_ml), ws + D.part_o, W_UV, out, lse,
                            nullptr, nullptr, s);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "sparse decode launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free decode step
namespace {

// Scratch of mla_decode_step_noalloc: one decode-step workspace of at most
// NOALLOC_SCRATCH_BYTES in a file-scope device array (each GPU the library
// runs on holds its own copy until the process ends).  In host code the name
// `scratch` is only a host-side stand-in: every host use of the array goes
// through the device address hipGetSymbolAddress returned for the current
// device, kept in g_scratch.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)80 << 20;
static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
char* g_scratch[NOALLOC_MAX_DEVICES] = {};

__global__ void __launch_bounds__(256) zero_words_kernel(int32_t* p, int32_t n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// The current device's scratch.  On the first call on a device its address is
// looked up (with that device current) and the words that must start at zero
// -- the flag area and the split-K tile counters, which every completed step
// leaves at zero again -- are cleared by a fill kernel on stream s.
mla_status noalloc_scratch(hipStream_t s, char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
    return fail(MLA_ERR_UNSUPPORTED, "device %d: the allocation-free step supports devices 0..%d", dev,
                NOALLOC_MAX_DEVICES - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    // flags and counters precede everything that depends on the batch size
    const int32_t words = (int32_t)(mla::decode_ws_layout(1, 1, 1, 2, true).prefix / 4);
    zero_words_kernel<<<dim3((words + 255) / 256), 256, 0, s>>>((int32_t*)p, words);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "scratch clear launch: %s", hipGetErrorString(e));
    g_scratch[dev] = (char*)p;
  }
  *out = g_scratch[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_decode_step_noalloc(const mla_dims* dims, int32_t B, const void* h_new, const void* W_DKV,
                                   const void* W_KR, const void* q_C, const void* q_R, const int32_t* pos_q,
                                   const void* W_UK, const void* W_UV, void* c_KV, void* k_R, int64_t row_stride,
                                   int32_t num_pages, const int32_t* page_table, int32_t max_pages,
                                   const int32_t* seq_lens, float* out, float* lse, int32_t* err_flags,
                                   void* stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (B < 1 || B > MAX_ROWS) return fail(MLA_ERR_INVALID_ARG, "B=%d out of range [1, 2^20]", B);
  const int32_t n_splits = default_splits();
  const size_t need = mla::decode_ws_layout(B, dims->n_h, n_splits, elt_size(dims), true).total;
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(MLA_ERR_WORKSPACE,
                "B=%d, n_h=%d needs %zu bytes of scratch; the allocation-free step has %zu (use mla_decode_step)", B,
                dims->n_h, need, NOALLOC_SCRATCH_BYTES);
  char* ws = nullptr;
  st = noalloc_scratch((hipStream_t)stream, &ws);
  if (st != MLA_OK) return st;
  const StepAppendIn in{h_new, W_DKV, W_KR, nullptr};
  return decode_impl(dims, B, q_C, q_R, pos_q, W_UK, W_UV, c_KV, k_R, row_stride, num_pages, page_table, max_pages,
                     seq_lens, out, lse, ws, NOALLOC_SCRATCH_BYTES, n_splits, nullptr, &in, stream, false,
                     err_flags);
}

mla_status mla_read_error_flags(void* workspace_or_flag, int32_t* flags, void* stream) {
  if (!workspace_or_flag || !flags) return fail(MLA_ERR_INVALID_ARG, "null pointer");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(flags, workspace_or_flag, sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess) {
    const int32_t zero = 0;
    e = hipMemcpy(workspace_or_flag, &zero, sizeof(int32_t), hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "read flags: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
