// C ABI entry points of libmla.so: argument checks, workspace layout,
// kernel selection and launch order.  No device memory is allocated here.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "append_splitk.h"

namespace {

thread_local std::string g_err;

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
  if (!(d->softmax_scale > 0.f) || !(d->rope_base > 0.f))
    return fail(MLA_ERR_INVALID_ARG, "softmax_scale and rope_base must be positive");
  return MLA_OK;
}

mla_status check_pool(const mla_dims* d, const void* c_KV, const void* k_R, int64_t row_stride, int32_t num_pages) {
  if (!c_KV || !k_R) return fail(MLA_ERR_INVALID_ARG, "c_KV / k_R is NULL");
  if (!aligned16(c_KV) || !aligned16(k_R)) return fail(MLA_ERR_INVALID_ARG, "c_KV / k_R not 16-byte aligned");
  if (row_stride < mla::D_C || (row_stride * elt_size(d)) % 16 != 0)
    return fail(MLA_ERR_INVALID_ARG, "row_stride=%lld must be >= 512 and a multiple of 16 bytes",
                (long long)row_stride);
  if (num_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_pages=%d must be >= 1", num_pages);
  if ((int64_t)num_pages * d->page_size >= ((int64_t)1 << 31))
    return fail(MLA_ERR_UNSUPPORTED, "pool holds more than 2^31 rows");
  return MLA_OK;
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
  if (T < 0) return fail(MLA_ERR_INVALID_ARG, "T=%d < 0", T);
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
  if (check_dims(dims) != MLA_OK || T < 1) return 0;
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
  if (check_dims(dims) != MLA_OK || B < 1) return 0;
  if (n_splits <= 0) n_splits = default_splits();
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
};

static mla_status decode_impl(const mla_dims* dims, int32_t B, const void* q_C, const void* q_R, const int32_t* pos_q,
                              const void* W_UK, const void* W_UV, const void* c_KV, const void* k_R,
                              int64_t row_stride, int32_t num_pages, const int32_t* page_table, int32_t max_pages,
                              const int32_t* seq_lens, float* out, float* lse, void* workspace, size_t ws_bytes,
                              int32_t n_splits, const mla_decode_opts* opts, const StepAppendIn* step,
                              void* stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (B < 1) return fail(MLA_ERR_INVALID_ARG, "B=%d must be >= 1", B);
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
  if (n_splits <= 0) n_splits = default_splits();
  if (n_splits > (1 << 20)) return fail(MLA_ERR_INVALID_ARG, "n_splits=%d too large", n_splits);
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
  hipError_t e = hipSuccess;
  if (step && mla::step_prep_supported(*dims)) {
    // append (split-K, finished in the same launch), absorption and plan in one launch
    const mla::AppendDst dst{nullptr, pos_q, page_table, B, max_pages, dims->page_size, num_pages,
                             (mla::bf16*)c_KV, (mla::bf16*)k_R, row_stride, mla::rope_table(dims->rope_base),
                             flags + 1};
    e = mla::launch_step_prep(*dims, B, step->h_new, step->W_DKV, step->W_KR, q_C, q_R, pos_q, W_UK, qabs, pa,
                              (float*)(ws + L.app_part), (int32_t*)(ws + L.app_cnt), dst, s);
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
    e = mla::launch_combine(*dims, B, prefix, n_splits, part_ml, part_o, W_UV, out, lse, step ? flags : nullptr, s);
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
  if (check_dims(dims) != MLA_OK || B < 1) return 0;
  if (n_splits <= 0) n_splits = default_splits();
  return mla::decode_ws_layout(B, dims->n_h, n_splits, elt_size(dims), true).total;
}

mla_status mla_decode_step(const mla_dims* dims, int32_t B, const void* h_new, const void* W_DKV, const void* W_KR,
                           const void* q_C, const void* q_R, const int32_t* pos_q, const void* W_UK,
                           const void* W_UV, void* c_KV, void* k_R, int64_t row_stride, int32_t num_pages,
                           const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens, float* out,
                           float* lse, void* workspace, size_t ws_bytes, int32_t n_splits,
                           const mla_decode_opts* opts, void* stream) {
  const StepAppendIn in{h_new, W_DKV, W_KR};
  return decode_impl(dims, B, q_C, q_R, pos_q, W_UK, W_UV, c_KV, k_R, row_stride, num_pages, page_table, max_pages,
                     seq_lens, out, lse, workspace, ws_bytes, n_splits, opts, &in, stream);
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
