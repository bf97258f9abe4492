/*
 * Host-side misuse driver for libmla.so, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code (test_host_sanitizers.py builds
 * it; no GPU is needed or used).
 *
 * Every entry point of include/mla.h is called with arguments that are valid
 * except for one, and with the extreme values each integer argument can take.
 * Device pointers are fake (aligned addresses that nothing on the host may
 * read), so any host dereference of one, any out-of-bounds host access and
 * any signed overflow or other undefined behaviour in the argument checks,
 * the workspace layouts or the launch set-up stops the run with a sanitizer
 * report.  A call whose arguments all pass the checks reaches the HIP launch,
 * which fails without a GPU: MLA_ERR_HIP is the expected status there.
 *
 * The workspace-size functions are checked for wrap-around: over a ladder of
 * growing arguments the size never decreases until it drops to 0 (arguments
 * no call accepts), and stays 0 after that.
 *
 * Exit status: 0 when every case gave its expected status.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mla.h"

static int g_cases = 0, g_fail = 0;

/* fake device addresses: 256-byte aligned, far apart, never dereferenced */
#define DP(i) ((void*)(uintptr_t)(0x7f0000000000ull + (uint64_t)(i) * 0x10000000ull))
#define IP(i) ((int32_t*)DP(i))
#define FP(i) ((float*)DP(i))
#define OFF(p, n) ((void*)((char*)(p) + (n)))

static void expect(const char* what, mla_status got, mla_status want) {
  ++g_cases;
  const char* msg = mla_last_error();
  if (got != want) {
    ++g_fail;
    printf("FAIL %s: status %d, expected %d (%s)\n", what, (int)got, (int)want, msg ? msg : "(null)");
  } else if (want != MLA_OK && (!msg || !msg[0])) {
    ++g_fail;
    printf("FAIL %s: status %d without a message\n", what, (int)got);
  }
}

static void expect_true(const char* what, int ok) {
  ++g_cases;
  if (!ok) {
    ++g_fail;
    printf("FAIL %s\n", what);
  }
}

static mla_dims base_dims(void) {
  mla_dims d;
  memset(&d, 0, sizeof d);
  d.n_h = 128;
  d.d_h = 128;
  d.d_c = 512;
  d.d_hR = 64;
  d.d_model = 5120;
  d.page_size = 64;
  d.softmax_scale = 0.0721687836f;
  d.rope_base = 10000.f;
  d.dtype = MLA_BF16;
  return d;
}

/* dims variants every dims-taking entry point must reject (expected status) */
typedef struct {
  const char* name;
  mla_dims d;
  mla_status st;
} BadDims;

static int bad_dims(BadDims* out) {
  int n = 0;
  mla_dims d;
#define BAD(label, field, value, status) \
  d = base_dims();                       \
  d.field = value;                       \
  out[n].name = label;                   \
  out[n].d = d;                          \
  out[n].st = status;                    \
  ++n;
  BAD("dtype=7", dtype, 7, MLA_ERR_INVALID_ARG);
  BAD("dtype=-1", dtype, -1, MLA_ERR_INVALID_ARG);
  BAD("d_c=256", d_c, 256, MLA_ERR_UNSUPPORTED);
  BAD("d_hR=32", d_hR, 32, MLA_ERR_UNSUPPORTED);
  BAD("d_h=64", d_h, 64, MLA_ERR_UNSUPPORTED);
  BAD("n_h=0", n_h, 0, MLA_ERR_INVALID_ARG);
  BAD("n_h=INT32_MAX", n_h, INT32_MAX, MLA_ERR_INVALID_ARG);
  BAD("n_h=INT32_MIN", n_h, INT32_MIN, MLA_ERR_INVALID_ARG);
  BAD("d_model=100", d_model, 100, MLA_ERR_UNSUPPORTED);
  BAD("d_model=-64", d_model, -64, MLA_ERR_UNSUPPORTED);
  BAD("page_size=0", page_size, 0, MLA_ERR_INVALID_ARG);
  BAD("page_size=INT32_MIN", page_size, INT32_MIN, MLA_ERR_INVALID_ARG);
  BAD("softmax_scale=NaN", softmax_scale, NAN, MLA_ERR_INVALID_ARG);
  BAD("softmax_scale=-1", softmax_scale, -1.f, MLA_ERR_INVALID_ARG);
  BAD("softmax_scale=-NaN", softmax_scale, -NAN, MLA_ERR_INVALID_ARG);
  BAD("softmax_scale=inf", softmax_scale, INFINITY, MLA_ERR_INVALID_ARG);
  BAD("softmax_scale=-0", softmax_scale, -0.f, MLA_ERR_INVALID_ARG);
  BAD("rope_base=0", rope_base, 0.f, MLA_ERR_INVALID_ARG);
  BAD("rope_base=NaN", rope_base, NAN, MLA_ERR_INVALID_ARG);
#undef BAD
  return n;
}

/* ------------------------------------------------------------------ decode */
typedef struct {
  mla_dims d;
  int has_dims;
  int32_t B;
  const void *q_C, *q_R, *W_UK, *W_UV, *c_KV, *k_R;
  const int32_t *pos_q, *page_table, *seq_lens;
  int64_t row_stride;
  int32_t num_pages, max_pages, n_splits;
  float *out, *lse;
  void* ws;
  size_t ws_bytes;
  mla_decode_opts opts;
  const mla_decode_opts* optp;
  /* decode step: the append half */
  const void *h_new, *W_DKV, *W_KR;
} DecodeArgs;

static DecodeArgs decode_args(void) {
  DecodeArgs a;
  memset(&a, 0, sizeof a);
  a.d = base_dims();
  a.has_dims = 1;
  a.B = 4;
  a.q_C = DP(1);
  a.q_R = DP(2);
  a.pos_q = IP(3);
  a.W_UK = DP(4);
  a.W_UV = DP(5);
  a.c_KV = DP(6);
  a.k_R = OFF(DP(6), 1024);
  a.row_stride = 576;
  a.num_pages = 1000;
  a.page_table = IP(7);
  a.max_pages = 64;
  a.seq_lens = IP(8);
  a.out = FP(9);
  a.lse = FP(10);
  a.ws = DP(11);
  a.ws_bytes = SIZE_MAX;
  a.n_splits = 16;
  a.optp = NULL;
  a.h_new = DP(12);
  a.W_DKV = DP(13);
  a.W_KR = DP(14);
  return a;
}

static mla_status run_decode(DecodeArgs* a) {
  return mla_decode_ex(a->has_dims ? &a->d : NULL, a->B, a->q_C, a->q_R, a->pos_q, a->W_UK, a->W_UV, a->c_KV, a->k_R, a->row_stride,
                       a->num_pages, a->page_table, a->max_pages, a->seq_lens, a->out, a->lse, a->ws, a->ws_bytes,
                       a->n_splits, a->optp, NULL);
}

static mla_status run_decode_plain(DecodeArgs* a) {
  return mla_decode(a->has_dims ? &a->d : NULL, a->B, a->q_C, a->q_R, a->pos_q, a->W_UK, a->W_UV, a->c_KV, a->k_R,
                    a->row_stride, a->num_pages, a->page_table, a->max_pages, a->seq_lens, a->out, a->lse, a->ws,
                    a->ws_bytes, a->n_splits, NULL);
}

static mla_status run_step(DecodeArgs* a) {
  return mla_decode_step(a->has_dims ? &a->d : NULL, a->B, a->h_new, a->W_DKV, a->W_KR, a->q_C, a->q_R, a->pos_q,
                         a->W_UK, a->W_UV, (void*)a->c_KV, (void*)a->k_R, a->row_stride, a->num_pages,
                         a->page_table, a->max_pages, a->seq_lens, a->out, a->lse, a->ws, a->ws_bytes, a->n_splits,
                         a->optp, NULL);
}

static mla_status run_step_noalloc(DecodeArgs* a) {
  return mla_decode_step_noalloc(a->has_dims ? &a->d : NULL, a->B, a->h_new, a->W_DKV, a->W_KR, a->q_C, a->q_R,
                                 a->pos_q, a->W_UK, a->W_UV, (void*)a->c_KV, (void*)a->k_R, a->row_stride,
                                 a->num_pages, a->page_table, a->max_pages, a->seq_lens, a->out, a->lse, NULL,
                                 NULL);
}

typedef mla_status (*DecodeFn)(DecodeArgs*);

static void decode_family(const char* fam, DecodeFn fn, int is_step, int takes_ws, int takes_opts) {
  char what[256];
  DecodeArgs a;
#define CASE(label, mutation, want)                     \
  do {                                                  \
    a = decode_args();                                  \
    mutation;                                           \
    snprintf(what, sizeof what, "%s %s", fam, label);   \
    expect(what, fn(&a), want);                         \
  } while (0)

  CASE("valid", (void)0, MLA_ERR_HIP);
  CASE("dims NULL", a.has_dims = 0, MLA_ERR_INVALID_ARG);
  {
    BadDims bd[32];
    const int n = bad_dims(bd);
    for (int i = 0; i < n; ++i) CASE(bd[i].name, a.d = bd[i].d, bd[i].st);
  }
  CASE("B=0", a.B = 0, MLA_ERR_INVALID_ARG);
  CASE("B=-1", a.B = -1, MLA_ERR_INVALID_ARG);
  CASE("B=INT32_MIN", a.B = INT32_MIN, MLA_ERR_INVALID_ARG);
  CASE("q_C NULL", a.q_C = NULL, MLA_ERR_INVALID_ARG);
  CASE("q_R NULL", a.q_R = NULL, MLA_ERR_INVALID_ARG);
  CASE("pos_q NULL", a.pos_q = NULL, MLA_ERR_INVALID_ARG);
  CASE("W_UK NULL", a.W_UK = NULL, MLA_ERR_INVALID_ARG);
  CASE("W_UV NULL", a.W_UV = NULL, MLA_ERR_INVALID_ARG);
  CASE("c_KV NULL", a.c_KV = NULL, MLA_ERR_INVALID_ARG);
  CASE("k_R NULL", a.k_R = NULL, MLA_ERR_INVALID_ARG);
  CASE("page_table NULL", a.page_table = NULL, MLA_ERR_INVALID_ARG);
  CASE("seq_lens NULL", a.seq_lens = NULL, MLA_ERR_INVALID_ARG);
  CASE("out NULL", a.out = NULL, MLA_ERR_INVALID_ARG);
  CASE("q_C +8", a.q_C = OFF(a.q_C, 8), MLA_ERR_INVALID_ARG);
  CASE("W_UV +2", a.W_UV = OFF(a.W_UV, 2), MLA_ERR_INVALID_ARG);
  CASE("out +4", a.out = (float*)OFF(a.out, 4), MLA_ERR_INVALID_ARG);
  CASE("c_KV +8", a.c_KV = OFF(a.c_KV, 8), MLA_ERR_INVALID_ARG);
  CASE("row_stride=500", a.row_stride = 500, MLA_ERR_INVALID_ARG);
  CASE("row_stride=580", a.row_stride = 580, MLA_ERR_INVALID_ARG);
  CASE("row_stride=-576", a.row_stride = -576, MLA_ERR_INVALID_ARG);
  CASE("row_stride=INT64_MAX", a.row_stride = INT64_MAX, MLA_ERR_INVALID_ARG);
  CASE("row_stride=INT64_MIN", a.row_stride = INT64_MIN, MLA_ERR_INVALID_ARG);
  CASE("row_stride=INT64_MAX-7", a.row_stride = INT64_MAX - 7, MLA_ERR_INVALID_ARG);
  CASE("num_pages=0", a.num_pages = 0, MLA_ERR_INVALID_ARG);
  CASE("num_pages=INT32_MAX", a.num_pages = INT32_MAX, MLA_ERR_UNSUPPORTED);
  CASE("max_pages=0", a.max_pages = 0, MLA_ERR_INVALID_ARG);
  CASE("max_pages=INT32_MAX", a.max_pages = INT32_MAX, MLA_ERR_INVALID_ARG);
  CASE("B*max_pages*page_size=2^31", (a.B = 1 << 15, a.max_pages = 1 << 10), MLA_ERR_UNSUPPORTED);
  CASE("B=INT32_MAX", a.B = INT32_MAX, MLA_ERR_INVALID_ARG);
  CASE("B=2^20+1", a.B = (1 << 20) + 1, MLA_ERR_INVALID_ARG);
  CASE("n_splits=INT32_MAX", a.n_splits = INT32_MAX, MLA_ERR_INVALID_ARG);
  CASE("n_splits=2^20+1", a.n_splits = (1 << 20) + 1, MLA_ERR_INVALID_ARG);
  CASE("n_splits=INT32_MIN (default)", a.n_splits = INT32_MIN, MLA_ERR_HIP);
  /* the largest shapes the checks accept reach the launch */
  CASE("B*max_pages*page_size=2^31-64", (a.B = 1, a.max_pages = (1 << 25) - 1), MLA_ERR_HIP);
  CASE("B=2^20, max_pages=1", (a.B = 1 << 20, a.max_pages = 1), MLA_ERR_HIP);
  CASE("n_splits=2^20", a.n_splits = 1 << 20, MLA_ERR_HIP);
  CASE("num_pages*page_size=2^31-64", a.num_pages = (1 << 25) - 1, MLA_ERR_HIP);
  CASE("page_size=1", (a.d.page_size = 1, a.max_pages = 4096), MLA_ERR_HIP);
  CASE("page_size=2^30", (a.d.page_size = 1 << 30, a.max_pages = 1, a.B = 1, a.num_pages = 1), MLA_ERR_HIP);
  CASE("fp32", (a.d.dtype = MLA_FP32, a.row_stride = 576), MLA_ERR_HIP);
  CASE("n_h=1", a.d.n_h = 1, MLA_ERR_HIP);
  CASE("n_h=1024", a.d.n_h = 1024, MLA_ERR_HIP);
  if (takes_ws) {
    CASE("workspace NULL", a.ws = NULL, MLA_ERR_INVALID_ARG);
    CASE("workspace +16", a.ws = OFF(a.ws, 16), MLA_ERR_INVALID_ARG);
    CASE("ws_bytes=0", a.ws_bytes = 0, MLA_ERR_WORKSPACE);
    CASE("ws_bytes=100", a.ws_bytes = 100, MLA_ERR_WORKSPACE);
    {
      a = decode_args();
      const size_t need = is_step ? mla_decode_step_workspace_size(&a.d, a.B, a.n_splits)
                                  : mla_decode_workspace_size(&a.d, a.B, a.n_splits);
      snprintf(what, sizeof what, "%s workspace size > 0", fam);
      expect_true(what, need > 0);
      CASE("ws_bytes=need-1", a.ws_bytes = need - 1, MLA_ERR_WORKSPACE);
      CASE("ws_bytes=need", a.ws_bytes = need, MLA_ERR_HIP);
    }
  }
  if (takes_opts) {
    CASE("opts impl=2", (a.opts.impl = 2, a.optp = &a.opts), MLA_ERR_INVALID_ARG);
    CASE("opts impl=-1", (a.opts.impl = -1, a.optp = &a.opts), MLA_ERR_INVALID_ARG);
    CASE("opts impl=1", (a.opts.impl = 1, a.optp = &a.opts), MLA_ERR_HIP);
  }
  if (is_step) {
    CASE("h_new NULL", a.h_new = NULL, MLA_ERR_INVALID_ARG);
    CASE("W_DKV NULL", a.W_DKV = NULL, MLA_ERR_INVALID_ARG);
    CASE("W_KR +8", a.W_KR = OFF(a.W_KR, 8), MLA_ERR_INVALID_ARG);
  }
#undef CASE
}

static void noalloc_cases(void) {
  char what[256];
  DecodeArgs a;
#define CASE(label, mutation, want)                           \
  do {                                                        \
    a = decode_args();                                        \
    mutation;                                                 \
    snprintf(what, sizeof what, "decode_step_noalloc %s", label); \
    expect(what, run_step_noalloc(&a), want);                 \
  } while (0)
  CASE("valid", (void)0, MLA_ERR_HIP);
  CASE("dims NULL", a.has_dims = 0, MLA_ERR_INVALID_ARG);
  CASE("d_c=256", a.d.d_c = 256, MLA_ERR_UNSUPPORTED);
  CASE("B=0", a.B = 0, MLA_ERR_INVALID_ARG);
  CASE("B=INT32_MIN", a.B = INT32_MIN, MLA_ERR_INVALID_ARG);
  CASE("B=4096 (beyond the scratch)", a.B = 4096, MLA_ERR_WORKSPACE);
  CASE("B=INT32_MAX", a.B = INT32_MAX, MLA_ERR_INVALID_ARG);
  CASE("n_h=1024, B=2048", (a.d.n_h = 1024, a.B = 2048), MLA_ERR_WORKSPACE);
#undef CASE
}

/* ------------------------------------------------------------------ append */
typedef struct {
  mla_dims d;
  int has_dims;
  int32_t T, num_seqs, max_pages, num_pages;
  const void *h, *W_DKV, *W_KR;
  const int32_t *seq_id, *pos, *page_table;
  void *c_KV, *k_R, *ws;
  int64_t row_stride;
  size_t ws_bytes;
} AppendArgs;

static AppendArgs append_args(void) {
  AppendArgs a;
  memset(&a, 0, sizeof a);
  a.d = base_dims();
  a.has_dims = 1;
  a.T = 8;
  a.h = DP(1);
  a.W_DKV = DP(2);
  a.W_KR = DP(3);
  a.seq_id = IP(4);
  a.pos = IP(5);
  a.page_table = IP(6);
  a.num_seqs = 8;
  a.max_pages = 64;
  a.c_KV = DP(7);
  a.k_R = OFF(DP(7), 1024);
  a.row_stride = 576;
  a.num_pages = 1000;
  a.ws = DP(8);
  a.ws_bytes = SIZE_MAX;
  return a;
}

static void append_cases(int with_ws) {
  char what[256];
  AppendArgs a;
  const char* fam = with_ws ? "cache_append_ws" : "cache_append";
#define CASE(label, mutation, want)                                                                              \
  do {                                                                                                           \
    a = append_args();                                                                                           \
    mutation;                                                                                                    \
    snprintf(what, sizeof what, "%s %s", fam, label);                                                            \
    const mla_dims* dp = a.has_dims ? &a.d : NULL;                                                               \
    mla_status st = with_ws                                                                                      \
        ? mla_cache_append_ws(dp, a.T, a.h, a.W_DKV, a.W_KR, a.seq_id, a.pos, a.page_table, a.num_seqs,          \
                              a.max_pages, a.c_KV, a.k_R, a.row_stride, a.num_pages, NULL, a.ws, a.ws_bytes, NULL) \
        : mla_cache_append(dp, a.T, a.h, a.W_DKV, a.W_KR, a.seq_id, a.pos, a.page_table, a.num_seqs,              \
                           a.max_pages, a.c_KV, a.k_R, a.row_stride, a.num_pages, NULL, NULL);                   \
    expect(what, st, want);                                                                                      \
  } while (0)
  CASE("valid", (void)0, MLA_ERR_HIP);
  CASE("dims NULL", a.has_dims = 0, MLA_ERR_INVALID_ARG);
  {
    BadDims bd[32];
    const int n = bad_dims(bd);
    for (int i = 0; i < n; ++i) CASE(bd[i].name, a.d = bd[i].d, bd[i].st);
  }
  CASE("T=0", a.T = 0, MLA_OK);
  CASE("T=-1", a.T = -1, MLA_ERR_INVALID_ARG);
  CASE("T=INT32_MIN", a.T = INT32_MIN, MLA_ERR_INVALID_ARG);
  CASE("h NULL", a.h = NULL, MLA_ERR_INVALID_ARG);
  CASE("pos NULL", a.pos = NULL, MLA_ERR_INVALID_ARG);
  CASE("page_table NULL", a.page_table = NULL, MLA_ERR_INVALID_ARG);
  CASE("h +8", a.h = OFF(a.h, 8), MLA_ERR_INVALID_ARG);
  CASE("num_seqs=0", a.num_seqs = 0, MLA_ERR_INVALID_ARG);
  CASE("max_pages=0", a.max_pages = 0, MLA_ERR_INVALID_ARG);
  CASE("seq_id NULL, T > num_seqs", (a.seq_id = NULL, a.num_seqs = 4), MLA_ERR_INVALID_ARG);
  CASE("seq_id NULL, T == num_seqs", a.seq_id = NULL, MLA_ERR_HIP);
  CASE("c_KV NULL", a.c_KV = NULL, MLA_ERR_INVALID_ARG);
  CASE("row_stride=INT64_MAX", a.row_stride = INT64_MAX, MLA_ERR_INVALID_ARG);
  CASE("row_stride=INT64_MIN", a.row_stride = INT64_MIN, MLA_ERR_INVALID_ARG);
  CASE("num_pages=INT32_MAX", a.num_pages = INT32_MAX, MLA_ERR_UNSUPPORTED);
  CASE("max_pages=INT32_MAX", a.max_pages = INT32_MAX, MLA_ERR_UNSUPPORTED);
  CASE("workspace +64", a.ws = with_ws ? OFF(a.ws, 64) : NULL, with_ws ? MLA_ERR_INVALID_ARG : MLA_ERR_HIP);
  CASE("T=INT32_MAX", (a.T = INT32_MAX, a.seq_id = IP(4)), MLA_ERR_INVALID_ARG);
  CASE("T=2^20+1", a.T = (1 << 20) + 1, MLA_ERR_INVALID_ARG);
  CASE("T=2^20", a.T = 1 << 20, MLA_ERR_HIP);
  CASE("T=1024 (split path)", a.T = 1024, MLA_ERR_HIP);
  CASE("T=512 fp32", (a.T = 512, a.d.dtype = MLA_FP32), MLA_ERR_HIP);
  CASE("d_model=64", a.d.d_model = 64, MLA_ERR_HIP);
  CASE("d_model=2^30", a.d.d_model = 1 << 30, MLA_ERR_HIP);
  CASE("ws_bytes=1", a.ws_bytes = 1, MLA_ERR_HIP);
#undef CASE
}

/* ------------------------------------------------------------------ projections */
static void projection_cases(void) {
  char what[256];
  mla_dims d = base_dims();
  const int32_t B = 64, d_cq = 1536;
  const size_t qneed = mla_query_project_workspace_size(&d, B, d_cq);
  expect_true("query_project workspace size > 0", qneed > 0);
#define Q(label, dims, b, dcq, h, wdq, ws, wsb, want)                                                              \
  do {                                                                                                            \
    snprintf(what, sizeof what, "query_project %s", label);                                                      \
    expect(what, mla_query_project(dims, b, dcq, h, wdq, DP(3), DP(4), DP(5), DP(6), ws, wsb, NULL), want);      \
  } while (0)
  Q("valid", &d, B, d_cq, DP(1), DP(2), DP(7), qneed, MLA_ERR_HIP);
  Q("no down-projection", &d, B, 0, DP(1), NULL, DP(7), SIZE_MAX, MLA_ERR_HIP);
  Q("dims NULL", NULL, B, d_cq, DP(1), DP(2), DP(7), qneed, MLA_ERR_INVALID_ARG);
  Q("B=0", &d, 0, d_cq, DP(1), DP(2), DP(7), qneed, MLA_ERR_INVALID_ARG);
  Q("B=2^20+1", &d, (1 << 20) + 1, d_cq, DP(1), DP(2), DP(7), SIZE_MAX, MLA_ERR_INVALID_ARG);
  Q("B=INT32_MAX", &d, INT32_MAX, d_cq, DP(1), DP(2), DP(7), SIZE_MAX, MLA_ERR_INVALID_ARG);
  Q("B=2^20", &d, 1 << 20, d_cq, DP(1), DP(2), DP(7), SIZE_MAX, MLA_ERR_HIP);
  Q("d_cq=100", &d, B, 100, DP(1), DP(2), DP(7), qneed, MLA_ERR_UNSUPPORTED);
  Q("d_cq=-128", &d, B, -128, DP(1), DP(2), DP(7), qneed, MLA_ERR_UNSUPPORTED);
  Q("d_cq=INT32_MAX", &d, B, INT32_MAX, DP(1), DP(2), DP(7), qneed, MLA_ERR_UNSUPPORTED);
  Q("d_cq=65536", &d, B, 65536, DP(1), DP(2), DP(7), SIZE_MAX, MLA_ERR_HIP);
  Q("W_DQ without d_cq", &d, B, 0, DP(1), DP(2), DP(7), SIZE_MAX, MLA_ERR_INVALID_ARG);
  Q("W_DQ NULL with d_cq", &d, B, d_cq, DP(1), NULL, DP(7), qneed, MLA_ERR_INVALID_ARG);
  Q("h NULL", &d, B, d_cq, NULL, DP(2), DP(7), qneed, MLA_ERR_INVALID_ARG);
  Q("h +8", &d, B, d_cq, OFF(DP(1), 8), DP(2), DP(7), qneed, MLA_ERR_INVALID_ARG);
  Q("workspace NULL", &d, B, d_cq, DP(1), DP(2), NULL, qneed, MLA_ERR_INVALID_ARG);
  Q("workspace +16", &d, B, d_cq, DP(1), DP(2), OFF(DP(7), 16), qneed, MLA_ERR_INVALID_ARG);
  Q("ws_bytes=need-1", &d, B, d_cq, DP(1), DP(2), DP(7), qneed - 1, MLA_ERR_WORKSPACE);
  {
    mla_dims f = base_dims();
    f.dtype = MLA_FP32;
    Q("fp32", &f, B, d_cq, DP(1), DP(2), DP(7), SIZE_MAX, MLA_ERR_HIP);
    mla_dims m = base_dims();
    m.d_model = 192;
    Q("bf16 d_model=192", &m, B, d_cq, DP(1), DP(2), DP(7), SIZE_MAX, MLA_ERR_UNSUPPORTED);
  }
  for (int32_t b = 1; b <= 256; b = b * 2 + 1) {
    snprintf(what, sizeof what, "B=%d", b);
    Q(what, &d, b, d_cq, DP(1), DP(2), DP(7), SIZE_MAX, MLA_ERR_HIP);
  }
#undef Q

  const size_t oneed = mla_output_project_workspace_size(&d, B);
  expect_true("output_project workspace size > 0", oneed > 0);
#define O(label, dims, b, o, ws, wsb, want)                                                    \
  do {                                                                                         \
    snprintf(what, sizeof what, "output_project %s", label);                                  \
    expect(what, mla_output_project(dims, b, (const float*)(o), DP(2), FP(3), ws, wsb, NULL), want); \
  } while (0)
  O("valid", &d, B, DP(1), DP(7), oneed, MLA_ERR_HIP);
  O("dims NULL", NULL, B, DP(1), DP(7), oneed, MLA_ERR_INVALID_ARG);
  O("B=0", &d, 0, DP(1), DP(7), oneed, MLA_ERR_INVALID_ARG);
  O("B=INT32_MAX", &d, INT32_MAX, DP(1), DP(7), SIZE_MAX, MLA_ERR_INVALID_ARG);
  O("B=2^20", &d, 1 << 20, DP(1), DP(7), SIZE_MAX, MLA_ERR_HIP);
  O("o NULL", &d, B, NULL, DP(7), oneed, MLA_ERR_INVALID_ARG);
  O("o +4", &d, B, OFF(DP(1), 4), DP(7), oneed, MLA_ERR_INVALID_ARG);
  O("workspace +128", &d, B, DP(1), OFF(DP(7), 128), oneed, MLA_ERR_INVALID_ARG);
  O("ws_bytes=need-1", &d, B, DP(1), DP(7), oneed - 1, MLA_ERR_WORKSPACE);
  for (int32_t b = 1; b <= 256; b = b * 2 + 1) {
    snprintf(what, sizeof what, "B=%d", b);
    O(what, &d, b, DP(1), DP(7), SIZE_MAX, MLA_ERR_HIP);
  }
#undef O

#define PK(label, dims, rows, K, W, Wp, want)                                     \
  do {                                                                            \
    snprintf(what, sizeof what, "pack_weight %s", label);                        \
    expect(what, mla_pack_weight(dims, rows, K, W, Wp, NULL), want);              \
  } while (0)
  PK("valid", &d, 5120, 1536, DP(1), DP(2), MLA_ERR_HIP);
  PK("dims NULL", NULL, 5120, 1536, DP(1), DP(2), MLA_ERR_INVALID_ARG);
  PK("rows=8", &d, 8, 1536, DP(1), DP(2), MLA_ERR_INVALID_ARG);
  PK("rows=INT32_MIN", &d, INT32_MIN, 1536, DP(1), DP(2), MLA_ERR_INVALID_ARG);
  PK("K=16", &d, 5120, 16, DP(1), DP(2), MLA_ERR_INVALID_ARG);
  PK("rows*K=2^40", &d, 1 << 20, 1 << 20, DP(1), DP(2), MLA_ERR_INVALID_ARG);
  PK("rows=K=INT32_MAX&~31", &d, INT32_MAX & ~31, INT32_MAX & ~31, DP(1), DP(2), MLA_ERR_INVALID_ARG);
  PK("rows=2^30, K=32", &d, 1 << 30, 32, DP(1), DP(2), MLA_ERR_HIP);
  PK("rows=16, K=2^30", &d, 16, 1 << 30, DP(1), DP(2), MLA_ERR_HIP);
  PK("W NULL", &d, 5120, 1536, NULL, DP(2), MLA_ERR_INVALID_ARG);
  PK("W_packed +8", &d, 5120, 1536, DP(1), OFF(DP(2), 8), MLA_ERR_INVALID_ARG);
#undef PK
}

/* ------------------------------------------------------------------ prefill */
static void prefill_cases(void) {
  char what[256];
  typedef struct {
    mla_dims d;
    int has_dims;
    int32_t T, num_seqs, max_pages, num_pages, n_splits;
    const void* h;
    const int32_t *seq_id, *pos;
    void* ws;
    size_t ws_bytes;
    int64_t row_stride;
  } PA;
  PA a;
#define CASE(label, mutation, want)                                                                              \
  do {                                                                                                           \
    memset(&a, 0, sizeof a);                                                                                     \
    a.d = base_dims();                                                                                           \
    a.has_dims = 1;                                                                                              \
    a.T = 512;                                                                                                   \
    a.num_seqs = 4;                                                                                              \
    a.max_pages = 64;                                                                                            \
    a.num_pages = 1000;                                                                                          \
    a.n_splits = 0;                                                                                              \
    a.h = DP(1);                                                                                                 \
    a.seq_id = IP(2);                                                                                            \
    a.pos = IP(3);                                                                                               \
    a.ws = DP(20);                                                                                               \
    a.ws_bytes = SIZE_MAX;                                                                                       \
    a.row_stride = 576;                                                                                          \
    mutation;                                                                                                    \
    snprintf(what, sizeof what, "prefill %s", label);                                                            \
    expect(what,                                                                                                 \
           mla_prefill(a.has_dims ? &a.d : NULL, a.T, a.h, DP(4), DP(5), DP(6), DP(7), a.seq_id, a.pos, DP(8),   \
                       DP(9), DP(10), OFF(DP(10), 1024), a.row_stride, a.num_pages, IP(11), a.num_seqs,          \
                       a.max_pages, FP(12), FP(13), a.ws, a.ws_bytes, a.n_splits, NULL),                         \
           want);                                                                                                \
  } while (0)
  CASE("valid", (void)0, MLA_ERR_HIP);
  CASE("dims NULL", a.has_dims = 0, MLA_ERR_INVALID_ARG);
  CASE("T=0", a.T = 0, MLA_ERR_INVALID_ARG);
  CASE("T=2^20+1", a.T = (1 << 20) + 1, MLA_ERR_INVALID_ARG);
  CASE("T=INT32_MAX", a.T = INT32_MAX, MLA_ERR_INVALID_ARG);
  CASE("T=2^20, max_pages=1", (a.T = 1 << 20, a.max_pages = 1), MLA_ERR_HIP);
  CASE("h NULL", a.h = NULL, MLA_ERR_INVALID_ARG);
  CASE("seq_id NULL", a.seq_id = NULL, MLA_ERR_INVALID_ARG);
  CASE("h +8", a.h = OFF(a.h, 8), MLA_ERR_INVALID_ARG);
  CASE("num_seqs=0", a.num_seqs = 0, MLA_ERR_INVALID_ARG);
  CASE("max_pages=0", a.max_pages = 0, MLA_ERR_INVALID_ARG);
  CASE("max_pages=INT32_MAX", a.max_pages = INT32_MAX, MLA_ERR_UNSUPPORTED);
  CASE("T*max_pages*page_size=2^31", (a.T = 1 << 10, a.max_pages = 1 << 15), MLA_ERR_UNSUPPORTED);
  CASE("n_splits=INT32_MAX", a.n_splits = INT32_MAX, MLA_ERR_INVALID_ARG);
  CASE("n_splits=2^20", a.n_splits = 1 << 20, MLA_ERR_HIP);
  CASE("row_stride=INT64_MAX", a.row_stride = INT64_MAX, MLA_ERR_INVALID_ARG);
  CASE("num_pages=INT32_MAX", a.num_pages = INT32_MAX, MLA_ERR_UNSUPPORTED);
  CASE("workspace +16", a.ws = OFF(a.ws, 16), MLA_ERR_INVALID_ARG);
  CASE("ws_bytes=1000", a.ws_bytes = 1000, MLA_ERR_WORKSPACE);
  {
    mla_dims d = base_dims();
    const size_t need = mla_prefill_workspace_size(&d, 512, 64, 0);
    expect_true("prefill workspace size > 0", need > 0);
    CASE("ws_bytes=need-1", a.ws_bytes = need - 1, MLA_ERR_WORKSPACE);
    CASE("ws_bytes=need", a.ws_bytes = need, MLA_ERR_HIP);
  }
#undef CASE
}

/* ------------------------------------------------------------------ whole layer */
static void layer_cases(void) {
  char what[256];
  typedef struct {
    mla_dims d;
    int has_dims;
    int32_t B, d_cq, max_pages, num_pages, n_splits;
    const void *h, *W_DQ;
    void* ws;
    size_t ws_bytes;
    int64_t row_stride;
    mla_decode_opts opts;
    const mla_decode_opts* optp;
  } LA;
  LA a;
#define CASE(label, mutation, want)                                                                               \
  do {                                                                                                            \
    memset(&a, 0, sizeof a);                                                                                      \
    a.d = base_dims();                                                                                            \
    a.has_dims = 1;                                                                                               \
    a.B = 64;                                                                                                     \
    a.d_cq = 1536;                                                                                                \
    a.max_pages = 128;                                                                                            \
    a.num_pages = 9000;                                                                                           \
    a.h = DP(1);                                                                                                  \
    a.W_DQ = DP(2);                                                                                               \
    a.ws = DP(20);                                                                                                \
    a.ws_bytes = SIZE_MAX;                                                                                        \
    a.row_stride = 576;                                                                                           \
    a.optp = NULL;                                                                                                \
    mutation;                                                                                                     \
    snprintf(what, sizeof what, "decode_layer %s", label);                                                        \
    expect(what,                                                                                                  \
           mla_decode_layer(a.has_dims ? &a.d : NULL, a.B, a.d_cq, a.h, DP(3), DP(4), a.W_DQ, DP(5), DP(6), DP(7), \
                            DP(8), DP(9), IP(10), DP(11), OFF(DP(11), 1024), a.row_stride, a.num_pages, IP(12),   \
                            a.max_pages, IP(13), FP(14), FP(15), a.ws, a.ws_bytes, a.n_splits, a.optp, NULL),    \
           want);                                                                                                 \
  } while (0)
  CASE("valid", (void)0, MLA_ERR_HIP);
  CASE("no down-projection", (a.d_cq = 0, a.W_DQ = NULL), MLA_ERR_HIP);
  CASE("dims NULL", a.has_dims = 0, MLA_ERR_INVALID_ARG);
  CASE("B=0", a.B = 0, MLA_ERR_INVALID_ARG);
  CASE("B=INT32_MAX", a.B = INT32_MAX, MLA_ERR_INVALID_ARG);
  CASE("B=2^20, max_pages=1", (a.B = 1 << 20, a.max_pages = 1, a.d.page_size = 1), MLA_ERR_HIP);
  CASE("d_cq=100", a.d_cq = 100, MLA_ERR_UNSUPPORTED);
  CASE("W_DQ NULL", a.W_DQ = NULL, MLA_ERR_INVALID_ARG);
  CASE("h NULL", a.h = NULL, MLA_ERR_INVALID_ARG);
  CASE("h +8", a.h = OFF(a.h, 8), MLA_ERR_INVALID_ARG);
  CASE("workspace +16", a.ws = OFF(a.ws, 16), MLA_ERR_INVALID_ARG);
  CASE("row_stride=INT64_MAX", a.row_stride = INT64_MAX, MLA_ERR_INVALID_ARG);
  CASE("max_pages=0", a.max_pages = 0, MLA_ERR_INVALID_ARG);
  CASE("max_pages=INT32_MAX", a.max_pages = INT32_MAX, MLA_ERR_INVALID_ARG);
  CASE("n_splits=INT32_MAX", a.n_splits = INT32_MAX, MLA_ERR_INVALID_ARG);
  CASE("opts impl=3", (a.opts.impl = 3, a.optp = &a.opts), MLA_ERR_INVALID_ARG);
  CASE("ws_bytes=4096", a.ws_bytes = 4096, MLA_ERR_WORKSPACE);
  {
    mla_dims d = base_dims();
    const size_t need = mla_decode_layer_workspace_size(&d, 64, 1536, 0);
    expect_true("decode_layer workspace size > 0", need > 0);
    CASE("ws_bytes=need-1", a.ws_bytes = need - 1, MLA_ERR_WORKSPACE);
    CASE("ws_bytes=need", a.ws_bytes = need, MLA_ERR_HIP);
  }
#undef CASE
}

/* ------------------------------------------------------------------ sparse top-k */
static void sparse_cases(void) {
  char what[256];
  typedef struct {
    int32_t B, H_I, d_I, top_k, num_pages, page_size, max_pages;
    const void *q_I, *k_I;
    const float* w_I;
    float* scores;
    int32_t* sel_tok;
    int64_t idx_stride;
    void* ws;
    size_t ws_bytes;
  } SA;
  SA a;
#define SEL(label, mutation, want)                                                                               \
  do {                                                                                                           \
    a.B = 4;                                                                                                     \
    a.H_I = 64;                                                                                                  \
    a.d_I = 128;                                                                                                 \
    a.top_k = 2048;                                                                                              \
    a.num_pages = 1000;                                                                                          \
    a.page_size = 64;                                                                                            \
    a.max_pages = 128;                                                                                           \
    a.q_I = DP(1);                                                                                               \
    a.w_I = FP(2);                                                                                               \
    a.k_I = DP(3);                                                                                               \
    a.idx_stride = 128;                                                                                          \
    a.scores = FP(4);                                                                                            \
    a.sel_tok = IP(5);                                                                                           \
    a.ws = DP(6);                                                                                                \
    a.ws_bytes = SIZE_MAX;                                                                                       \
    mutation;                                                                                                    \
    snprintf(what, sizeof what, "indexer_select %s", label);                                                     \
    expect(what,                                                                                                 \
           mla_indexer_select(a.B, a.H_I, a.d_I, a.top_k, a.q_I, a.w_I, a.k_I, a.idx_stride, a.num_pages,        \
                              a.page_size, IP(7), a.max_pages, IP(8), a.scores, a.sel_tok, IP(9), IP(10), a.ws,  \
                              a.ws_bytes, NULL),                                                                 \
           want);                                                                                                \
  } while (0)
  SEL("valid", (void)0, MLA_ERR_HIP);
  SEL("B=0", a.B = 0, MLA_ERR_INVALID_ARG);
  SEL("B=INT32_MIN", a.B = INT32_MIN, MLA_ERR_INVALID_ARG);
  SEL("B=INT32_MAX", a.B = INT32_MAX, MLA_ERR_INVALID_ARG);
  SEL("d_I=64", a.d_I = 64, MLA_ERR_UNSUPPORTED);
  SEL("H_I=8", a.H_I = 8, MLA_ERR_UNSUPPORTED);
  SEL("H_I=16", a.H_I = 16, MLA_ERR_HIP);
  SEL("top_k=0", a.top_k = 0, MLA_ERR_INVALID_ARG);
  SEL("top_k=INT32_MAX", a.top_k = INT32_MAX, MLA_ERR_HIP);
  SEL("top_k=1", a.top_k = 1, MLA_ERR_HIP);
  SEL("q_I NULL", a.q_I = NULL, MLA_ERR_INVALID_ARG);
  SEL("w_I +2", a.w_I = (const float*)OFF(a.w_I, 2), MLA_ERR_INVALID_ARG);
  SEL("w_I +4", a.w_I = (const float*)OFF(a.w_I, 4), MLA_ERR_HIP);
  SEL("k_I +8", a.k_I = OFF(a.k_I, 8), MLA_ERR_INVALID_ARG);
  SEL("idx_stride=100", a.idx_stride = 100, MLA_ERR_INVALID_ARG);
  SEL("idx_stride=132", a.idx_stride = 132, MLA_ERR_INVALID_ARG);
  SEL("idx_stride=INT64_MAX", a.idx_stride = INT64_MAX, MLA_ERR_INVALID_ARG);
  SEL("idx_stride=INT64_MIN", a.idx_stride = INT64_MIN, MLA_ERR_INVALID_ARG);
  SEL("idx_stride=INT64_MAX-7", a.idx_stride = INT64_MAX - 7, MLA_ERR_INVALID_ARG);
  SEL("page_size=8", a.page_size = 8, MLA_ERR_UNSUPPORTED);
  SEL("page_size=INT32_MIN", a.page_size = INT32_MIN, MLA_ERR_UNSUPPORTED);
  SEL("scores +4", a.scores = (float*)OFF(a.scores, 4), MLA_ERR_INVALID_ARG);
  SEL("scores NULL", a.scores = NULL, MLA_ERR_INVALID_ARG);
  SEL("sel_tok NULL", a.sel_tok = NULL, MLA_ERR_INVALID_ARG);
  SEL("workspace +16", a.ws = OFF(a.ws, 16), MLA_ERR_INVALID_ARG);
  SEL("num_pages=0", a.num_pages = 0, MLA_ERR_INVALID_ARG);
  SEL("num_pages=INT32_MAX", a.num_pages = INT32_MAX, MLA_ERR_INVALID_ARG);
  SEL("max_pages=INT32_MAX", a.max_pages = INT32_MAX, MLA_ERR_INVALID_ARG);
  SEL("ws_bytes=0", a.ws_bytes = 0, MLA_ERR_WORKSPACE);
  SEL("max_tokens=2^31-16", (a.B = 1, a.page_size = 16, a.max_pages = (1 << 27) - 1, a.num_pages = (1 << 27) - 1),
      MLA_ERR_HIP);
  SEL("B=2^20, max_tokens=16", (a.B = 1 << 20, a.page_size = 16, a.max_pages = 1), MLA_ERR_HIP);
  SEL("B=2^20+1", a.B = (1 << 20) + 1, MLA_ERR_INVALID_ARG);
  {
    const size_t need = mla_indexer_select_workspace_size(4, 128, 64, 2048);
    expect_true("indexer_select workspace size > 0", need > 0);
    SEL("ws_bytes=need-1", a.ws_bytes = need - 1, MLA_ERR_WORKSPACE);
    SEL("ws_bytes=need", a.ws_bytes = need, MLA_ERR_HIP);
  }
#undef SEL

  typedef struct {
    mla_dims d;
    int has_dims;
    int32_t B, H_I, top_k, max_pages, n_splits;
    const void* q_I;
    int64_t idx_stride, row_stride;
    void* ws;
    size_t ws_bytes;
    mla_decode_opts opts;
    const mla_decode_opts* optp;
  } DA;
  DA s;
#define SP(label, mutation, want)                                                                                  \
  do {                                                                                                             \
    memset(&s, 0, sizeof s);                                                                                       \
    s.d = base_dims();                                                                                             \
    s.has_dims = 1;                                                                                                \
    s.B = 64;                                                                                                      \
    s.H_I = 64;                                                                                                    \
    s.top_k = 2048;                                                                                                \
    s.max_pages = 128;                                                                                             \
    s.q_I = DP(20);                                                                                                \
    s.idx_stride = 128;                                                                                            \
    s.row_stride = 576;                                                                                            \
    s.ws = DP(30);                                                                                                 \
    s.ws_bytes = SIZE_MAX;                                                                                         \
    s.optp = NULL;                                                                                                 \
    mutation;                                                                                                      \
    snprintf(what, sizeof what, "sparse_decode %s", label);                                                        \
    expect(what,                                                                                                   \
           mla_sparse_decode(s.has_dims ? &s.d : NULL, s.B, DP(1), DP(2), IP(3), DP(4), DP(5), DP(6),              \
                             OFF(DP(6), 1024), s.row_stride, 9000, IP(7), s.max_pages, IP(8), s.H_I, 128, s.top_k, \
                             s.q_I, FP(21), DP(22), s.idx_stride, FP(9), FP(10), IP(11), s.ws, s.ws_bytes,         \
                             s.n_splits, s.optp, NULL),                                                            \
           want);                                                                                                  \
  } while (0)
  SP("valid", (void)0, MLA_ERR_HIP);
  SP("sel_tok NULL", (void)0, MLA_ERR_HIP);
  SP("dims NULL", s.has_dims = 0, MLA_ERR_INVALID_ARG);
  SP("fp32", s.d.dtype = MLA_FP32, MLA_ERR_UNSUPPORTED);
  SP("n_h=16", s.d.n_h = 16, MLA_ERR_UNSUPPORTED);
  SP("page_size=48", s.d.page_size = 48, MLA_ERR_UNSUPPORTED);
  SP("B=0", s.B = 0, MLA_ERR_INVALID_ARG);
  SP("B=INT32_MAX", s.B = INT32_MAX, MLA_ERR_INVALID_ARG);
  SP("H_I=128", s.H_I = 128, MLA_ERR_UNSUPPORTED);
  SP("top_k=0", s.top_k = 0, MLA_ERR_INVALID_ARG);
  SP("top_k=INT32_MAX", s.top_k = INT32_MAX, MLA_ERR_UNSUPPORTED);
  SP("B*top_k=2^31", (s.B = 1 << 10, s.top_k = 1 << 21, s.max_pages = 1), MLA_ERR_UNSUPPORTED);
  SP("q_I NULL", s.q_I = NULL, MLA_ERR_INVALID_ARG);
  SP("idx_stride=INT64_MAX", s.idx_stride = INT64_MAX, MLA_ERR_INVALID_ARG);
  SP("row_stride=INT64_MAX", s.row_stride = INT64_MAX, MLA_ERR_INVALID_ARG);
  SP("max_pages=INT32_MAX", s.max_pages = INT32_MAX, MLA_ERR_INVALID_ARG);
  SP("n_splits=INT32_MAX", s.n_splits = INT32_MAX, MLA_ERR_INVALID_ARG);
  SP("n_splits=2^20", s.n_splits = 1 << 20, MLA_ERR_HIP);
  SP("opts impl=1", (s.opts.impl = 1, s.optp = &s.opts), MLA_ERR_INVALID_ARG);
  SP("workspace +16", s.ws = OFF(s.ws, 16), MLA_ERR_INVALID_ARG);
  SP("max_tokens=2^31-32", (s.B = 1, s.max_pages = (1 << 25) - 1, s.top_k = 1 << 30), MLA_ERR_HIP);
  {
    mla_dims d = base_dims();
    const size_t need = mla_sparse_decode_workspace_size(&d, 64, 128, 2048, 0);
    expect_true("sparse_decode workspace size > 0", need > 0);
    SP("ws_bytes=need-1", s.ws_bytes = need - 1, MLA_ERR_WORKSPACE);
    SP("ws_bytes=need", s.ws_bytes = need, MLA_ERR_HIP);
  }
#undef SP
}

/* ------------------------------------------------------------------ workspace sizes */
/* Sizes over a ladder of growing values of one argument: non-decreasing until
 * they drop to 0, then 0. */
static const int64_t LADDER[] = {1,         2,         7,        64,         1000,       1 << 16,
                                 1 << 20,   (1 << 20) + 1, 1 << 24, 1 << 27, 1 << 30,   INT32_MAX};
#define NL ((int)(sizeof LADDER / sizeof LADDER[0]))

typedef size_t (*SizeFn)(int32_t v);
static mla_dims g_sd;
static size_t sz_decode_B(int32_t v) { return mla_decode_workspace_size(&g_sd, v, 256); }
static size_t sz_decode_S(int32_t v) { return mla_decode_workspace_size(&g_sd, 64, v); }
static size_t sz_step_B(int32_t v) { return mla_decode_step_workspace_size(&g_sd, v, 0); }
static size_t sz_step_S(int32_t v) { return mla_decode_step_workspace_size(&g_sd, 64, v); }
static size_t sz_append_T(int32_t v) { return mla_cache_append_workspace_size(&g_sd, v) > 0 ? 1 : 0; }
static size_t sz_query_B(int32_t v) { return mla_query_project_workspace_size(&g_sd, v, 1536); }
static size_t sz_output_B(int32_t v) { return mla_output_project_workspace_size(&g_sd, v); }
static size_t sz_prefill_T(int32_t v) { return mla_prefill_workspace_size(&g_sd, v, 64, 0); }
static size_t sz_prefill_P(int32_t v) { return mla_prefill_workspace_size(&g_sd, 64, v, 0); }
static size_t sz_prefill_S(int32_t v) { return mla_prefill_workspace_size(&g_sd, 64, 64, v); }
static size_t sz_layer_B(int32_t v) { return mla_decode_layer_workspace_size(&g_sd, v, 1536, 0); }
static size_t sz_layer_S(int32_t v) { return mla_decode_layer_workspace_size(&g_sd, 64, 1536, v); }
static size_t sz_select_B(int32_t v) { return mla_indexer_select_workspace_size(v, 128, 64, 2048); }
static size_t sz_select_P(int32_t v) { return mla_indexer_select_workspace_size(4, v, 64, 2048); }
static size_t sz_select_ps(int32_t v) { return mla_indexer_select_workspace_size(4, 128, v, 2048); }
static size_t sz_select_K(int32_t v) { return mla_indexer_select_workspace_size(4, 128, 64, v); }
static size_t sz_sparse_B(int32_t v) { return mla_sparse_decode_workspace_size(&g_sd, v, 128, 2048, 0); }
static size_t sz_sparse_P(int32_t v) { return mla_sparse_decode_workspace_size(&g_sd, 64, v, 2048, 0); }
static size_t sz_sparse_K(int32_t v) { return mla_sparse_decode_workspace_size(&g_sd, 64, 128, v, 0); }
static size_t sz_sparse_S(int32_t v) { return mla_sparse_decode_workspace_size(&g_sd, 64, 128, 2048, v); }

static void ladder(const char* name, SizeFn fn, int must_start_positive) {
  char what[256];
  size_t prev = 0;
  int zero_seen = 0, ok = 1;
  for (int i = 0; i < NL; ++i) {
    const size_t s = fn((int32_t)LADDER[i]);
    if (i == 0 && must_start_positive && s == 0) ok = 0;
    if (zero_seen && s != 0) ok = 0;
    if (s == 0 && i > 0) zero_seen = 1;
    if (s != 0 && s < prev) ok = 0;
    if (!ok) {
      printf("  %s: size %zu at %lld after %zu\n", name, s, (long long)LADDER[i], prev);
      break;
    }
    if (s) prev = s;
  }
  snprintf(what, sizeof what, "workspace size ladder %s", name);
  expect_true(what, ok);
  /* values no call accepts */
  const int32_t bad[] = {0, -1, INT32_MIN};
  for (int i = 0; i < 3; ++i) {
    (void)fn(bad[i]);
  }
}

static void size_cases(void) {
  g_sd = base_dims();
  ladder("decode B", sz_decode_B, 1);
  ladder("decode n_splits", sz_decode_S, 1);
  ladder("step B", sz_step_B, 1);
  ladder("step n_splits", sz_step_S, 1);
  ladder("append T", sz_append_T, 1);
  ladder("query B", sz_query_B, 1);
  ladder("output B", sz_output_B, 1);
  ladder("prefill T", sz_prefill_T, 1);
  ladder("prefill max_pages", sz_prefill_P, 1);
  ladder("prefill n_splits", sz_prefill_S, 1);
  ladder("layer B", sz_layer_B, 1);
  ladder("layer n_splits", sz_layer_S, 1);
  ladder("select B", sz_select_B, 1);
  ladder("select max_pages", sz_select_P, 1);
  ladder("select page_size", sz_select_ps, 1);
  ladder("select top_k", sz_select_K, 1);
  ladder("sparse B", sz_sparse_B, 1);
  ladder("sparse max_pages", sz_sparse_P, 1);
  ladder("sparse top_k", sz_sparse_K, 1);
  ladder("sparse n_splits", sz_sparse_S, 1);
  expect_true("decode size, dims NULL", mla_decode_workspace_size(NULL, 4, 4) == 0);
  expect_true("step size, dims NULL", mla_decode_step_workspace_size(NULL, 4, 4) == 0);
  expect_true("append size, dims NULL", mla_cache_append_workspace_size(NULL, 4) == 0);
  expect_true("query size, dims NULL", mla_query_project_workspace_size(NULL, 4, 0) == 0);
  expect_true("output size, dims NULL", mla_output_project_workspace_size(NULL, 4) == 0);
  expect_true("prefill size, dims NULL", mla_prefill_workspace_size(NULL, 4, 4, 0) == 0);
  expect_true("layer size, dims NULL", mla_decode_layer_workspace_size(NULL, 4, 0, 0) == 0);
  expect_true("sparse size, dims NULL", mla_sparse_decode_workspace_size(NULL, 4, 4, 4, 0) == 0);
  /* sizes the calls reject */
  expect_true("decode size, n_splits=2^20+1", mla_decode_workspace_size(&g_sd, 4, (1 << 20) + 1) == 0);
  expect_true("prefill size, T=2^20+1", mla_prefill_workspace_size(&g_sd, (1 << 20) + 1, 4, 0) == 0);
  expect_true("select size, B*max_tokens=2^31", mla_indexer_select_workspace_size(1 << 10, 1 << 15, 64, 16) == 0);
}

/* ------------------------------------------------------------------ misc */
static void misc_cases(void) {
  int32_t flags = 7;
  expect("read_error_flags NULL workspace", mla_read_error_flags(NULL, &flags, NULL), MLA_ERR_INVALID_ARG);
  expect("read_error_flags NULL out", mla_read_error_flags(DP(1), NULL, NULL), MLA_ERR_INVALID_ARG);
  expect("read_error_flags without a device", mla_read_error_flags(DP(1), &flags, NULL), MLA_ERR_HIP);
  expect_true("read_error_flags leaves the output alone on failure", flags == 7);
  expect_true("cu count without a device", mla_device_cu_count() >= 1);
  expect_true("last error is a string", mla_last_error() != NULL);
}

int main(void) {
  decode_family("decode", run_decode_plain, 0, 1, 0);
  decode_family("decode_ex", run_decode, 0, 1, 1);
  decode_family("decode_step", run_step, 1, 1, 1);
  noalloc_cases();
  append_cases(0);
  append_cases(1);
  projection_cases();
  prefill_cases();
  layer_cases();
  sparse_cases();
  size_cases();
  misc_cases();
  printf("%d cases, %d failed\n", g_cases, g_fail);
  return g_fail ? 1 : 0;
}
