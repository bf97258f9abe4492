// Chunked prefill, per-query inputs of the decode attention.
//
// A chunk of T new tokens (any mix of sequences) is first appended to the
// latent cache; then each new token attends causally to rows 0 .. pos[t] of
// its own sequence, earlier tokens of the same chunk included
// ("DeepSeek-V2：在“大力出奇迹”的AI军备竞赛中，四两拨千斤" (liang.world), ch.2 §1:
// a token attends to the tokens before it and itself).  The attention runs as
// the decode path with one query per new token: query t gets a copy of its
// sequence's page-table row and the length pos[t] + 1, so the split plan lays
// the queries end to end and the splits of one sequence's queries, which
// run on one XCD, read the same pages through its L2.
#include "mla_common.h"

namespace mla {
namespace {

// Thread per (query, page slot): q_pt[t][j] = page_table[seq_id[t]][j];
// j == 0 also writes q_len[t] = pos[t] + 1.  A bad sequence id or position
// gives length 0 (the plan flags it and the query's output is empty) and
// page 0 in every slot.  Thread 0 clears the append's flag word, which the
// append launched next may set.
__global__ void __launch_bounds__(256) prefill_queries_kernel(int32_t T, const int32_t* __restrict__ seq_id,
                                                              const int32_t* __restrict__ pos,
                                                              const int32_t* __restrict__ page_table,
                                                              int32_t num_seqs, int32_t max_pages, int32_t max_tokens,
                                                              int32_t* __restrict__ q_pt, int32_t* __restrict__ q_len,
                                                              int32_t* __restrict__ append_flag) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i == 0) *append_flag = 0;
  if (i >= (int64_t)T * max_pages) return;
  const int32_t t = (int32_t)(i / max_pages), j = (int32_t)(i % max_pages);
  const int32_t s = seq_id[t], p = pos[t];
  const bool ok = s >= 0 && s < num_seqs && p >= 0 && p < max_tokens;
  q_pt[i] = ok ? page_table[(int64_t)s * max_pages + j] : 0;
  if (j == 0) q_len[t] = ok ? p + 1 : 0;
}

}  // namespace

hipError_t launch_prefill_queries(int32_t T, const int32_t* seq_id, const int32_t* pos, const int32_t* page_table,
                                  int32_t num_seqs, int32_t max_pages, int32_t page_size, int32_t* q_pt,
                                  int32_t* q_len, int32_t* append_flag, hipStream_t s) {
  const int64_t n = (int64_t)T * max_pages;
  prefill_queries_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(
      T, seq_id, pos, page_table, num_seqs, max_pages, max_pages * page_size, q_pt, q_len, append_flag);
  return hipGetLastError();
}

}  // namespace mla
