// Decode step, first launch: everything the attention kernel waits for, as one
// grid of independent workgroups.
//  * workgroup 0: the decode plan (prefix sums, split records; mla_common.h);
//  * then the split-K append of each sequence's newest token (append_splitk.h):
//    c^KV = W^DKV h and k^R = RoPE(W^KR h) ("DeepSeek-V2：在“大力出奇迹”的AI军备竞赛中，
//    四两拨千斤" (liang.world), ch.2 §2-§3), the last workgroup of each
//    (column, token) tile adding the chunks and storing the rows;
//  * then the query absorption q~ = W^UK^T q^C and RoPE(q^R) (absorb_mfma.h;
//    ch.2 §2 absorption paragraph).
// None of the three reads what another writes, so one launch replaces three
// (append, append finish, absorb + plan) and their latency chains overlap.
// The attention kernel reads the new rows after this launch has completed.
// In the decode layer with a low-rank bf16 query the absorption is left out
// of this launch (absorb = false): absorb_fused_kernel (absorb.hip) forms
// q^C = W^UQ c^Q and absorbs it in a launch of its own.
#include "absorb_mfma.h"
#include "append_splitk.h"

namespace mla {
namespace {

struct StepPrepArgs {
  // plan
  PlanArgs pa;
  // append
  const bf16* h_new;
  const bf16* W_DKV;
  const bf16* W_KR;
  float* app_part;
  int32_t* app_cnt;
  AppendDst dst;
  int32_t n_app;        // append workgroups: SK_SPLIT * (D_K / 16) * ceil(B / (16 * append_mt(B)))
  int32_t d_model;
  // absorb
  const bf16* q_C;
  const bf16* q_R;
  const int32_t* pos_q;
  const bf16* W_UK;
  bf16* qabs;
  float qscale;
  int32_t B, n_h;
};

// AMT: 16-row tiles per append workgroup (append_mt).
template <int AMT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) step_prep_kernel(StepPrepArgs a) {
  // absorb's W^UK block (32 KB, so that five workgroups fit in a CU's LDS);
  // the append uses its first gk_red_floats(AMT) floats and one int after them
  __shared__ __attribute__((aligned(1024))) char smem[D_H * 256];
  static_assert(gk_red_floats(4) * 4 + 4 <= D_H * 256, "append reduction fits the absorb block");
  int bid = blockIdx.x;
  if (bid == 0) {
    plan_block<256>(a.pa, (int32_t*)smem, D_H * 256 / 4 - 256);
    return;
  }
  bid -= 1;
  if (bid < a.n_app) {
    // the SK_SPLIT chunks of a tile are neighbours in the grid
    const int kc = bid % SK_SPLIT;
    const int col_blk = (bid / SK_SPLIT) % (D_K / 16);
    const int tok_blk = bid / (SK_SPLIT * (D_K / 16));
    append_splitk_block<true, AMT>(col_blk, kc, tok_blk, a.B, a.d_model, a.h_new, a.W_DKV, a.W_KR, a.app_part,
                                   (float*)smem);
    append_splitk_finish_tile<AMT>(col_blk, tok_blk, a.B, a.d_model, a.app_part, a.app_cnt, a.dst,
                                   (int*)(smem + gk_red_floats(AMT) * 4));
    return;
  }
  bid -= a.n_app;
  const int nx = 4 * a.n_h;
  absorb_mfma_block(bid % nx, bid / nx, 1, a.B, a.n_h, a.q_C, a.q_R, a.pos_q, a.W_UK, a.qscale, a.dst.rope, a.qabs,
                    smem);
}

}  // namespace

bool step_prep_supported(const mla_dims& d, int32_t B) {
  return d.dtype == MLA_BF16 && d.d_model % (SK_SPLIT * 4 * 32) == 0 &&
         (int64_t)((B + SK_TOK - 1) / SK_TOK) * (D_K / 16) <= SPLITK_COUNTERS;
}

hipError_t launch_step_prep(const mla_dims& d, int32_t B, const void* h_new, const void* W_DKV, const void* W_KR,
                            const void* q_C, const void* q_R, const int32_t* pos_q, const void* W_UK, void* qabs,
                            const PlanArgs& pa, float* app_part, int32_t* app_cnt, const AppendDst& dst,
                            hipStream_t s, bool absorb) {
  StepPrepArgs a;
  a.pa = pa;
  a.h_new = (const bf16*)h_new;
  a.W_DKV = (const bf16*)W_DKV;
  a.W_KR = (const bf16*)W_KR;
  a.app_part = app_part;
  a.app_cnt = app_cnt;
  a.dst = dst;
  const int rows = 16 * append_mt(B);
  a.n_app = SK_SPLIT * (D_K / 16) * ((B + rows - 1) / rows);
  a.d_model = d.d_model;
  a.q_C = (const bf16*)q_C;
  a.q_R = (const bf16*)q_R;
  a.pos_q = pos_q;
  a.W_UK = (const bf16*)W_UK;
  a.qabs = (bf16*)qabs;
  a.qscale = d.softmax_scale * LOG2E;
  a.B = B;
  a.n_h = d.n_h;
  const int64_t n_abs = absorb ? (int64_t)4 * d.n_h * ((B + 63) / 64) : 0;
  const int64_t grid = 1 + (int64_t)a.n_app + n_abs;
  // Above 32 sequences each workgroup also requests 12 KB of LDS that it
  // does not use, so that at most three share a CU (4 x 44 KB exceeds the
  // 160 KB): fewer workgroups then wait on their first loads at once, and
  // the launch ends earlier (24.7 against 27.0 us at B = 64, L = 8192).  At
  // 32 sequences or fewer the cap did not help and is not applied.
  const size_t cap_lds = B > 32 ? 12 * 1024 : 0;
  if (append_mt(B) == 4)
    step_prep_kernel<4><<<dim3((unsigned)grid), 256, cap_lds, s>>>(a);
  else
    step_prep_kernel<2><<<dim3((unsigned)grid), 256, cap_lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
