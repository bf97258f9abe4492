// Query absorption for bf16 on the matrix cores, as a device function shared
// by the absorb launch (absorb.hip) and the fused decode step (step.hip).
//
// q~_i = W^UK_i^T q^C_i and RoPE(q^R_i) at the query position, both scaled by
// softmax_scale * log2(e) ("DeepSeek-V2：在“大力出奇迹”的AI军备竞赛中，四两拨千斤"
// (liang.world), ch.2 §2 absorption paragraph, §3 decoupled RoPE).
#pragma once

#include "mla_common.h"

namespace mla {

// Workgroup (head h, latent columns 128q .. 128q+127, nby blocks of 64
// sequences: blocks by*nby .. by*nby + nby - 1), 4 waves.
// q~^T[c][b] = sum_d W^UK_h[d][c] q^C[b][d] as v_mfma_f32_32x32x16_bf16 with
// M = latent column c, N = sequence, K = d.  The W^UK_h column block (128 rows
// x 256 B = 32 KB) is copied to LDS once, with global_load_lds, 4 rows of
// 256 B per copy instruction; 16-byte chunk c16 of row d sits at chunk
// c16 ^ 4*(d & 3), which keeps the transposed reads (ds_read_b64_tr_b16, 4
// rows x 4 chunks per half-wave) bank-conflict free.  Wave w produces columns
// 128q + 32w .. +31.  With more than one block (long batches: prefill), the
// W^UK block serves all of them.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// Stores one wave's 32-column x 32-sequence block of q~, scaled and rounded
// to bf16.  The accumulator is in the C layout of v_mfma_f32_32x32x16_bf16
// (lane -> sequence lane & 31, latent rows (r/4)*8 + 4*(lane>>5) + r%4), so
// each lane holds four runs of 4 rows.  v_permlane32_swap trades row runs
// between the half-waves until half k holds rows 16p + 8k .. 16p + 8k + 7 for
// p = 0, 1; one 16-byte store per p then gives each sequence 32 contiguous
// bytes of its 64-byte run of the q~ layout per store instruction, where
// 8-byte stores gave 16.  Every lane of the wave takes part in the swaps;
// qb is null for lanes whose sequence is past the batch.
__device__ __forceinline__ void store_qabs_block(const f32x16& acc, float qscale, bf16* qb, int32_t n_h, int h,
                                                 int dbase, int lane) {
  unsigned int w[8];
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      bf16x2 v;
      v[0] = (bf16)(acc[4 * r4 + 2 * i] * qscale);
      v[1] = (bf16)(acc[4 * r4 + 2 * i + 1] * qscale);
      w[2 * r4 + i] = __builtin_bit_cast(unsigned int, v);
    }
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      // lanes 32..63 of the first operand trade with lanes 0..31 of the second
      const auto x = __builtin_amdgcn_permlane32_swap(w[4 * p + i], w[4 * p + 2 + i], false, false);
      w[4 * p + i] = x[0];
      w[4 * p + 2 + i] = x[1];
    }
  }
  if (qb != nullptr) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      u32x4 o;
      o[0] = w[4 * p];
      o[1] = w[4 * p + 1];
      o[2] = w[4 * p + 2];
      o[3] = w[4 * p + 3];
      *(u32x4*)(qb + qabs_offset(n_h, true, h, dbase + 16 * p + 8 * (lane >> 5))) = o;
    }
  }
}

__device__ __forceinline__ void absorb_mfma_block(int bx, int by, int nby, int32_t B, int32_t n_h,
                                                  const bf16* __restrict__ q_C, const bf16* __restrict__ q_R,
                                                  const int32_t* __restrict__ pos_q, const bf16* __restrict__ W_UK,
                                                  float qscale, const RopeTab& rope, bf16* __restrict__ qabs,
                                                  char* wl) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // bx -> (head, quarter): quarter = bits 0-1, head bit 1 = bit 2, head bit 0
  // = bit 3, head >> 2 = bits 4 and up.  Heads h and h^1 share the 128-byte
  // lines of the q~ layout; with this order their workgroups for one quarter
  // are 8 apart in the grid, so on the same XCD (workgroups are dealt to the
  // 8 XCDs in turn) and their halves of each line meet in one L2.
  int h = bx >> 2;
  const int cq = bx & 3;
  if ((n_h & 3) == 0) h = ((bx >> 4) << 2) | (((bx >> 2) & 1) << 1) | ((bx >> 3) & 1);
  // W^UK_h[:, 128cq .. 128cq+127] -> LDS (2048 chunks of 16 B; 8 copy instructions per wave)
  const char* wsrc = (const char*)(W_UK + (int64_t)h * D_H * D_C) + 256 * cq;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int sigma = (wave * 8 + k) * 64 + lane;
    const int d = sigma >> 4, pos = sigma & 15;
    const int c16 = pos ^ ((d & 3) << 2);
    __builtin_amdgcn_global_load_lds((const void*)(wsrc + (int64_t)d * 1024 + c16 * 16),
                                     (lds_void_t*)(wl + (wave * 8 + k) * 1024), 16, 0, 0);
  }
  // q^C fragments of one 32-sequence block: lane -> sequence b0 + 32*nblk +
  // (lane & 31), d = 16*ks + 8*(lane >> 5).  The second block (sequences
  // 32..63) is loaded after the first block's MFMAs have read their operands.
  bf16x8 qf[8];
  auto load_qf = [&](int b0, int nblk) {
    const int b = min(b0 + 32 * nblk + (lane & 31), B - 1);
    const bf16* qp = q_C + ((int64_t)b * n_h + h) * D_H + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8*)(qp + 16 * ks);
  };
  // transposed-read source address: row d = 16ks + 8*(lane>>5) + 4rr + ((lane&15)>>2),
  // local columns 32w + 16*((lane>>4)&1) + 4*(lane&3)
  const int t_row = 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int t_c16 = 4 * wave + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int t_half = (lane & 1) * 8;
  auto block_product = [&]() -> f32x16 {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bf16x8 af;
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int d = 16 * ks + t_row + 4 * rr;
        const int c16 = t_c16 ^ ((d & 3) << 2);
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(wl + d * 256 + c16 * 16 + t_half));
        const bf16x4 vb = __builtin_bit_cast(bf16x4, v);
        af[4 * rr + 0] = vb[0];
        af[4 * rr + 1] = vb[1];
        af[4 * rr + 2] = vb[2];
        af[4 * rr + 3] = vb[3];
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ks], acc, 0, 0, 0);
    }
    return acc;
  };
  // C layout: lane -> sequence (lane & 31) of the block, latent rows (r/4)*8 + 4*(lane>>5) + r%4
  auto store_block = [&](const f32x16& acc, int b0, int nb, int nblk) {
    const int bb = 32 * nblk + (lane & 31);
    store_qabs_block(acc, qscale, bb < nb ? qabs + (int64_t)(b0 + bb) * n_h * D_K : nullptr, n_h, h,
                     128 * cq + 32 * wave, lane);
  };
  // RoPE half (32 pairs per sequence), shared by the 4 column-quarter
  // workgroups of the head (pairs 512q .. 512q+511 of a 64-sequence block,
  // two per thread): its operands are loaded with the block's first query
  // fragments, so that their latency passes with that of the W^UK copy, and
  // it is computed and stored after the first 32 sequences' product.
  constexpr int RJ = 64 * (D_R / 2) / (4 * 256);
  bf16x2 rx[RJ];
  int32_t rpos[RJ];
  auto load_rope = [&](int b0, int nb) {
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
      const int i = tid + 256 * (RJ * cq + j);
      if (i < nb * (D_R / 2)) {
        const int b = b0 + i / (D_R / 2), k = i % (D_R / 2);
        rx[j] = *(const bf16x2*)(q_R + ((int64_t)b * n_h + h) * D_R + 2 * k);
        rpos[j] = pos_q[b];
      }
    }
  };
  auto store_rope = [&](int b0, int nb) {
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
      const int i = tid + 256 * (RJ * cq + j);
      if (i < nb * (D_R / 2)) {
        const int b = b0 + i / (D_R / 2), k = i % (D_R / 2);
        const float x0 = (float)rx[j][0], x1 = (float)rx[j][1];
        float cs, sn;
        rope_cos_sin(rpos[j], k, rope, &cs, &sn);
        bf16x2 o;
        o[0] = (bf16)((x0 * cs - x1 * sn) * qscale);
        o[1] = (bf16)((x0 * sn + x1 * cs) * qscale);
        *(bf16x2*)(qabs + (int64_t)b * n_h * D_K + qabs_offset(n_h, true, h, D_C + 2 * k)) = o;
      }
    }
  };
  for (int j = 0; j < nby; ++j) {
    const int b0 = (by * nby + j) * 64;
    if (b0 >= B) break;
    const int nb = min(64, B - b0);
    load_qf(b0, 0);
    load_rope(b0, nb);
    __builtin_amdgcn_s_waitcnt(0);
    if (j == 0) __syncthreads();   // the W^UK block has landed (it is only read from here on)
    {
      const f32x16 acc0 = block_product();
      if (nb > 32) load_qf(b0, 1);
      store_block(acc0, b0, nb, 0);
    }
    // while the second block's query loads are in flight
    store_rope(b0, nb);
    if (nb > 32) store_block(block_product(), b0, nb, 1);
  }
}


}  // namespace mla
