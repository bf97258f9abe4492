"""The allocation-free decode step (mla_decode_step_noalloc, through the C
ABI) against mla_decode_step on a workspace of its own: two calls in a row,
the second with a smaller batch, bit for bit (same kernels, same default
split count), and within the oracle bound on sampled sequences."""
import numpy as np
import pytest
import torch

import workloads as W
from cases import oracle_decode_modes, rel_err, lse_err

pytestmark = pytest.mark.gpu


def test_noalloc_step_equals_decode_step_twice_second_smaller():
    import compressed_kv_cache_mla_amd as mla
    for i, (B, lens) in enumerate([(48, (200, 2500)), (5, (30, 700))]):
        cfg = W.scaled(W.CONFIGS["b64_ragged"], name=f"noalloc_{i}", d_model=1024, B=B, lens=lens, seed=1500 + i)
        print(f"case noalloc call {i}: B={B}", flush=True)
        wl = W.Workload(cfg)
        rows = torch.from_numpy(wl.pool_rows(np.arange(B), wl.n - 1)).to(wl.device)
        h = wl._newest_token_states()
        # the reference: mla_decode_step on a zero-filled workspace of its own
        wl.pool[rows] = 0
        ws = mla.decode_step_workspace(wl.dims, B)
        mla.decode_step(wl.dims, h, wl.W_DKV, wl.W_KR, wl.q_C, wl.q_R, wl.pos_q, wl.W_UK, wl.W_UV, wl.c_KV, wl.k_R,
                        wl.row_stride, wl.num_pages, wl.page_table, wl.seq_lens, wl.out, wl.lse, ws)
        torch.cuda.synchronize()
        assert mla.read_error_flags(ws) == 0
        ref_rows, ref_out, ref_lse = wl.pool[rows].clone(), wl.out.clone(), wl.lse.clone()
        # the allocation-free step on the same inputs
        wl.pool[rows] = 0
        out = torch.full_like(wl.out, float("nan"))
        lse = torch.full_like(wl.lse, float("nan"))
        flags = torch.zeros(1, dtype=torch.int32, device=wl.device)
        mla.decode_step_noalloc(wl.dims, h, wl.W_DKV, wl.W_KR, wl.q_C, wl.q_R, wl.pos_q, wl.W_UK, wl.W_UV, wl.c_KV,
                                wl.k_R, wl.row_stride, wl.num_pages, wl.page_table, wl.seq_lens, out, lse, flags)
        torch.cuda.synchronize()
        assert int(flags.item()) == 0
        assert torch.equal(wl.pool[rows], ref_rows), f"call {i}: appended rows differ"
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"call {i}: outputs differ"
        got, got_lse = out.cpu().numpy(), lse.cpu().numpy()
        for b in (0, B - 1):
            (ref, rlse), = oracle_decode_modes(wl, b, [("absorbed", None)])
            assert rel_err(got[b], ref) <= 1e-2 and lse_err(got_lse[b], rlse) <= 1e-2


def test_noalloc_step_rejects_a_batch_beyond_its_scratch_and_reports_flags():
    import compressed_kv_cache_mla_amd as mla
    cfg = W.scaled(W.CONFIGS["b64_ragged"], name="noalloc_flags", d_model=1024, B=3, lens=(40, 300), seed=1510)
    print("case noalloc limits and flags", flush=True)
    wl = W.Workload(cfg)
    h = wl._newest_token_states()
    flags = torch.zeros(1, dtype=torch.int32, device=wl.device)
    args = lambda pos: (wl.dims, h, wl.W_DKV, wl.W_KR, wl.q_C, wl.q_R, pos, wl.W_UK, wl.W_UV, wl.c_KV,  # noqa
                        wl.k_R, wl.row_stride, wl.num_pages, wl.page_table, wl.seq_lens, wl.out, wl.lse, flags)
    bad = wl.pos_q.clone()
    bad[1] = wl.max_pages * cfg.page_size      # one past the table: the row is skipped and flagged
    mla.decode_step_noalloc(*args(bad))
    torch.cuda.synchronize()
    assert int(flags.item()) & mla.FLAG_BAD_POSITION
    flags.zero_()
    mla.decode_step_noalloc(*args(wl.pos_q))
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    # a batch whose scratch exceeds the array is refused before anything runs
    big = W.Config("noalloc_big", n_h=128, d_model=1024, B=400, lens=1)
    dims = wl.dims
    need = mla.decode_step_workspace_size(dims, big.B)
    assert need > 80 << 20
    q = torch.zeros((big.B, 128, 128), dtype=torch.bfloat16, device="cuda")
    qr = torch.zeros((big.B, 128, 64), dtype=torch.bfloat16, device="cuda")
    hb = torch.zeros((big.B, 1024), dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(big.B, dtype=torch.int32, device="cuda")
    pt = torch.zeros((big.B, 1), dtype=torch.int32, device="cuda")
    ob = torch.zeros((big.B, 128, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(mla.MlaError) as ei:
        mla.decode_step_noalloc(dims, hb, wl.W_DKV, wl.W_KR, q, qr, pos, wl.W_UK, wl.W_UV, wl.c_KV, wl.k_R,
                                wl.row_stride, wl.num_pages, pt, pos + 1, ob)
    assert ei.value.status == mla.MLA_ERR_WORKSPACE
