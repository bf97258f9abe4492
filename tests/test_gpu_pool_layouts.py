"""GPU: pool layouts other than the interleaved one, through the C ABI.

mla_cache_append, mla_decode and mla_decode_step take the pool as two base
pointers (c_KV, k_R) with one row stride, so the latent part and the rotary
part may sit in separate buffers and rows may carry padding.  The kernels
read and write the same values in the same order whatever the layout, so
every result must be bitwise that of the interleaved pool (row stride 576)
on the same inputs, whose values the oracle tests check; padding columns
must never be written.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

D_C, D_R = 512, 64
STRIDE = 640          # elements per row of each separate buffer (1280 B in bf16, 2560 B in fp32)
PAD = 7.0             # value left in columns that no kernel may write


def _say(msg):
    print(msg, flush=True)


def _split_pools(wl, fill_from_interleaved=True):
    rows = wl.pool.shape[0]
    cpool = torch.full((rows, STRIDE), PAD, dtype=wl.pool.dtype, device=wl.device)
    rpool = torch.full((rows, STRIDE), PAD, dtype=wl.pool.dtype, device=wl.device)
    if fill_from_interleaved:
        cpool[:, :D_C] = wl.pool[:, :D_C]
        rpool[:, :D_R] = wl.pool[:, D_C:]
    return cpool, rpool


def _token_rows(wl):
    """Pool row of every cached token (rows of partly used pages hold none)."""
    seq, pos = wl.token_rows()
    ps = wl.cfg.page_size
    return torch.from_numpy(wl.page_table_np[seq, pos // ps].astype(np.int64) * ps + pos % ps).to(wl.device)


def _assert_rows_equal(wl, cpool, rpool):
    rows = _token_rows(wl)
    assert torch.equal(cpool[rows, :D_C], wl.pool[rows, :D_C]), "c^KV rows differ from the interleaved pool"
    assert torch.equal(rpool[rows, :D_R], wl.pool[rows, D_C:]), "k^R rows differ from the interleaved pool"
    assert torch.all(cpool[:, D_C:] == PAD) and torch.all(rpool[:, D_R:] == PAD), "padding columns were written"
    unused = torch.ones(cpool.shape[0], dtype=torch.bool, device=wl.device)
    unused[rows] = False
    assert torch.all(cpool[unused] == PAD) and torch.all(rpool[unused] == PAD), "rows of no token were written"


CASES = [
    # (name, n_h, d_model, B, lens, dtype, page_size)
    ("ragged_bf16_h32_p16", 32, 512, 5, (0, 400), torch.bfloat16, 16),
    ("ragged_bf16_h128_p64", 128, 1024, 3, (100, 700), torch.bfloat16, 64),
    ("tiny_fp32_h16_p64", 16, 1024, 2, (50, 300), torch.float32, 64),
]


@pytest.mark.parametrize("name,n_h,d_model,B,lens,dtype,page_size", CASES)
def test_separate_padded_pools_match_the_interleaved_pool(name, n_h, d_model, B, lens, dtype, page_size):
    import compressed_kv_cache_mla_amd as mla
    _say(f"case pools {name}")
    cfg = W.scaled(W.CONFIGS["b64_ragged"], name=f"pools_{name}", n_h=n_h, d_model=d_model, B=B, lens=lens,
                   dtype=dtype, page_size=page_size, seed=4100 + n_h + B)
    wl = W.Workload(cfg, n_splits=7)

    # append: every token of every sequence, into empty separate buffers
    cpool, rpool = _split_pools(wl, fill_from_interleaved=False)
    seq, pos = wl.token_rows()
    ids = np.arange(int(wl.prefix[-1]))
    mla.cache_append(wl.dims, wl.h_rows(torch.from_numpy(ids).to(wl.device)), wl.W_DKV, wl.W_KR,
                     torch.from_numpy(pos[ids]).to(wl.device), wl.page_table, cpool, rpool, STRIDE, wl.num_pages,
                     seq_id=torch.from_numpy(seq[ids]).to(wl.device))
    torch.cuda.synchronize()
    _assert_rows_equal(wl, cpool, rpool)

    # decode: bitwise the interleaved result
    wl.decode()
    out2, lse2 = torch.empty_like(wl.out), torch.empty_like(wl.lse)
    ws2 = torch.empty_like(wl.workspace)
    mla.decode(wl.dims, wl.q_C, wl.q_R, wl.pos_q, wl.W_UK, wl.W_UV, cpool, rpool, STRIDE, wl.num_pages,
               wl.page_table, wl.seq_lens, out2, lse2, ws2, wl.n_splits)
    torch.cuda.synchronize()
    assert torch.equal(out2, wl.out) and torch.equal(lse2, wl.lse), "decode differs on separate pools"

    # whole step (append of each newest token + decode): outputs and rows bitwise
    wl.step()
    h = wl._newest_token_states()
    ws3 = mla.decode_step_workspace(wl.dims, cfg.B, wl.n_splits, wl.device)
    out3, lse3 = torch.empty_like(wl.out), torch.empty_like(wl.lse)
    mla.decode_step(wl.dims, h, wl.W_DKV, wl.W_KR, wl.q_C, wl.q_R, wl.pos_q, wl.W_UK, wl.W_UV, cpool, rpool,
                    STRIDE, wl.num_pages, wl.page_table, wl.seq_lens, out3, lse3, ws3, wl.n_splits)
    torch.cuda.synchronize()
    assert torch.equal(out3, wl.out) and torch.equal(lse3, wl.lse), "decode step differs on separate pools"
    _assert_rows_equal(wl, cpool, rpool)


def test_padded_interleaved_rows():
    """One buffer, rows of 640 elements: c^KV in columns 0..511, k^R in
    512..575, padding after."""
    import compressed_kv_cache_mla_amd as mla
    _say("case pools padded interleaved")
    cfg = W.scaled(W.CONFIGS["b64_ragged"], name="pools_padded", n_h=64, d_model=512, B=4, lens=(10, 300),
                   page_size=32, seed=4200)
    wl = W.Workload(cfg, n_splits=5)
    wl.decode()
    torch.cuda.synchronize()
    rows = wl.pool.shape[0]
    pool = torch.full((rows, STRIDE), PAD, dtype=wl.pool.dtype, device=wl.device)
    pool[:, :D_C + D_R] = wl.pool
    out2, lse2 = torch.empty_like(wl.out), torch.empty_like(wl.lse)
    mla.decode(wl.dims, wl.q_C, wl.q_R, wl.pos_q, wl.W_UK, wl.W_UV, pool[:, :D_C], pool[:, D_C:], STRIDE,
               wl.num_pages, wl.page_table, wl.seq_lens, out2, lse2, torch.empty_like(wl.workspace), wl.n_splits)
    torch.cuda.synchronize()
    assert torch.equal(out2, wl.out) and torch.equal(lse2, wl.lse)
