"""Sparse top-k decode on the GPU (mla_indexer_select, mla_sparse_decode)
against the fp64 oracle (reading of DeepSeek architecture V3 to V4
(cyco.top), §4 V3.2 bullet and §6 question 7).

* Selection: integer work on the kernel's fp32 scores, so it is compared
  bit for bit.  With exact-grid inputs (small integers, every score exact in
  fp32) the GPU's scores equal the oracle's fp64 scores and its kept set is
  the oracle's own.  With N(0, 1) inputs the scores are compared within fp32
  rounding, and the kept set must be exactly oracle.topk_select applied to
  the GPU's scores (the decision is taken in the kernel's precision).
* Attention over the kept rows: within the bf16 bar (1e-2) of the oracle's
  attention over the same set.
"""
import numpy as np
import pytest
import torch

import compressed_kv_cache_mla_amd as mla
import oracle
import workloads as W
from cases import lse_err, oracle_decode, oracle_sparse, rel_err

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _small(name="sp_small", B=5, lens=(1, 5000), n_h=128, permute=True, seed=4101):
    cfg = W.scaled(W.CONFIGS["b64_ragged"], name=name, B=B, lens=lens, n_h=n_h, permute_pages=permute, seed=seed)
    return W.Workload(cfg)


def _select(wl, idx, top_k):
    B = wl.cfg.B
    dev = wl.device
    max_tokens = wl.max_pages * wl.cfg.page_size
    scores = torch.full((B, max_tokens), float("nan"), dtype=torch.float32, device=dev)
    sel_tok = torch.full((B, top_k), -1, dtype=torch.int32, device=dev)
    sel_row = torch.full((B, top_k), -1, dtype=torch.int32, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    mla.indexer_select(idx.q_I, idx.w_I, idx.pool, idx.row_stride, wl.num_pages, wl.cfg.page_size, wl.page_table,
                       wl.seq_lens, top_k, scores, sel_tok, sel_row, flags)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), sel_tok.cpu().numpy(), sel_row.cpu().numpy(), int(flags.item())


def _check_selection(wl, idx, top_k, exact):
    scores, sel_tok, sel_row, flags = _select(wl, idx, top_k)
    assert flags == 0
    for b in range(wl.cfg.B):
        n = int(wl.n[b])
        io = idx.oracle_inputs(b)
        ref = oracle.indexer_scores(io["q_I"], io["w_I"], io["k_I"])
        got = scores[b, :n].astype(np.float64)
        m = min(n, top_k)
        if exact:
            assert np.array_equal(got, ref), f"seq {b}: scores differ"
            want = oracle.topk_select(ref, top_k)
        else:
            assert rel_err(got, ref) <= 1e-5, f"seq {b}: scores rel err {rel_err(got, ref)}"
            want = oracle.topk_select(got, top_k)      # the decision in the kernel's precision
        assert np.array_equal(sel_tok[b, :m], want), f"seq {b}: kept set differs"
        assert np.array_equal(sel_row[b, :m], wl.pool_rows(np.full(m, b), want)), f"seq {b}: pool rows differ"
        assert np.all(sel_tok[b, m:] == -1), "entries past the kept count were written"


@pytest.mark.parametrize("H_I", [16, 32, 64])
def test_select_exact_grid(H_I):
    wl = _small()
    idx = W.IndexerInputs(wl, H_I=H_I, exact=True)
    _check_selection(wl, idx, 700, exact=True)


@pytest.mark.parametrize("top_k", [1, 33, 512, 4096])
def test_select_normal_inputs(top_k):
    wl = _small(seed=4102)
    idx = W.IndexerInputs(wl, H_I=64)
    _check_selection(wl, idx, top_k, exact=False)


def test_select_massive_ties():
    """Only four distinct keys: most scores tie, and the smaller index wins."""
    wl = _small(B=3, lens=(2000, 6000), seed=4103)
    idx = W.IndexerInputs(wl, H_I=64, exact=True)
    seq, pos = wl.token_rows()
    keys4 = idx.key_rows(range(4), device=torch.device("cpu"))
    g = np.arange(seq.size)
    rows = torch.from_numpy(wl.pool_rows(seq, pos)).to(wl.device)
    idx.pool[rows] = keys4[torch.from_numpy(g % 4)].to(wl.device)
    scores, sel_tok, _, _ = _select(wl, idx, 1000)
    for b in range(3):
        n = int(wl.n[b])
        io = idx.oracle_inputs(b)
        k_I = keys4.to(torch.float64).numpy()[(np.arange(n) + int(wl.prefix[b])) % 4]
        ref = oracle.indexer_scores(io["q_I"], io["w_I"], k_I)
        assert np.array_equal(scores[b, :n].astype(np.float64), ref)
        assert np.array_equal(sel_tok[b, :min(n, 1000)], oracle.topk_select(ref, 1000))


@pytest.mark.parametrize("lens,B,top_k,exact", [((20000, 60000), 3, 3000, True),
                                                 ((262200, 300000), 2, 2048, False)])
def test_select_long_sequences(lens, B, top_k, exact):
    """Sequences past one selection chunk: each radix pass spread over the
    chunks of a sequence, with the count pass placing each chunk's kept
    tokens (the shorter workloads select in one workgroup per sequence)."""
    cfg = W.scaled(W.CONFIGS["b64_ragged"], name=f"sp_long_{lens[0]}", B=B, lens=lens, cache_mode="direct",
                   seed=4104 + B)
    wl = W.Workload(cfg)
    idx = W.IndexerInputs(wl, H_I=64, exact=exact)
    _check_selection(wl, idx, top_k, exact=exact)


def _sparse(wl, idx, top_k, n_splits=0):
    B = wl.cfg.B
    sel = torch.full((B, top_k), -1, dtype=torch.int32, device=wl.device)
    ws = mla.sparse_decode(wl.dims, wl.q_C, wl.q_R, wl.pos_q, wl.W_UK, wl.W_UV, wl.c_KV, wl.k_R, wl.row_stride,
                           wl.num_pages, wl.page_table, wl.seq_lens, idx.q_I, idx.w_I, idx.pool, idx.row_stride,
                           top_k, wl.out, wl.lse, sel_tok=sel, n_splits=n_splits)
    flags = mla.read_error_flags(ws)
    torch.cuda.synchronize()
    return wl.out.cpu().numpy().copy(), wl.lse.cpu().numpy().copy(), sel.cpu().numpy(), flags


@pytest.mark.parametrize("n_h", [32, 64, 128])
def test_sparse_decode_parity(n_h):
    wl = _small(n_h=n_h, seed=4110 + n_h)
    idx = W.IndexerInputs(wl, H_I=64, exact=True)
    top_k = 300
    out, lse, sel, flags = _sparse(wl, idx, top_k)
    assert flags == 0
    for b in range(wl.cfg.B):
        r_out, r_lse, r_sel, _ = oracle_sparse(wl, idx, b, top_k)
        m = r_sel.size
        assert np.array_equal(sel[b, :m], r_sel)
        assert rel_err(out[b], r_out) <= TOL, f"seq {b}: out rel err {rel_err(out[b], r_out)}"
        assert lse_err(lse[b], r_lse) <= TOL


def test_sparse_all_kept_is_dense():
    """top_k above every length: the dense decode's result (oracle)."""
    wl = _small(B=3, lens=(10, 900), seed=4120)
    idx = W.IndexerInputs(wl, H_I=64)
    out, lse, sel, _ = _sparse(wl, idx, 2048)
    for b in range(3):
        r_out, r_lse = oracle_decode(wl, b)
        assert rel_err(out[b], r_out) <= TOL
        assert lse_err(lse[b], r_lse) <= TOL
        assert np.array_equal(sel[b, :int(wl.n[b])], np.arange(int(wl.n[b])))


@pytest.mark.parametrize("top_k,n_splits", [(1, 0), (33, 7), (257, 1), (1000, 300)])
def test_sparse_ragged_kept_counts(top_k, n_splits):
    """Kept counts that are not multiples of the 32-row tile, one split, and
    more splits than kept tiles."""
    wl = _small(B=4, lens=(20, 3000), seed=4130 + top_k)
    idx = W.IndexerInputs(wl, H_I=32, exact=True)
    out, lse, sel, flags = _sparse(wl, idx, top_k, n_splits)
    assert flags == 0
    for b in range(4):
        r_out, r_lse, r_sel, _ = oracle_sparse(wl, idx, b, top_k)
        assert np.array_equal(sel[b, :r_sel.size], r_sel)
        assert rel_err(out[b], r_out) <= TOL
        assert lse_err(lse[b], r_lse) <= TOL


def test_sparse_deterministic_and_bad_inputs():
    wl = _small(B=4, lens=(100, 2000), seed=4140)
    idx = W.IndexerInputs(wl, H_I=64)
    a = _sparse(wl, idx, 256)
    b = _sparse(wl, idx, 256)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    # sequence 1 empty: zero output, -inf lse, BAD_SEQ_LEN; a bad page id in sequence 2: BAD_PAGE
    lens = wl.seq_lens.clone()
    wl.seq_lens[1] = 0
    pt = wl.page_table.clone()
    wl.page_table[2, 0] = wl.num_pages + 5
    out, lse, sel, flags = _sparse(wl, idx, 256)
    wl.seq_lens.copy_(lens)
    wl.page_table.copy_(pt)
    assert flags & mla.FLAG_BAD_SEQ_LEN and flags & mla.FLAG_BAD_PAGE
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    for b in (0, 3):   # the split boundaries moved: equal up to the split rounding
        assert rel_err(out[b], a[0][b]) <= 5e-3 and lse_err(lse[b], a[1][b]) <= 5e-3


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name,top_k,seqs", [("b4_l131072", 2048, (0, 1, 2, 3)), ("b64_l8192", 2048, (0, 37, 63))])
def test_sparse_full_size(name, top_k, seqs):
    """The benchmark shapes: every sequence's kept set against the oracle's
    selection on the GPU scores, scores against the fp64 indexer, and the
    attention output of some sequences against the oracle over that set."""
    wl = W.Workload(W.CONFIGS[name])
    idx = W.IndexerInputs(wl, H_I=64)
    out, lse, sel, flags = _sparse(wl, idx, top_k)
    assert flags == 0
    scores, sel2, _, _ = _select(wl, idx, top_k)
    assert np.array_equal(sel, sel2)
    for b in range(wl.cfg.B):
        n = int(wl.n[b])
        got = scores[b, :n].astype(np.float64)
        assert np.array_equal(sel[b], oracle.topk_select(got, top_k))
        if b in seqs:
            r_out, r_lse, r_sel, ref_scores = oracle_sparse(wl, idx, b, top_k, sel=sel[b])
            assert rel_err(got, ref_scores) <= 1e-5
            assert rel_err(out[b], r_out) <= TOL, f"seq {b}: out rel err {rel_err(out[b], r_out)}"
            assert lse_err(lse[b], r_lse) <= TOL
