"""GPU parity of the projections around the decode attention, through the C
ABI, against the fp64 CPU oracle:

* mla_query_project: c^Q = W^DQ h, q^C = W^UQ c^Q, q^R = W^QR h (and the
  full-rank form without W^DQ) against oracle.query_project_lowrank /
  oracle.query_project;
* mla_output_project: u = W^O [o_1; ...; o_n_h] against oracle.output_project.

Tolerance as for the decode: max|gpu - oracle| / max|oracle| <= 1e-2 (bf16),
<= 1e-5 (fp32).  Inputs come from the seeded generator, regenerated on the CPU
for the oracle; weights ~ N(0, 1/fan_in), h ~ N(0, 1), o ~ N(0, 1).  Shapes
cover the DeepSeek-V2 sizes (n_h = 128, d_model = 5120, d_cq = 1536) at the
decode batches 32 and 64, split and unsplit products, ragged row blocks, row-major and packed
activations, and two calls in a row on one workspace (the split-K counters
are reset).
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from cases import rel_err

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 1e-2, torch.float32: 1e-5}


def _say(msg):
    print(msg, flush=True)


def _gen(seed, name, shape, fan_in, dtype, device):
    return si.normal(si.stream_key(seed, name), shape, 1.0 / np.sqrt(fan_in) if fan_in else 1.0, dtype, device)


def _query_inputs(seed, B, d_model, n_h, d_cq, dtype, device):
    g = lambda name, shape, fan_in: _gen(seed, name, shape, fan_in, dtype, device)  # noqa: E731
    return dict(h=g("h", (B, d_model), 0),
                W_DQ=g("W_DQ", (d_cq, d_model), d_model) if d_cq else None,
                W_UQ=g("W_UQ", (n_h * 128, d_cq or d_model), d_cq or d_model),
                W_QR=g("W_QR", (n_h * 64, d_model), d_model))


def _dims(mla, n_h, d_model, dtype):
    return mla.Dims(n_h=n_h, d_model=d_model, dtype=dtype)


def _packed(mla, dims, x):
    return {k: (v if v is None or k == "h" else mla.pack_weight(dims, v)) for k, v in x.items()}


def _run_query(mla, dims, x, ws):
    B, n_h = x["h"].shape[0], dims.n_h
    q_C = torch.full((B, n_h, 128), float("nan"), dtype=dims.dtype, device="cuda")
    q_R = torch.full((B, n_h, 64), float("nan"), dtype=dims.dtype, device="cuda")
    mla.query_project(dims, x["h"], x["W_DQ"], x["W_UQ"], x["W_QR"], q_C, q_R, ws)
    torch.cuda.synchronize()
    return q_C.double().cpu().numpy(), q_R.double().cpu().numpy()


def _oracle_query(x, n_h):
    f = {k: (None if v is None else v.double().numpy()) for k, v in x.items()}
    if f["W_DQ"] is None:
        pairs = [oracle.query_project(f["h"][b], f["W_UQ"], f["W_QR"], n_h) for b in range(f["h"].shape[0])]
        return np.stack([p[0] for p in pairs]), np.stack([p[1] for p in pairs])
    return oracle.query_project_lowrank(f["h"], f["W_DQ"], f["W_UQ"], f["W_QR"], n_h)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_pack_weight_is_the_documented_permutation(dtype):
    """Bit-exact: packed[((r/16)*(K/32) + c/32)*512 + ((c%32)/8)*128 + (r%16)*8 + c%8] = W[r, c]."""
    import compressed_kv_cache_mla_amd as mla
    _say(f"case pack {dtype}")
    rows, K = 48, 96
    dims = _dims(mla, 16, 1024, dtype)
    W = _gen(77, "W", (rows, K), 0, dtype, "cuda")
    P = mla.pack_weight(dims, W).cpu().reshape(-1)
    r = np.arange(rows)[:, None]
    c = np.arange(K)[None, :]
    idx = ((r // 16) * (K // 32) + c // 32) * 512 + ((c % 32) // 8) * 128 + (r % 16) * 8 + c % 8
    assert np.array_equal(np.sort(idx.reshape(-1)), np.arange(rows * K))
    assert torch.equal(P[torch.from_numpy(idx.reshape(-1))].reshape(rows, K), W.cpu())


QUERY_CASES = [
    # (B, d_model, n_h, d_cq, dtype)
    (32, 5120, 128, 1536, torch.bfloat16),    # 32-row tiles, both products unsplit
    (64, 5120, 128, 1536, torch.bfloat16),    # 64-row tiles, both unsplit
    (5, 1024, 16, 256, torch.bfloat16),       # row-major h; split 8 and 2
    (40, 1024, 16, 0, torch.bfloat16),        # no down-projection; 32 + 8 rows
    (3, 1024, 16, 128, torch.bfloat16),
    (8, 1024, 16, 128, torch.bfloat16),       # last row-major batch
    (9, 1024, 16, 128, torch.bfloat16),       # first packed batch (16-row tiles)
    (20, 1024, 16, 256, torch.bfloat16),      # 32-row tile, h read row-major (rows past 20 repeat row 19)
    (33, 1024, 16, 256, torch.bfloat16),      # 64-row tiles, one ragged
    (100, 1024, 16, 256, torch.bfloat16),     # two 64-row blocks, the second ragged
    (1, 1024, 16, 512, torch.float32),
    (6, 1024, 16, 0, torch.float32),
]


@pytest.mark.parametrize("B,d_model,n_h,d_cq,dtype", QUERY_CASES)
def test_query_project_matches_oracle(B, d_model, n_h, d_cq, dtype):
    import compressed_kv_cache_mla_amd as mla
    _say(f"case query B={B} d_model={d_model} n_h={n_h} d_cq={d_cq} {dtype}")
    dims = _dims(mla, n_h, d_model, dtype)
    seed = 7000 + B + d_cq
    x = _packed(mla, dims, _query_inputs(seed, B, d_model, n_h, d_cq, dtype, "cuda"))
    ws = mla.query_project_workspace(dims, B, d_cq)
    got_C, got_R = _run_query(mla, dims, x, ws)
    ref_C, ref_R = _oracle_query(_query_inputs(seed, B, d_model, n_h, d_cq, dtype, "cpu"), n_h)
    tol = TOL[dtype]
    assert rel_err(got_C, ref_C) <= tol, f"q_C rel err {rel_err(got_C, ref_C):.3e}"
    assert rel_err(got_R, ref_R) <= tol, f"q_R rel err {rel_err(got_R, ref_R):.3e}"
    # deterministic: a second call on the same workspace gives the same bits
    again_C, again_R = _run_query(mla, dims, x, ws)
    assert np.array_equal(again_C, got_C) and np.array_equal(again_R, got_R)


def test_query_project_two_calls_smaller_second():
    """One workspace, B = 32 then B = 7: the split-K counters left by the first
    call are zero, so the second is right too (and the first's results are
    reproduced on a third call)."""
    import compressed_kv_cache_mla_amd as mla
    _say("case query two calls")
    dims = _dims(mla, 128, 5120, torch.bfloat16)
    ws = mla.query_project_workspace(dims, 32, 1536)
    assert ws.numel() >= mla.query_project_workspace_size(dims, 7, 1536)
    first = None
    for B, seed in ((32, 7100), (7, 7101), (32, 7100)):
        x = _packed(mla, dims, _query_inputs(seed, B, 5120, 128, 1536, torch.bfloat16, "cuda"))
        got_C, got_R = _run_query(mla, dims, x, ws)
        ref_C, ref_R = _oracle_query(_query_inputs(seed, B, 5120, 128, 1536, torch.bfloat16, "cpu"), 128)
        assert rel_err(got_C, ref_C) <= 1e-2 and rel_err(got_R, ref_R) <= 1e-2, f"B={B}"
        if B == 32:
            if first is None:
                first = got_C
            else:
                assert np.array_equal(first, got_C)


OUTPUT_CASES = [
    # (B, d_model, n_h, dtype)
    (32, 5120, 128, torch.bfloat16),          # split 4, in-launch finish
    (64, 5120, 128, torch.bfloat16),          # split 4, 64-row tiles
    (1, 1024, 16, torch.bfloat16),            # split 16, one row
    (37, 1024, 16, torch.bfloat16),           # 64-row tile, ragged
    (8, 1024, 16, torch.bfloat16),            # row-major activations
    (17, 1024, 16, torch.bfloat16),           # 32-row tile
    (130, 1024, 16, torch.bfloat16),          # three 64-row blocks, the last ragged
    (3, 1024, 16, torch.float32),
]


def _output_inputs(seed, B, d_model, n_h, dtype, device):
    o = _gen(seed, "o", (B, n_h, 128), 0, torch.float32, device)
    W_O = _gen(seed, "W_O", (d_model, n_h * 128), n_h * 128, dtype, device)
    return o, W_O


@pytest.mark.parametrize("B,d_model,n_h,dtype", OUTPUT_CASES)
def test_output_project_matches_oracle(B, d_model, n_h, dtype):
    import compressed_kv_cache_mla_amd as mla
    _say(f"case output B={B} d_model={d_model} n_h={n_h} {dtype}")
    dims = _dims(mla, n_h, d_model, dtype)
    seed = 8000 + B
    o, W_O = _output_inputs(seed, B, d_model, n_h, dtype, "cuda")
    W_O = mla.pack_weight(dims, W_O)
    ws = mla.output_project_workspace(dims, B)
    u = torch.full((B, d_model), float("nan"), dtype=torch.float32, device="cuda")
    mla.output_project(dims, o, W_O, u, ws)
    torch.cuda.synchronize()
    got = u.double().cpu().numpy()
    o_c, W_c = _output_inputs(seed, B, d_model, n_h, dtype, "cpu")
    ref = oracle.output_project(o_c.double().numpy(), W_c.double().numpy())
    e = rel_err(got, ref)
    assert e <= TOL[dtype], f"u rel err {e:.3e}"
    u2 = torch.empty_like(u)
    mla.output_project(dims, o, W_O, u2, ws)
    torch.cuda.synchronize()
    assert torch.equal(u, u2)


def test_output_project_two_calls_smaller_second():
    import compressed_kv_cache_mla_amd as mla
    _say("case output two calls")
    dims = _dims(mla, 128, 5120, torch.bfloat16)
    ws = mla.output_project_workspace(dims, 32)
    for B, seed in ((32, 8100), (5, 8101)):
        o, W_O = _output_inputs(seed, B, 5120, 128, torch.bfloat16, "cuda")
        W_O = mla.pack_weight(dims, W_O)
        u = torch.empty((B, 5120), dtype=torch.float32, device="cuda")
        mla.output_project(dims, o, W_O, u, ws)
        torch.cuda.synchronize()
        o_c, W_c = _output_inputs(seed, B, 5120, 128, torch.bfloat16, "cpu")
        e = rel_err(u.double().cpu().numpy(), oracle.output_project(o_c.double().numpy(), W_c.double().numpy()))
        assert e <= 1e-2, f"B={B}: rel err {e:.3e}"
