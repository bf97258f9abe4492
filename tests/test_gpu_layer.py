"""GPU parity of the whole decode layer (mla_decode_layer): query projection,
decode step and output projection from the new tokens' states h to u.

Checked two ways: against the three entry points called one after the other
(mla_query_project, mla_decode_step, mla_output_project), and against the
fp64 oracle chained the same way -- oracle.query_project_lowrank, the absorbed
attention over the oracle's own cache rows, oracle.output_project -- on
sampled sequences, within the bf16 bound, with the cache rows the layer
appended held to the oracle's down-projection.  Against the parts the layer is
bit for bit the same except where it forms q^C = W^UQ c^Q inside the
absorption launch (bf16, a low-rank query, more than 8 sequences): there
q^C's fp32 sums run in another order before their bf16 rounding, and u is held
to the parts within a bound far below the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import workloads as W
from cases import gpu_cache_rows, oracle_cache, rel_err

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _proj_weights(seed, n_h, d_model, d_cq, device, dtype=torch.bfloat16):
    g = lambda name, r, c: si.normal(si.stream_key(seed, name), (r, c), c ** -0.5, dtype, device)  # noqa
    return dict(W_DQ=g("W_DQ", d_cq, d_model) if d_cq else None,
                W_UQ=g("W_UQ", n_h * 128, d_cq or d_model), W_QR=g("W_QR", n_h * 64, d_model),
                W_O=g("W_O", d_model, n_h * 128))


@pytest.mark.parametrize("B,d_model,d_cq,lens,dtype", [(5, 1024, 512, (40, 700), torch.bfloat16),
                                                    (40, 1024, 0, (20, 300), torch.bfloat16),
                                                    (1, 1024, 256, (1, 90), torch.bfloat16),
                                                    (3, 1024, 256, (10, 200), torch.float32),
                                                    (20, 1024, 512, (30, 400), torch.bfloat16),
                                                    (64, 1024, 256, (20, 300), torch.bfloat16),
                                                    (70, 2048, 384, (10, 200), torch.bfloat16)])
def test_decode_layer_equals_its_parts_and_the_oracle(B, d_model, d_cq, lens, dtype):
    import compressed_kv_cache_mla_amd as mla
    n_h_cfg = 16 if dtype == torch.float32 else 128
    cfg = W.scaled(W.CONFIGS["b64_ragged"], name=f"layer_b{B}_q{d_cq}", d_model=d_model, B=B, lens=lens,
                   seed=1300 + B + d_cq, dtype=dtype, n_h=n_h_cfg)
    _say(f"case {cfg.name}")
    wl = W.Workload(cfg, n_splits=37)
    dims, n_h = wl.dims, cfg.n_h
    P = _proj_weights(cfg.seed, n_h, d_model, d_cq, "cuda", dtype)
    Pp = {k: (None if v is None else mla.pack_weight(dims, v)) for k, v in P.items()}
    h = wl._newest_token_states()
    u = torch.full((B, d_model), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, n_h), dtype=torch.float32, device="cuda")
    ws = mla.decode_layer_workspace(dims, B, d_cq, 37)
    for call in range(2):
        mla.decode_layer(dims, h, wl.W_DKV, wl.W_KR, Pp["W_DQ"], Pp["W_UQ"], Pp["W_QR"], wl.W_UK, wl.W_UV, Pp["W_O"],
                         wl.pos_q, wl.c_KV, wl.k_R, wl.row_stride, wl.num_pages, wl.page_table, wl.seq_lens, u, lse,
                         ws, n_splits=37)
        torch.cuda.synchronize()
        assert mla.read_error_flags(ws) == 0
    sampled = sorted({0, B - 1, B // 2})
    # the rows the layer appended (the parts below write them again)
    new_rows = {b: gpu_cache_rows(wl, b, [int(wl.prefix[b + 1] - wl.prefix[b]) - 1])[0] for b in sampled}
    # the three parts, one after the other, on workspaces of their own
    q_C = torch.empty((B, n_h, 128), dtype=dtype, device="cuda")
    q_R = torch.empty((B, n_h, 64), dtype=dtype, device="cuda")
    mla.query_project(dims, h, Pp["W_DQ"], Pp["W_UQ"], Pp["W_QR"], q_C, q_R,
                      mla.query_project_workspace(dims, B, d_cq))
    out = torch.empty((B, n_h, 128), dtype=torch.float32, device="cuda")
    lse2 = torch.empty_like(lse)
    mla.decode_step(dims, h, wl.W_DKV, wl.W_KR, q_C, q_R, wl.pos_q, wl.W_UK, wl.W_UV, wl.c_KV, wl.k_R,
                    wl.row_stride, wl.num_pages, wl.page_table, wl.seq_lens, out, lse2,
                    mla.decode_step_workspace(dims, B, 37), 37)
    u2 = torch.empty_like(u)
    mla.output_project(dims, out, Pp["W_O"], u2, mla.output_project_workspace(dims, B))
    torch.cuda.synchronize()
    fused = dtype == torch.bfloat16 and d_cq > 0 and B > 8
    if fused:
        assert rel_err(u.double().cpu().numpy(), u2.double().cpu().numpy()) <= 2e-3
        assert float((lse - lse2).abs().max()) <= 1e-3 * max(1.0, float(lse2.abs().max()))
    else:
        assert torch.equal(u, u2) and torch.equal(lse, lse2)
    # the oracle, chained
    f = {k: (None if v is None else v.double().cpu().numpy()) for k, v in P.items()}
    got = u.double().cpu().numpy()
    for b in sampled:
        d = wl.oracle_inputs(b)
        c, kR = oracle_cache(wl, d)
        e_row = rel_err(new_rows[b], np.concatenate([c[-1], kR[-1]]))
        assert e_row <= (1e-2 if dtype == torch.bfloat16 else 1e-5), f"sequence {b}: appended row rel err {e_row:.3e}"
        h_b = d["h"][d["n"] - 1]
        if d_cq:
            qc, qr = oracle.query_project_lowrank(h_b, f["W_DQ"], f["W_UQ"], f["W_QR"], n_h)
        else:
            qc, qr = oracle.query_project(h_b, f["W_UQ"], f["W_QR"], n_h)
        o, _ = oracle.attend_absorbed(qc, qr, d["pos_q"], c, kR, d["W_UK"], d["W_UV"], dims.rope_base, dims.scale)
        ref = oracle.output_project(o, f["W_O"])
        e = rel_err(got[b], ref)
        assert e <= (1e-2 if dtype == torch.bfloat16 else 1e-5), f"sequence {b}: rel err {e:.3e}"


def test_decode_layer_workspace_reused_at_a_smaller_batch():
    # One workspace, sized for B = 64, serves a B = 64 call and then a B = 8
    # call.  At B = 8 the output projection is split over K and finished in
    # the launch, through tile counters that must sit where the B = 64 call
    # left zeros (not inside its partials): u must equal, bit for bit, the
    # same B = 8 call on a fresh workspace.
    import compressed_kv_cache_mla_amd as mla
    d_model, d_cq = 1024, 512
    runs = {}
    for B in (64, 8):
        cfg = W.scaled(W.CONFIGS["b64_ragged"], name=f"layer_reuse_b{B}", d_model=d_model, B=B, lens=(20, 300),
                       seed=1400 + B)
        wl = W.Workload(cfg)
        P = _proj_weights(cfg.seed, cfg.n_h, d_model, d_cq, "cuda")
        runs[B] = (wl, {k: mla.pack_weight(wl.dims, v) for k, v in P.items()})
    _say("case decode layer workspace B=64 then B=8")
    dims = runs[64][0].dims
    shared = mla.decode_layer_workspace(dims, 64, d_cq)

    def call(B, ws):
        wl, Pp = runs[B]
        u = torch.full((B, d_model), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, wl.cfg.n_h), dtype=torch.float32, device="cuda")
        mla.decode_layer(dims, wl._newest_token_states(), wl.W_DKV, wl.W_KR, Pp["W_DQ"], Pp["W_UQ"], Pp["W_QR"],
                         wl.W_UK, wl.W_UV, Pp["W_O"], wl.pos_q, wl.c_KV, wl.k_R, wl.row_stride, wl.num_pages,
                         wl.page_table, wl.seq_lens, u, lse, ws)
        torch.cuda.synchronize()
        assert mla.read_error_flags(ws) == 0
        return u, lse

    for B in (64, 8, 64, 8):
        u, lse = call(B, shared)
        u_ref, lse_ref = call(B, mla.decode_layer_workspace(dims, B, d_cq))
        assert torch.isfinite(u).all()
        assert torch.equal(u, u_ref) and torch.equal(lse, lse_ref), f"B={B} on the reused workspace"
