"""Pins of the fp64 CPU oracle to facts fixed outside itself.

* cache sizes printed by the pages (tests/golden/cache_sizes.json);
* RoPE against RoFormer's complex-number form (a different formulation of the
  same rotation) and against its defining invariants;
* the whole decode attention against PyTorch's own scaled_dot_product_attention
  (float64, CPU) run on keys/queries/values that this file materialises with
  torch ops from the token states and weights (MHA over reconstructed K/V,
  DeepSeek-V2 architecture revolution (liang.world), ch.2 §1-§3);
* lse against torch.logsumexp of independently computed scores;
* closed forms of softmax attention (q = 0, one token, identical latents);
* the absorbed form against the reconstructed form (associativity,
  ch.2 §2 of the same page), bit-exact on integer data;
* brute-force loops for the down-projection on a tiny input;
* the low-rank query path (c^Q = W^DQ h) against the same torch attention with
  the product matrix W^UQ W^DQ formed first, against the full-rank path when
  W^DQ is the identity, and by the rank bound it implies;
* the output projection W^O by head selectors, the sum of heads, and the
  absorption of W^UV into W^O (ch.2 §2);
* a causal chunk of new tokens against torch's scaled_dot_product_attention
  with an explicit causal mask over materialised q, k, v, and by the
  no-future-leak invariant.

The last tests plant typical mistakes in copies of the oracle's functions and
check that the pins above catch each of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mla as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cache_sizes.json")
BASE = 10000.0


# ----------------------------------------------------------------------------- sizes
def test_cache_sizes_match_pages():
    g = json.load(open(GOLDEN))
    e = g["mha_elements_per_token"]
    assert oracle.mha_cache_elements_per_token(e["n_h"], e["d_h"]) == e["value"]
    e = g["mla_elements_per_token"]
    assert oracle.mla_cache_elements_per_token(e["d_c"], e["d_hR"]) == e["value"]
    e = g["mla_elements_per_token_60_layers"]
    assert oracle.mla_cache_elements_per_token(e["d_c"], e["d_hR"]) * e["layers"] == e["value"]
    e = g["gqa_equivalent_groups"]
    assert oracle.gqa_equivalent_groups(e["d_c"], e["d_hR"], e["d_h"]) == e["value"]
    # the exact MLA/MHA ratio at DeepSeek-V2 dims (the page's "about 2.2%" is loose)
    assert 576 / 32768 == pytest.approx(0.017578125)


# ----------------------------------------------------------------------------- RoPE
def _rope_complex(x, pos, base=BASE):
    """RoFormer complex form: pair k is the complex number x[2k] + i x[2k+1],
    multiplied by exp(i * pos * theta_k), theta_k = base^(-2k/d)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    theta = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    z = z * np.exp(1j * pos * theta)
    out = np.empty_like(x)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


@pytest.mark.parametrize("pos", [0, 1, 7, 255, 4096, 131071])
def test_rope_matches_complex_form(pos):
    rng = np.random.default_rng(pos)
    x = rng.standard_normal((5, 64))
    np.testing.assert_allclose(oracle.rope(x, pos, BASE), _rope_complex(x, pos), rtol=0, atol=1e-12)


def test_rope_identity_norm_and_first_pair():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(64)
    assert np.array_equal(oracle.rope(x, 0, BASE), x)
    for p in (3, 1000, 131072):
        y = oracle.rope(x, p, BASE)
        assert np.linalg.norm(y) == pytest.approx(np.linalg.norm(x), rel=1e-14)
    e0 = np.zeros(64)
    e0[0] = 1.0
    y = oracle.rope(e0, 2.5, BASE)            # theta_0 = 1: pair 0 turns by pos radians
    assert y[0] == pytest.approx(math.cos(2.5), abs=1e-15)
    assert y[1] == pytest.approx(math.sin(2.5), abs=1e-15)
    assert np.all(y[2:] == 0)


def test_rope_relative_position_invariance():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n, s in [(5, 2, 11), (4096, 17, 1000), (100, 100, 131000)]:
        a = oracle.rope(q, m, BASE) @ oracle.rope(k, n, BASE)
        b = oracle.rope(q, m + s, BASE) @ oracle.rope(k, n + s, BASE)
        assert a == pytest.approx(b, rel=1e-9, abs=1e-9)


# ----------------------------------------------------------------------------- helpers
def _problem(rng, n_h=3, d_h=8, d_c=12, d_hR=6, d_model=20, n=9, integer=False):
    if integer:
        f = lambda *s: rng.integers(-2, 3, size=s).astype(np.float64)  # noqa: E731
    else:
        f = lambda *s: rng.standard_normal(s) / math.sqrt(s[-1])       # noqa: E731
    return dict(h=f(n, d_model) * (1 if integer else math.sqrt(d_model)),
                W_DKV=f(d_c, d_model), W_KR=f(d_hR, d_model), W_UK=f(n_h * d_h, d_c),
                W_UV=f(n_h * d_h, d_c), W_UQ=f(n_h * d_h, d_model), W_QR=f(n_h * d_hR, d_model),
                n_h=n_h, d_h=d_h, d_hR=d_hR, n=n)


def _torch_mha(P, pos_shift=0):
    """Multi-head attention of the last token over all n tokens, with q, k, v
    materialised per head from h (k^C = W^UK W^DKV h, v = W^UV W^DKV h,
    k^R = RoPE(W^KR h) shared by all heads, q = [W^UQ h ; RoPE(W^QR h)]),
    run through torch's scaled_dot_product_attention (float64, CPU) with its
    default 1/sqrt(head width) scale.  Returns (out [n_h, d_h], lse [n_h])."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    n_h, d_h, d_hR, n = P["n_h"], P["d_h"], P["d_hR"], P["n"]
    h = t(P["h"])
    pos = torch.arange(n, dtype=torch.float64) + pos_shift

    def rot(x, p):  # complex form, torch
        d = x.shape[-1]
        theta = BASE ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
        z = torch.view_as_complex(x.reshape(*x.shape[:-1], d // 2, 2).contiguous())
        z = z * torch.polar(torch.ones_like(theta), p[..., None] * theta)
        return torch.view_as_real(z).reshape(x.shape)

    c = h @ t(P["W_DKV"]).T
    kC = torch.einsum("hdc,nc->hnd", t(P["W_UK"]).reshape(n_h, d_h, -1), c)
    v = torch.einsum("hdc,nc->hnd", t(P["W_UV"]).reshape(n_h, d_h, -1), c)
    kR = rot(h @ t(P["W_KR"]).T, pos)                       # [n, d_hR]
    k = torch.cat([kC, kR.unsqueeze(0).expand(n_h, n, d_hR)], dim=-1)
    hq = h[n - 1]
    # with a query down-projection, q^C = (W^UQ W^DQ) h: the product matrix is formed first
    W_q = t(P["W_UQ"]) @ t(P["W_DQ"]) if "W_DQ" in P else t(P["W_UQ"])
    qC = (W_q @ hq).reshape(n_h, d_h)
    qR = rot((t(P["W_QR"]) @ hq).reshape(n_h, d_hR), pos[n - 1].expand(n_h))
    q = torch.cat([qC, qR], dim=-1)[:, None, :]              # [n_h, 1, E]
    out = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None])[0, :, 0]
    scores = (q @ k.transpose(1, 2))[:, 0] / math.sqrt(d_h + d_hR)
    return out.numpy(), torch.logsumexp(scores, dim=-1).numpy()


def _oracle_run(P, attend=oracle.attend_reconstruct, pos_shift=0, down=oracle.down_project,
                scale=None):
    n = P["n"]
    pos = np.arange(n) + pos_shift
    c, kR = down(P["h"], P["W_DKV"], P["W_KR"], pos, BASE)
    if "W_DQ" in P:
        qC, qR = oracle.query_project_lowrank(P["h"][n - 1], P["W_DQ"], P["W_UQ"], P["W_QR"], P["n_h"])
    else:
        qC, qR = oracle.query_project(P["h"][n - 1], P["W_UQ"], P["W_QR"], P["n_h"])
    if scale is None:
        scale = oracle.softmax_scale(P["d_h"], P["d_hR"])
    return attend(qC, qR, pos[-1], c, kR, P["W_UK"], P["W_UV"], BASE, scale)


def _rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / np.max(np.abs(b)))


# ----------------------------------------------------------------------------- attention pins
@pytest.mark.parametrize("seed,shape", [(0, {}), (1, dict(n_h=2, d_h=4, d_c=8, d_hR=4, d_model=16, n=5)),
                                        (2, dict(n_h=4, d_h=16, d_c=32, d_hR=8, d_model=40, n=33))])
@pytest.mark.parametrize("attend", [oracle.attend_reconstruct, oracle.attend_absorbed])
def test_attention_matches_torch_sdpa(seed, shape, attend):
    P = _problem(np.random.default_rng(seed), **shape)
    out, lse = _oracle_run(P, attend)
    ref, ref_lse = _torch_mha(P)
    assert _rel(out, ref) < 1e-12
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_attention_is_invariant_to_a_common_position_shift():
    P = _problem(np.random.default_rng(5))
    a, la = _oracle_run(P)
    b, lb = _oracle_run(P, pos_shift=1000)
    assert _rel(b, a) < 1e-9
    np.testing.assert_allclose(lb, la, rtol=1e-9)


def test_absorbed_equals_reconstructed_bitwise_scores_on_integers():
    """Integer data with the RoPE weights zeroed: every score is an exact
    integer times the scale in both forms, so the softmax weights agree
    bit for bit; outputs agree to rounding of the final sums."""
    rng = np.random.default_rng(3)
    P = _problem(rng, integer=True, n=11)
    P["W_KR"] = np.zeros_like(P["W_KR"])
    P["W_QR"] = np.zeros_like(P["W_QR"])
    o1, l1, p1 = _oracle_run(P, lambda *a: oracle.attend_reconstruct(*a, return_probs=True))
    o2, l2, p2 = _oracle_run(P, lambda *a: oracle.attend_absorbed(*a, return_probs=True))
    assert np.array_equal(p1, p2)
    assert np.array_equal(l1, l2)
    assert _rel(o2, o1) < 1e-13


def test_absorbed_equals_reconstructed_deepseek_head_dims():
    rng = np.random.default_rng(4)
    P = _problem(rng, n_h=4, d_h=128, d_c=512, d_hR=64, d_model=96, n=40)
    o1, l1 = _oracle_run(P, oracle.attend_reconstruct)
    o2, l2 = _oracle_run(P, oracle.attend_absorbed)
    assert _rel(o2, o1) < 1e-12
    np.testing.assert_allclose(l2, l1, rtol=1e-12)


def test_softmax_rows_sum_to_one():
    P = _problem(np.random.default_rng(6), n=50)
    for attend in (oracle.attend_reconstruct, oracle.attend_absorbed):
        _, _, p = _oracle_run(P, lambda *a: attend(*a, return_probs=True))
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-14
        assert np.all(p > 0)


# ----------------------------------------------------------------------------- closed forms
def _latents(rng, n, n_h=4, d_h=16, d_c=32, d_hR=8):
    return (rng.standard_normal((n_h, d_h)), rng.standard_normal((n_h, d_hR)),
            rng.standard_normal((n, d_c)), rng.standard_normal((n, d_hR)),
            rng.standard_normal((n_h * d_h, d_c)) / math.sqrt(d_c),
            rng.standard_normal((n_h * d_h, d_c)) / math.sqrt(d_c))


@pytest.mark.parametrize("attend", [oracle.attend_reconstruct, oracle.attend_absorbed])
def test_zero_query_gives_mean_latent(attend):
    rng = np.random.default_rng(7)
    qC, qR, c, kR, WUK, WUV = _latents(rng, 23)
    out, lse = attend(np.zeros_like(qC), np.zeros_like(qR), 22, c, kR, WUK, WUV, BASE, 0.1)
    ref = (WUV.reshape(4, 16, 32) @ c.mean(axis=0))
    assert _rel(out, ref) < 1e-13
    np.testing.assert_allclose(lse, np.log(23.0), rtol=1e-14)


@pytest.mark.parametrize("attend", [oracle.attend_reconstruct, oracle.attend_absorbed])
def test_single_token_returns_its_value(attend):
    rng = np.random.default_rng(8)
    qC, qR, c, kR, WUK, WUV = _latents(rng, 1)
    out, _ = attend(qC, qR, 0, c, kR, WUK, WUV, BASE, 0.3)
    assert _rel(out, WUV.reshape(4, 16, 32) @ c[0]) < 1e-14


@pytest.mark.parametrize("attend", [oracle.attend_reconstruct, oracle.attend_absorbed])
def test_identical_latents_give_that_value(attend):
    rng = np.random.default_rng(9)
    qC, qR, c, kR, WUK, WUV = _latents(rng, 17)
    c[:] = c[3]
    out, _ = attend(qC, qR, 16, c, kR, WUK, WUV, BASE, 0.2)
    assert _rel(out, WUV.reshape(4, 16, 32) @ c[3]) < 1e-13


def test_down_project_brute_force():
    rng = np.random.default_rng(10)
    h = rng.standard_normal((3, 5))
    Wd = rng.standard_normal((4, 5))
    Wr = rng.standard_normal((2, 5))
    c, kR = oracle.down_project(h, Wd, Wr, np.array([0, 1, 2]), BASE)
    for t in range(3):
        for o in range(4):
            assert c[t, o] == pytest.approx(sum(Wd[o, i] * h[t, i] for i in range(5)), abs=1e-13)
        x = [sum(Wr[o, i] * h[t, i] for i in range(5)) for o in range(2)]
        ang = float(t)  # theta_0 = 1 for the only pair
        assert kR[t, 0] == pytest.approx(x[0] * math.cos(ang) - x[1] * math.sin(ang), abs=1e-13)
        assert kR[t, 1] == pytest.approx(x[0] * math.sin(ang) + x[1] * math.cos(ang), abs=1e-13)


# ----------------------------------------------------------------------------- planted mistakes
def _mutant_attend(kind):
    def attend(q_C, q_R, pos_q, c_KV, k_R, W_UK, W_UV, base, scale):
        n_h, d_h = q_C.shape
        d_c = c_KV.shape[1]
        WUK = W_UK.reshape(n_h, d_h, d_c)
        WUV = W_UV.reshape(n_h, d_h, d_c)
        if kind == "head_interleave":          # head i taken as rows i, i+n_h, ...
            WUK = W_UK.reshape(d_h, n_h, d_c).transpose(1, 0, 2)
        q_rot = om.rope(q_R, pos_q, base)
        if kind == "rope_sign":
            q_rot = om.rope(q_R, -pos_q, base)   # rotation in the wrong sense
        if kind == "query_unrotated":
            q_rot = q_R
        s = np.einsum("hd,hdc->hc", q_C, WUK) @ c_KV.T
        if kind != "drop_rope_term":
            s = s + q_rot @ k_R.T
        if kind == "scale_dh_only":
            scale = 1.0 / math.sqrt(d_h)
        s = s * scale
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        z = p.sum(axis=1, keepdims=True)
        if kind == "no_normalise":
            z = np.ones_like(z)
        o = p / z @ c_KV
        return np.einsum("hdc,hc->hd", WUV, o), (m + np.log(z))[:, 0]
    return attend


@pytest.mark.parametrize("kind", ["head_interleave", "rope_sign", "query_unrotated", "drop_rope_term",
                                  "scale_dh_only", "no_normalise"])
def test_pins_catch_planted_mistakes(kind):
    P = _problem(np.random.default_rng(11), n_h=4, d_h=8, d_c=12, d_hR=6, d_model=20, n=9)
    good, _ = _oracle_run(P, _mutant_attend("none"))
    ref, _ = _torch_mha(P)
    assert _rel(good, ref) < 1e-12          # the unmutated copy passes the pin
    bad, _ = _oracle_run(P, _mutant_attend(kind))
    assert _rel(bad, ref) > 1e-6             # each planted mistake fails it


def test_pins_catch_wrong_key_position():
    P = _problem(np.random.default_rng(12))

    def down_off_by_one(h, W_DKV, W_KR, pos, base):
        return om.down_project(h, W_DKV, W_KR, np.asarray(pos) + 1, base)
    bad, _ = _oracle_run(P, down=down_off_by_one)
    ref, _ = _torch_mha(P)
    assert _rel(bad, ref) > 1e-6


# ----------------------------------------------------------------------------- query down-projection
def _with_lowrank_query(P, rng, d_cq, integer=False):
    """P with a query down-projection W^DQ [d_cq, d_model] and W^UQ [n_h*d_h, d_cq]."""
    d_model = P["h"].shape[1]
    if integer:
        f = lambda *s: rng.integers(-2, 3, size=s).astype(np.float64)  # noqa: E731
    else:
        f = lambda *s: rng.standard_normal(s) / math.sqrt(s[-1])       # noqa: E731
    Q = dict(P)
    Q["W_DQ"] = f(d_cq, d_model)
    Q["W_UQ"] = f(P["n_h"] * P["d_h"], d_cq)
    return Q


@pytest.mark.parametrize("seed,d_cq", [(20, 5), (21, 24), (22, 40)])
def test_lowrank_query_attention_matches_torch_sdpa(seed, d_cq):
    rng = np.random.default_rng(seed)
    P = _with_lowrank_query(_problem(rng, n_h=4, d_h=8, d_c=12, d_hR=6, d_model=20, n=9), rng, d_cq)
    out, lse = _oracle_run(P, oracle.attend_absorbed)
    ref, ref_lse = _torch_mha(P)
    assert _rel(out, ref) < 1e-12
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_lowrank_query_with_identity_down_projection_is_the_full_rank_query():
    rng = np.random.default_rng(23)
    h = rng.integers(-3, 4, size=(7, 16)).astype(np.float64)
    W_UQ = rng.integers(-2, 3, size=(4 * 8, 16)).astype(np.float64)
    W_QR = rng.integers(-2, 3, size=(4 * 6, 16)).astype(np.float64)
    a_C, a_R = oracle.query_project_lowrank(h, np.eye(16), W_UQ, W_QR, 4)
    for t in range(7):
        b_C, b_R = oracle.query_project(h[t], W_UQ, W_QR, 4)
        assert np.array_equal(a_C[t], b_C) and np.array_equal(a_R[t], b_R)


def test_lowrank_query_integer_product_matrix_bitwise():
    """Integer data: W^UQ (W^DQ h) and (W^UQ W^DQ) h are the same exact integers."""
    rng = np.random.default_rng(24)
    h = rng.integers(-3, 4, size=(5, 24)).astype(np.float64)
    W_DQ = rng.integers(-2, 3, size=(10, 24)).astype(np.float64)
    W_UQ = rng.integers(-2, 3, size=(3 * 8, 10)).astype(np.float64)
    W_QR = rng.integers(-2, 3, size=(3 * 4, 24)).astype(np.float64)
    q_C, q_R = oracle.query_project_lowrank(h, W_DQ, W_UQ, W_QR, 3)
    for t in range(5):
        for i in range(3):
            for d in range(8):
                r = i * 8 + d
                want = sum(sum(W_UQ[r, k] * W_DQ[k, j] for k in range(10)) * h[t, j] for j in range(24))
                assert q_C[t, i, d] == want
            for d in range(4):
                assert q_R[t, i, d] == sum(W_QR[i * 4 + d, j] * h[t, j] for j in range(24))


def test_lowrank_query_rank_bound_and_rope_input():
    """Every q^C lies in the d_cq-dimensional image of W^UQ (so 60 tokens give a
    rank-d_cq matrix), and q^R does not depend on W^DQ (it is fed from h)."""
    rng = np.random.default_rng(25)
    n_h, d_h, d_hR, d_model, d_cq = 4, 8, 6, 32, 5
    h = rng.standard_normal((60, d_model))
    W_DQ = rng.standard_normal((d_cq, d_model))
    W_UQ = rng.standard_normal((n_h * d_h, d_cq))
    W_QR = rng.standard_normal((n_h * d_hR, d_model))
    q_C, q_R = oracle.query_project_lowrank(h, W_DQ, W_UQ, W_QR, n_h)
    sv = np.linalg.svd(q_C.reshape(60, -1), compute_uv=False)
    assert sv[d_cq - 1] > 1e-6 * sv[0] and sv[d_cq] < 1e-10 * sv[0]
    _, q_R2 = oracle.query_project_lowrank(h, rng.standard_normal((d_cq, d_model)), W_UQ, W_QR, n_h)
    assert np.array_equal(q_R, q_R2)


def test_lowrank_query_head_layout():
    """Head i's q^C comes from rows i*d_h .. i*d_h + d_h - 1 of W^UQ only."""
    rng = np.random.default_rng(26)
    n_h, d_h, d_hR, d_model, d_cq = 4, 8, 6, 16, 6
    h = rng.standard_normal((3, d_model))
    W_UQ = np.zeros((n_h * d_h, d_cq))
    W_UQ[2 * d_h:3 * d_h] = rng.standard_normal((d_h, d_cq))
    W_QR = np.zeros((n_h * d_hR, d_model))
    W_QR[1 * d_hR:2 * d_hR] = rng.standard_normal((d_hR, d_model))
    q_C, q_R = oracle.query_project_lowrank(h, rng.standard_normal((d_cq, d_model)), W_UQ, W_QR, n_h)
    assert np.all(q_C[:, [0, 1, 3]] == 0) and np.all(q_C[:, 2] != 0)
    assert np.all(q_R[:, [0, 2, 3]] == 0) and np.all(q_R[:, 1] != 0)


# ----------------------------------------------------------------------------- output projection
def test_output_projection_selects_and_sums_heads():
    rng = np.random.default_rng(27)
    n_h, d_h = 5, 4
    o = rng.standard_normal((3, n_h, d_h))
    for i in range(n_h):                       # W^O = [0 .. I .. 0]: u = o_i exactly
        W_O = np.zeros((d_h, n_h * d_h))
        W_O[:, i * d_h:(i + 1) * d_h] = np.eye(d_h)
        assert np.array_equal(oracle.output_project(o, W_O), o[:, i])
    W_O = np.tile(np.eye(d_h), (1, n_h))       # [I I .. I]: u = sum_i o_i
    np.testing.assert_allclose(oracle.output_project(o, W_O), o.sum(axis=1), rtol=0, atol=1e-14)
    W_O = rng.standard_normal((7, n_h * d_h))  # d_model != n_h*d_h: u = sum_i W^O_i o_i
    u = oracle.output_project(o, W_O)
    assert u.shape == (3, 7)
    ref = sum(o[:, i] @ W_O[:, i * d_h:(i + 1) * d_h].T for i in range(n_h))
    np.testing.assert_allclose(u, ref, rtol=0, atol=1e-12)


def test_output_projection_absorbs_the_value_up_projection():
    """W^UV folded into W^O ([V2-arch] ch.2 §2): with W^O_i W^UV_i as the
    projection of head i's latent output O~_i (obtained with W^UV = I, d_h =
    d_c), u is the same as W^O applied to the o_i = W^UV_i O~_i."""
    rng = np.random.default_rng(28)
    n_h, d_c, d_hR, n, d_model = 3, 8, 4, 13, 11
    q_C = rng.standard_normal((n_h, d_c))
    q_R = rng.standard_normal((n_h, d_hR))
    c = rng.standard_normal((n, d_c))
    kR = rng.standard_normal((n, d_hR))
    W_UK = rng.standard_normal((n_h * d_c, d_c))
    W_UV = rng.standard_normal((n_h * d_c, d_c))
    W_O = rng.standard_normal((d_model, n_h * d_c))
    o, _ = oracle.attend_reconstruct(q_C, q_R, n - 1, c, kR, W_UK, W_UV, BASE, 0.3)
    o_lat, _ = oracle.attend_reconstruct(q_C, q_R, n - 1, c, kR, W_UK, np.tile(np.eye(d_c), (n_h, 1)), BASE, 0.3)
    W_abs = np.concatenate([W_O[:, i * d_c:(i + 1) * d_c] @ W_UV[i * d_c:(i + 1) * d_c] for i in range(n_h)], axis=1)
    np.testing.assert_allclose(oracle.output_project(o, W_O), oracle.output_project(o_lat, W_abs), rtol=1e-12,
                               atol=1e-12)


@pytest.mark.parametrize("kind", ["interleaved_concat", "transposed_head_block", "rope_from_latent_query"])
def test_projection_pins_catch_planted_mistakes(kind):
    rng = np.random.default_rng(29)
    if kind == "rope_from_latent_query":       # q^R = W^QR c^Q instead of W^QR h (d_cq = d_model)
        h = rng.standard_normal((60, 16))
        W_DQ, W_UQ, W_QR = (rng.standard_normal((16, 16)), rng.standard_normal((32, 16)),
                            rng.standard_normal((24, 16)))
        bad = lambda Wd: (h @ Wd.T) @ W_QR.T    # noqa: E731
        good = oracle.query_project_lowrank(h, W_DQ, W_UQ, W_QR, 4)[1].reshape(60, -1)
        assert np.array_equal(good, oracle.query_project_lowrank(h, 2 * W_DQ, W_UQ, W_QR, 4)[1].reshape(60, -1))
        assert not np.array_equal(bad(W_DQ), bad(2 * W_DQ))   # the rope-input pin fails it
        return
    n_h, d_h = 4, 4
    o = rng.standard_normal((2, n_h, d_h))
    if kind == "interleaved_concat":           # heads concatenated element-major
        proj = lambda o, W: o.transpose(0, 2, 1).reshape(o.shape[0], -1) @ W.T    # noqa: E731
    else:                                      # each head's d_h x d_h block used transposed
        proj = lambda o, W: sum(o[:, i] @ W[:, i * d_h:(i + 1) * d_h] for i in range(n_h))  # noqa: E731
    caught = False
    for i in range(n_h):
        W_O = np.zeros((d_h, n_h * d_h))
        W_O[:, i * d_h:(i + 1) * d_h] = rng.standard_normal((d_h, d_h)) if kind != "interleaved_concat" \
            else np.eye(d_h)
        assert np.allclose(oracle.output_project(o, W_O), o[:, i] @ W_O[:, i * d_h:(i + 1) * d_h].T)
        caught |= not np.allclose(proj(o, W_O), o[:, i] @ W_O[:, i * d_h:(i + 1) * d_h].T)
    assert caught


# ----------------------------------------------------------------------------- causal chunk (prefill)
def _torch_chunk(P, L):
    """The last T = n - L tokens as queries, each attending causally to all
    earlier tokens and itself, through torch SDPA with an explicit boolean
    mask over materialised per-head q, k, v (float64, CPU)."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    n_h, d_h, d_hR, n = P["n_h"], P["d_h"], P["d_hR"], P["n"]
    h = t(P["h"])
    pos = torch.arange(n, dtype=torch.float64)

    def rot(x, p):
        d = x.shape[-1]
        theta = BASE ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
        z = torch.view_as_complex(x.reshape(*x.shape[:-1], d // 2, 2).contiguous())
        z = z * torch.polar(torch.ones_like(theta), p[..., None] * theta)
        return torch.view_as_real(z).reshape(x.shape)

    c = h @ t(P["W_DKV"]).T
    kC = torch.einsum("hdc,nc->hnd", t(P["W_UK"]).reshape(n_h, d_h, -1), c)
    v = torch.einsum("hdc,nc->hnd", t(P["W_UV"]).reshape(n_h, d_h, -1), c)
    kR = rot(h @ t(P["W_KR"]).T, pos)
    k = torch.cat([kC, kR.unsqueeze(0).expand(n_h, n, d_hR)], dim=-1)
    hq = h[L:]
    qC = (hq @ t(P["W_UQ"]).T).reshape(-1, n_h, d_h).transpose(0, 1)
    qR = rot((hq @ t(P["W_QR"]).T).reshape(-1, n_h, d_hR), pos[L:, None].expand(-1, n_h)).transpose(0, 1)
    q = torch.cat([qC, qR], dim=-1)                                    # [n_h, T, E]
    mask = torch.arange(n)[None, :] <= torch.arange(L, n)[:, None]     # [T, n]: key j visible to query i
    out = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask)[0]
    return out.transpose(0, 1).numpy()                                 # [T, n_h, d_h]


@pytest.mark.parametrize("reconstruct", [False, True])
def test_causal_chunk_matches_torch_sdpa_with_a_causal_mask(reconstruct):
    P = _problem(np.random.default_rng(30), n_h=3, d_h=8, d_c=12, d_hR=6, d_model=20, n=14)
    L = 9
    n = P["n"]
    c, kR = oracle.down_project(P["h"], P["W_DKV"], P["W_KR"], np.arange(n), BASE)
    qs = [oracle.query_project(P["h"][i], P["W_UQ"], P["W_QR"], P["n_h"]) for i in range(L, n)]
    q_C, q_R = np.stack([a for a, _ in qs]), np.stack([b for _, b in qs])
    out, lse = oracle.attend_causal_chunk(q_C, q_R, np.arange(L, n), c, kR, P["W_UK"], P["W_UV"], BASE,
                                          oracle.softmax_scale(P["d_h"], P["d_hR"]), reconstruct=reconstruct)
    assert out.shape == (n - L, P["n_h"], P["d_h"]) and lse.shape == (n - L, P["n_h"])
    assert _rel(out, _torch_chunk(P, L)) < 1e-12


def test_causal_chunk_has_no_future_leak():
    """Rows after a token's position never change its output; its output is
    the single-token decode over its own prefix."""
    rng = np.random.default_rng(31)
    n_h, d_h, d_c, d_hR, n, T = 4, 16, 32, 8, 20, 6
    q_C, q_R = rng.standard_normal((T, n_h, d_h)), rng.standard_normal((T, n_h, d_hR))
    c, kR = rng.standard_normal((n, d_c)), rng.standard_normal((n, d_hR))
    W_UK, W_UV = rng.standard_normal((n_h * d_h, d_c)), rng.standard_normal((n_h * d_h, d_c))
    pos = np.arange(n - T, n)
    a, la = oracle.attend_causal_chunk(q_C, q_R, pos, c, kR, W_UK, W_UV, BASE, 0.2)
    c2, kR2 = c.copy(), kR.copy()
    c2[n - 2:] += 5.0
    kR2[n - 2:] -= 3.0
    b, lb = oracle.attend_causal_chunk(q_C, q_R, pos, c2, kR2, W_UK, W_UV, BASE, 0.2)
    assert np.array_equal(a[:T - 2], b[:T - 2]) and np.array_equal(la[:T - 2], lb[:T - 2])
    assert _rel(b[T - 1], a[T - 1]) > 1e-3                  # the last tokens do see the changed rows
    o, l = oracle.attend_absorbed(q_C[2], q_R[2], pos[2], c[:pos[2] + 1], kR[:pos[2] + 1], W_UK, W_UV, BASE, 0.2)
    assert np.array_equal(o, a[2]) and np.array_equal(l, la[2])
