"""Pins of the oracle's sparse top-k decode to facts fixed outside itself
(reading of DeepSeek architecture V3 to V4 (cyco.top), §4 V3.2 bullet and §6
question 7: an indexer picks the few most relevant cached tokens, attention
then runs over those alone).

* the indexer score on unit-vector keys, where it reduces to reading the
  query's coordinates, and against plain Python loops on tiny integer data;
* the selection against its defining order property and against a brute
  force over all k-subsets of tiny inputs;
* the whole sparse decode against the dense absorbed attention (already
  pinned in test_oracle_pins.py) when every token is kept, and when the
  dropped tokens' scores are so low that their softmax weight underflows;
* closed forms when all kept rows are the same row (O~ = c, lse = s + log k).

The last test plants typical mistakes in copies of the functions and checks
that these pins catch each of them.
"""
import itertools

import numpy as np
import pytest

import oracle

BASE = 10000.0


# ----------------------------------------------------------------------------- checks (take the functions under test)
def check_indexer_basis(indexer):
    """Keys = unit vectors e_0 .. e_{d-1}: I_j = sum_h w_h max(q_h[j], 0)."""
    rng = np.random.default_rng(7)
    H, d = 5, 6
    q = rng.integers(-4, 5, size=(H, d)).astype(np.float64)
    w = rng.integers(-3, 4, size=H).astype(np.float64)
    got = indexer(q, w, np.eye(d))
    for j in range(d):
        want = 0.0
        for h in range(H):
            if q[h, j] > 0:
                want += w[h] * q[h, j]
        if got[j] != want:
            return False
    return True


def check_indexer_loops(indexer):
    """Plain loops on tiny integer data (exact in fp64)."""
    rng = np.random.default_rng(11)
    H, d, n = 3, 4, 9
    q = rng.integers(-3, 4, size=(H, d)).astype(np.float64)
    w = rng.integers(-2, 3, size=H).astype(np.float64)
    k = rng.integers(-3, 4, size=(n, d)).astype(np.float64)
    got = indexer(q, w, k)
    for j in range(n):
        tot = 0.0
        for h in range(H):
            dot = 0.0
            for c in range(d):
                dot += q[h, c] * k[j, c]
            if dot > 0:
                tot += w[h] * dot
        if got[j] != tot:
            return False
    return True


def check_topk_order_property(topk):
    """|S| = min(k, n), ascending, and every kept j beats every dropped i:
    s_j > s_i, or s_j == s_i and j < i."""
    rng = np.random.default_rng(3)
    for trial in range(40):
        n = int(rng.integers(1, 40))
        s = rng.integers(-3, 4, size=n).astype(np.float64)   # many ties
        for k in (1, 2, 5, 17, 64):
            S = np.asarray(topk(s, k))
            if len(S) != min(k, n) or np.any(np.diff(S) <= 0):
                return False
            kept = set(S.tolist())
            for j in kept:
                for i in range(n):
                    if i in kept:
                        continue
                    if not (s[j] > s[i] or (s[j] == s[i] and j < i)):
                        return False
    return True


def check_topk_brute(topk):
    """All k-subsets of n <= 7 tokens: the kept set is the one whose scores,
    sorted descending, are largest, ties settled toward smaller indices."""
    rng = np.random.default_rng(5)
    for trial in range(30):
        n = int(rng.integers(1, 8))
        s = rng.integers(0, 3, size=n).astype(np.float64)
        for k in range(1, n + 1):
            best = None
            for sub in itertools.combinations(range(n), k):
                key = (sorted((-s[j] for j in sub)), list(sub))
                if best is None or key < best[0]:
                    best = (key, sub)
            if list(topk(s, k)) != list(best[1]):
                return False
    return True


def _case(rng, n_h=4, d_h=8, d_c=16, d_hR=4, n=24, H_I=3, d_I=8):
    return dict(q_C=rng.standard_normal((n_h, d_h)), q_R=rng.standard_normal((n_h, d_hR)), pos_q=n - 1,
                c_KV=rng.standard_normal((n, d_c)), k_R=rng.standard_normal((n, d_hR)),
                W_UK=rng.standard_normal((n_h * d_h, d_c)) / 4, W_UV=rng.standard_normal((n_h * d_h, d_c)) / 4,
                q_I=rng.standard_normal((H_I, d_I)), w_I=rng.random(H_I), k_I=rng.standard_normal((n, d_I)))


def check_all_kept_is_dense(sparse):
    rng = np.random.default_rng(2)
    P = _case(rng)
    n = P["c_KV"].shape[0]
    for k in (n, n + 5):
        out, lse, sel = sparse(P["q_C"], P["q_R"], P["pos_q"], P["c_KV"], P["k_R"], P["W_UK"], P["W_UV"], BASE, 0.3,
                               P["q_I"], P["w_I"], P["k_I"], k)
        d_out, d_lse = oracle.attend_absorbed(P["q_C"], P["q_R"], P["pos_q"], P["c_KV"], P["k_R"], P["W_UK"],
                                              P["W_UV"], BASE, 0.3)
        if list(sel) != list(range(n)) or np.max(np.abs(out - d_out)) > 1e-12 or np.max(np.abs(lse - d_lse)) > 1e-12:
            return False
    return True


def check_dropped_tokens_vanish(sparse):
    """One head.  The indexer keeps tokens 0..k-1 (their keys point along the
    indexer query); the other tokens' latents point against q~ so far that
    exp underflows: the dense attention over all tokens then equals the
    sparse one over the kept tokens."""
    rng = np.random.default_rng(9)
    d_h, d_c, d_hR, n, k, d_I = 8, 16, 4, 20, 7, 8
    q_C = rng.standard_normal((1, d_h))
    q_R = np.zeros((1, d_hR))
    W_UK = rng.standard_normal((d_h, d_c))
    W_UV = rng.standard_normal((d_h, d_c))
    q_abs = q_C[0] @ W_UK                       # q~ of the one head
    c_KV = rng.standard_normal((n, d_c))
    c_KV[k:] = -1e4 * q_abs / np.dot(q_abs, q_abs)
    k_R = rng.standard_normal((n, d_hR))
    q_I = np.ones((1, d_I))
    w_I = np.ones(1)
    k_I = -np.ones((n, d_I))
    k_I[:k] = np.arange(1, k + 1)[:, None]      # kept tokens score 8, 16, ...; dropped ones 0
    out, lse, sel = sparse(q_C, q_R, n - 1, c_KV, k_R, W_UK, W_UV, BASE, 1.0, q_I, w_I, k_I, k)
    d_out, d_lse = oracle.attend_absorbed(q_C, q_R, n - 1, c_KV, k_R, W_UK, W_UV, BASE, 1.0)
    return list(sel) == list(range(k)) and np.max(np.abs(out - d_out)) <= 1e-12 * np.max(np.abs(d_out)) \
        and np.max(np.abs(lse - d_lse)) <= 1e-12


def check_identical_kept_rows(sparse):
    """The indexer keeps the odd tokens, whose cached rows are all the same
    [c ; k^R]; the even tokens hold other rows.  Every kept score is then the
    same s, so each head's weights are 1/|S| and O~_i = c: out_i = W^UV_i c
    and lse_i = s_i + log |S| (closed forms)."""
    rng = np.random.default_rng(4)
    n_h, d_h, d_c, d_hR, n, d_I = 3, 8, 16, 4, 21, 6
    q_C = rng.standard_normal((n_h, d_h))
    q_R = rng.standard_normal((n_h, d_hR))
    W_UK = rng.standard_normal((n_h * d_h, d_c)) / 4
    W_UV = rng.standard_normal((n_h * d_h, d_c)) / 4
    c, kr = rng.standard_normal(d_c), rng.standard_normal(d_hR)
    c_KV = rng.standard_normal((n, d_c))
    k_R = rng.standard_normal((n, d_hR))
    c_KV[1::2] = c
    k_R[1::2] = kr
    q_I = rng.standard_normal((2, d_I))
    w_I = np.array([1.0, 0.5])
    k_I = np.zeros((n, d_I))
    k_I[1::2] = q_I[0] + q_I[1]                 # odd tokens: a positive dot on both heads (this draw)
    k = (n - 1) // 2
    assert np.all(q_I @ (q_I[0] + q_I[1]) > 0)   # the seeded draw makes the case
    out, lse, sel = sparse(q_C, q_R, n - 1, c_KV, k_R, W_UK, W_UV, BASE, 0.4, q_I, w_I, k_I, k)
    q_abs = np.einsum("hd,hdc->hc", q_C, W_UK.reshape(n_h, d_h, d_c))
    s_i = (q_abs @ c + oracle.rope(q_R, n - 1, BASE) @ kr) * 0.4
    want_out = np.einsum("hdc,c->hd", W_UV.reshape(n_h, d_h, d_c), c)
    want_lse = s_i + np.log(k)
    return list(sel) == list(range(1, n, 2)) and np.max(np.abs(out - want_out)) <= 1e-12 * np.max(np.abs(want_out)) \
        and np.max(np.abs(lse - want_lse)) <= 1e-12 * max(1.0, np.max(np.abs(want_lse)))


# ----------------------------------------------------------------------------- the pins
def test_indexer_unit_keys():
    assert check_indexer_basis(oracle.indexer_scores)


def test_indexer_loops():
    assert check_indexer_loops(oracle.indexer_scores)


def test_topk_order_property():
    assert check_topk_order_property(oracle.topk_select)


def test_topk_brute_force():
    assert check_topk_brute(oracle.topk_select)


def test_sparse_all_kept_is_dense():
    assert check_all_kept_is_dense(oracle.sparse_decode)


def test_sparse_dropped_tokens_vanish():
    assert check_dropped_tokens_vanish(oracle.sparse_decode)


def test_sparse_identical_kept_rows():
    assert check_identical_kept_rows(oracle.sparse_decode)


# ----------------------------------------------------------------------------- planted mistakes
def _idx_no_relu(q, w, k):
    return (np.asarray(w)[:, None] * (np.asarray(q, float) @ np.asarray(k, float).T)).sum(0)


def _idx_no_weights(q, w, k):
    return np.maximum(np.asarray(q, float) @ np.asarray(k, float).T, 0).sum(0)


def _idx_relu_after_weight(q, w, k):
    return np.maximum(np.asarray(w)[:, None] * (np.asarray(q, float) @ np.asarray(k, float).T), 0).sum(0)


def _top_ties_high(s, k):
    s = np.asarray(s)
    n = len(s)
    if n <= k:
        return np.arange(n)
    return np.array(sorted(sorted(range(n), key=lambda j: (-s[j], -j))[:k]))


def _top_smallest(s, k):
    s = np.asarray(s)
    n = len(s)
    if n <= k:
        return np.arange(n)
    return np.array(sorted(sorted(range(n), key=lambda j: (s[j], j))[:k]))


def _top_off_by_one(s, k):
    return oracle.topk_select(s, max(k - 1, 1))


def _sparse_with(topk=None, attend=None):
    def f(q_C, q_R, pos_q, c_KV, k_R, W_UK, W_UV, base, scale, q_I, w_I, k_I, k):
        sel = (topk or oracle.topk_select)(oracle.indexer_scores(q_I, w_I, k_I), k)
        out, lse = (attend or oracle.attend_sparse)(q_C, q_R, pos_q, c_KV, k_R, W_UK, W_UV, base, scale, sel)
        return out, lse, sel
    return f


def _attend_all_rows(q_C, q_R, pos_q, c_KV, k_R, W_UK, W_UV, base, scale, sel):
    return oracle.attend_absorbed(q_C, q_R, pos_q, c_KV, k_R, W_UK, W_UV, base, scale)


def _attend_first_rows(q_C, q_R, pos_q, c_KV, k_R, W_UK, W_UV, base, scale, sel):
    m = len(sel)
    return oracle.attend_absorbed(q_C, q_R, pos_q, np.asarray(c_KV)[:m], np.asarray(k_R)[:m], W_UK, W_UV, base, scale)


@pytest.mark.parametrize("fn", [_idx_no_relu, _idx_no_weights, _idx_relu_after_weight])
def test_pins_catch_indexer_mistakes(fn):
    assert check_indexer_basis(oracle.indexer_scores) and check_indexer_loops(oracle.indexer_scores)
    assert not (check_indexer_basis(fn) and check_indexer_loops(fn))


@pytest.mark.parametrize("fn", [_top_ties_high, _top_smallest, _top_off_by_one])
def test_pins_catch_selection_mistakes(fn):
    assert not (check_topk_order_property(fn) and check_topk_brute(fn))


@pytest.mark.parametrize("attend", [_attend_all_rows, _attend_first_rows])
def test_pins_catch_sparse_attention_mistakes(attend):
    f = _sparse_with(attend=attend)
    assert not (check_all_kept_is_dense(f) and check_dropped_tokens_vanish(f) and check_identical_kept_rows(f))
