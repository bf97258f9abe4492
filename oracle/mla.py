"""Plain fp64 CPU oracle for Multi-head Latent Attention (MLA) decode over the
compressed latent KV cache.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The GPU
library never routes through it and shares no code with it.

Sources (web pages on DeepSeek-V2 MLA; citations name the page and its section):

* [V2-arch]  "DeepSeek-V2：在“大力出奇迹”的AI军备竞赛中，四两拨千斤" (liang.world),
  chapter 2 "侠客甲——MLA": §1 MHA baseline, §2 low-rank joint KV compression,
  §3 decoupled RoPE.
* [DS-report] "DeepSeek 系列模型技术深度解读" (tuntang.top), section
  "Multi-head Latent Attention (MLA)": KV-cache formula, "MLA 的核心思想",
  "RoPE 的兼容性处理" (q_t / k_t concatenation formula).
* [pptc-note] DeepSeek MoE/MLA engineering note (pptc.cn): §3.4 cache layout,
  §6 pitfall 2 (k_rope must be cached beside the latent).

Readings where the pages are silent (each is listed in the design notes):

* RoPE: RoFormer's rotation of adjacent pairs (x_{2k}, x_{2k+1}) by the angle
  pos * base^(-2k/d_h^R), base 10000; angles in fp64.
* Softmax scale 1/sqrt(d_h + d_h^R) (the concatenated q/k width).
* Positions: cached token j sits at position j; the decode query of a sequence
  holding n cached tokens (itself included, it was appended first) is at
  position n - 1 and attends to all n tokens (causal j <= t).
* Weights are stored [out, in] row-major: W^DKV [d_c, d_model],
  W^KR [d_h^R, d_model], W^UK and W^UV [n_h*d_h, d_c] with head i owning rows
  i*d_h .. i*d_h + d_h - 1, W^UQ [n_h*d_h, d_model], W^QR [n_h*d_h^R, d_model].
* Query path, two forms.  Without a query down-projection (c^Q := h):
  q^C = W^UQ h and q^R = W^QR h (``query_project``).  With the query's own
  low-rank compression (``query_project_lowrank``): c^Q = W^DQ h, by analogy
  with c^KV = W^DKV h (the pages name c^Q but print no formula for it), its
  rank d_cq a free parameter (the pages give no value); q^C = W^UQ c^Q; and
  q^R = W^QR h, fed from h_t as [DS-report] writes it.  Both return q^R not
  yet rotated (the decode rotates it at the query position).
* The output projection W^O [d_model, n_h*d_h] acts on the heads' outputs
  concatenated in head order (``output_project``); the decode attention itself
  returns each head's o_i.
* Sparse top-k decode ([V3-V4] "DeepSeek 架构精讲：从 V3 到 V4" (cyco.top),
  §4 V3.2 bullet and §6 self-test question 7): the pages say only that a
  light "indexer" first picks the few most relevant cached tokens and the
  attention then looks at those alone.  Reading taken: every cached token j
  carries a small indexer key k^I_j (d_I wide); a decode query carries H_I
  indexer heads q^I_h and head weights w_h; the token's relevance is
  I_j = sum_h w_h * max(0, q^I_h . k^I_j) (``indexer_scores``); the k tokens
  of largest I_j are kept, equal scores going to the smaller token index
  (``topk_select``; all tokens when n <= k); the MLA decode attention then
  runs over the kept rows only (``attend_sparse``).  How k^I, q^I and w are
  produced is outside the pages and outside this function set: they are
  inputs.

Everything is numpy float64; matrix products are numpy ``@``.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# Cache-size arithmetic ([V2-arch] ch.2 §1 and §2; [DS-report] MLA section)
# ----------------------------------------------------------------------------


def mha_cache_elements_per_token(n_h: int, d_h: int) -> int:
    """Standard MHA caches k and v for every head: 2 * n_h * d_h elements per
    token per layer ([V2-arch] ch.2 §1; [DS-report] "标准 MHA 的瓶颈")."""
    return 2 * n_h * d_h


def mla_cache_elements_per_token(d_c: int, d_hR: int) -> int:
    """MLA caches the latent c^KV (d_c) plus the one shared RoPE key k^R
    (d_h^R) per token per layer ([V2-arch] ch.2 §2; [DS-report] MLA vs GQA
    table, row "KV Cache/token")."""
    return d_c + d_hR


def gqa_equivalent_groups(d_c: int, d_hR: int, d_h: int) -> float:
    """Number of GQA groups n_g whose cache 2 * n_g * d_h equals MLA's
    ([V2-arch] ch.2 §3, closing paragraph)."""
    return mla_cache_elements_per_token(d_c, d_hR) / (2.0 * d_h)


# ----------------------------------------------------------------------------
# RoPE ([V2-arch] ch.2 §3; rotation convention: RoFormer adjacent pairs)
# ----------------------------------------------------------------------------


def rope_angles(pos, d_hR: int, base: float) -> np.ndarray:
    """Angles pos * base^(-2k/d_hR), k = 0 .. d_hR/2 - 1, in fp64.
    ``pos`` may be a scalar or a 1-D array; the result has shape [..., d_hR/2]."""
    k = np.arange(d_hR // 2, dtype=np.float64)
    theta = np.power(np.float64(base), -2.0 * k / d_hR)
    return np.multiply.outer(np.asarray(pos, dtype=np.float64), theta)


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate each adjacent pair (x[2k], x[2k+1]) of the last axis by angle
    pos * base^(-2k/d).  ``pos`` broadcasts against x's leading axes."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = rope_angles(pos, d, base)
    cos, sin = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * cos - xo * sin
    out[..., 1::2] = xe * sin + xo * cos
    return out


# ----------------------------------------------------------------------------
# Cache append: c^KV = W^DKV h, k^R = RoPE(W^KR h)
# ([V2-arch] ch.2 §2 eq. for c_t^KV; [DS-report] "RoPE 的兼容性处理" eq. for k_t)
# ----------------------------------------------------------------------------


def down_project(h: np.ndarray, W_DKV: np.ndarray, W_KR: np.ndarray, pos, base: float):
    """Cache rows for tokens h [n, d_model] at positions ``pos`` [n]:
    returns (c_KV [n, d_c], k_R [n, d_hR]) with k_R already rotated."""
    h = np.asarray(h, dtype=np.float64)
    c_KV = h @ np.asarray(W_DKV, dtype=np.float64).T              # c_t^KV = W^DKV h_t
    k_R = _rope_rows(h @ np.asarray(W_KR, dtype=np.float64).T, pos, base)  # k_t^R = RoPE(W^KR h_t)
    return c_KV, k_R


def _rope_rows(x: np.ndarray, pos, base: float) -> np.ndarray:
    """RoPE applied row by row: row r of x at position pos[r] (or one scalar)."""
    if np.ndim(pos) == 0:
        return rope(x, pos, base)
    out = np.empty_like(x)
    for r, p in enumerate(np.asarray(pos)):
        out[r] = rope(x[r], p, base)
    return out


def query_project(h_q: np.ndarray, W_UQ: np.ndarray, W_QR: np.ndarray, n_h: int):
    """Query of one token with c^Q := h: q^C = W^UQ h split per head [n_h, d_h],
    q^R = W^QR h split per head [n_h, d_hR] and NOT yet rotated
    ([DS-report] "RoPE 的兼容性处理" eq. for q_t)."""
    h_q = np.asarray(h_q, dtype=np.float64)
    q_C = (np.asarray(W_UQ, dtype=np.float64) @ h_q).reshape(n_h, -1)
    q_R = (np.asarray(W_QR, dtype=np.float64) @ h_q).reshape(n_h, -1)
    return q_C, q_R


def query_project_lowrank(h_q: np.ndarray, W_DQ: np.ndarray, W_UQ: np.ndarray, W_QR: np.ndarray, n_h: int):
    """Queries of tokens h_q [..., d_model] through the query's low-rank
    compression ([V2-arch] ch.2 §2, closing paragraph: q is compressed to c^Q
    as the keys and values are to c^KV; [DS-report] "RoPE 的兼容性处理": q_t =
    [W^UQ c_t^Q ; W^QR h_t RoPE(t)]):
        c^Q = W^DQ h              W_DQ [d_cq, d_model]
        q^C = W^UQ c^Q            W_UQ [n_h*d_h, d_cq], head i = rows i*d_h ..
        q^R = W^QR h              W_QR [n_h*d_hR, d_model], NOT yet rotated
    Returns q_C [..., n_h, d_h] and q_R [..., n_h, d_hR]."""
    h_q = np.asarray(h_q, dtype=np.float64)
    c_Q = h_q @ np.asarray(W_DQ, dtype=np.float64).T                 # c^Q = W^DQ h
    q_C = c_Q @ np.asarray(W_UQ, dtype=np.float64).T                 # q^C = W^UQ c^Q
    q_R = h_q @ np.asarray(W_QR, dtype=np.float64).T                 # q^R = W^QR h
    lead = h_q.shape[:-1]
    return q_C.reshape(*lead, n_h, -1), q_R.reshape(*lead, n_h, -1)


def output_project(o: np.ndarray, W_O: np.ndarray) -> np.ndarray:
    """u = W^O [o_1; o_2; ...; o_{n_h}] for per-head outputs o [..., n_h, d_h]
    ([V2-arch] ch.2 §1, "输出": the heads' results are concatenated and passed
    through the output matrix W_O).  W_O [d_model, n_h*d_h]; returns
    u [..., d_model]."""
    o = np.asarray(o, dtype=np.float64)
    cat = o.reshape(*o.shape[:-2], o.shape[-2] * o.shape[-1])        # heads concatenated in order
    return cat @ np.asarray(W_O, dtype=np.float64).T


# ----------------------------------------------------------------------------
# Decode attention of one query token, the definition: rebuild K and V
# ([V2-arch] ch.2 §1 (per-head softmax attention), §2 (k^C = W^UK c,
# v^C = W^UV c), §3 (q = [q^C; q^R], k = [k^C; k^R]))
# ----------------------------------------------------------------------------


def attend_reconstruct(q_C, q_R, pos_q, c_KV, k_R, W_UK, W_UV, base: float, scale: float,
                       heads=None, return_probs: bool = False):
    """One decode query against n cached tokens, rebuilding per-head keys and
    values from the latent.

    q_C [n_h, d_h], q_R [n_h, d_hR] (un-rotated; rotated here at pos_q),
    c_KV [n, d_c], k_R [n, d_hR] (already rotated), W_UK/W_UV [n_h*d_h, d_c].
    Returns out [len(heads), d_h], lse [len(heads)] (natural log of the softmax
    denominator of the scaled scores) and optionally P [len(heads), n]."""
    q_C = np.asarray(q_C, dtype=np.float64)
    q_R = np.asarray(q_R, dtype=np.float64)
    c_KV = np.asarray(c_KV, dtype=np.float64)
    k_R = np.asarray(k_R, dtype=np.float64)
    W_UK = np.asarray(W_UK, dtype=np.float64)
    W_UV = np.asarray(W_UV, dtype=np.float64)
    n_h, d_h = q_C.shape
    heads = range(n_h) if heads is None else heads
    outs, lses, probs = [], [], []
    for i in heads:
        W_UK_i = W_UK[i * d_h:(i + 1) * d_h]          # [d_h, d_c]
        W_UV_i = W_UV[i * d_h:(i + 1) * d_h]
        k_C = c_KV @ W_UK_i.T                          # k^C_{j,i} = W^UK_i c_j  -> [n, d_h]
        v = c_KV @ W_UV_i.T                            # v^C_{j,i} = W^UV_i c_j  -> [n, d_h]
        k = np.concatenate([k_C, k_R], axis=1)         # k_{j,i} = [k^C_{j,i}; k^R_j]
        q = np.concatenate([q_C[i], rope(q_R[i], pos_q, base)])  # q_i = [q^C_i; q^R_i]
        s = (k @ q) * scale                            # scores over all cached tokens
        m = s.max()
        e = np.exp(s - m)
        z = e.sum()
        p = e / z
        outs.append(p @ v)
        lses.append(m + np.log(z))
        probs.append(p)
    out = np.stack(outs)
    lse = np.array(lses)
    if return_probs:
        return out, lse, np.stack(probs)
    return out, lse


# ----------------------------------------------------------------------------
# Decode attention with the up-projections absorbed ([V2-arch] ch.2 §2,
# paragraph on absorbing W^UK into the query side and W^UV into the output side)
# ----------------------------------------------------------------------------


def attend_absorbed(q_C, q_R, pos_q, c_KV, k_R, W_UK, W_UV, base: float, scale: float,
                    return_probs: bool = False):
    """Same result as ``attend_reconstruct`` by associativity:
    q~_i = W^UK_i^T q^C_i, s_j = q~_i . c_j + RoPE(q^R_i) . k^R_j,
    O~_i = sum_j p_j c_j, o_i = W^UV_i O~_i.  All heads at once."""
    q_C = np.asarray(q_C, dtype=np.float64)
    q_R = np.asarray(q_R, dtype=np.float64)
    c_KV = np.asarray(c_KV, dtype=np.float64)
    k_R = np.asarray(k_R, dtype=np.float64)
    n_h, d_h = q_C.shape
    d_c = c_KV.shape[1]
    W_UK = np.asarray(W_UK, dtype=np.float64).reshape(n_h, d_h, d_c)
    W_UV = np.asarray(W_UV, dtype=np.float64).reshape(n_h, d_h, d_c)
    q_abs = np.einsum("hd,hdc->hc", q_C, W_UK)        # q~_i = W^UK_i^T q^C_i  [n_h, d_c]
    q_rot = rope(q_R, pos_q, base)                     # [n_h, d_hR]
    s = (q_abs @ c_KV.T + q_rot @ k_R.T) * scale       # [n_h, n]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    o_lat = p @ c_KV                                   # O~_i  [n_h, d_c]
    out = np.einsum("hdc,hc->hd", W_UV, o_lat)         # o_i = W^UV_i O~_i
    lse = (m + np.log(z))[:, 0]
    if return_probs:
        return out, lse, p
    return out, lse


def attend_causal_chunk(q_C, q_R, pos, c_KV, k_R, W_UK, W_UV, base: float, scale: float, reconstruct: bool = False):
    """A chunk of new tokens of one sequence, each attending causally: token t
    (query q_C[t], q_R[t] at position pos[t]) attends to cached rows
    0 .. pos[t] of the sequence, earlier tokens of the same chunk included
    ([V2-arch] ch.2 §1: each token attends to the tokens before it and itself).
    c_KV [n, d_c], k_R [n, d_hR] hold every row up to max(pos); returns
    out [T, n_h, d_h], lse [T, n_h]."""
    attend = attend_reconstruct if reconstruct else attend_absorbed
    outs, lses = [], []
    for t, p in enumerate(np.asarray(pos)):
        o, l = attend(q_C[t], q_R[t], p, c_KV[:p + 1], k_R[:p + 1], W_UK, W_UV, base, scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def softmax_scale(d_h: int, d_hR: int) -> float:
    """1/sqrt(d_h + d_h^R): q and k are the concatenations of width d_h + d_h^R."""
    return 1.0 / np.sqrt(d_h + d_hR)


# ----------------------------------------------------------------------------
# Sparse top-k decode ([V3-V4] §4 V3.2 bullet, §6 question 7)
# ----------------------------------------------------------------------------


def indexer_scores(q_I, w_I, k_I) -> np.ndarray:
    """Relevance of each cached token to one decode query:
    I_j = sum_h w_h * max(0, q^I_h . k^I_j).
    q_I [H_I, d_I], w_I [H_I], k_I [n, d_I]; returns [n] (fp64)."""
    q_I = np.asarray(q_I, dtype=np.float64)
    w_I = np.asarray(w_I, dtype=np.float64)
    k_I = np.asarray(k_I, dtype=np.float64)
    dots = q_I @ k_I.T                                  # [H_I, n]: q^I_h . k^I_j
    return (w_I[:, None] * np.maximum(dots, 0.0)).sum(axis=0)


def topk_select(scores, k: int) -> np.ndarray:
    """Indices (ascending) of the k largest scores; between equal scores the
    smaller index is kept first.  All indices when len(scores) <= k."""
    scores = np.asarray(scores)
    n = scores.shape[0]
    if n <= k:
        return np.arange(n, dtype=np.int64)
    order = sorted(range(n), key=lambda j: (-scores[j], j))   # largest first, then smaller index
    return np.array(sorted(order[:k]), dtype=np.int64)


def attend_sparse(q_C, q_R, pos_q, c_KV, k_R, W_UK, W_UV, base: float, scale: float, sel):
    """The absorbed MLA decode over the kept rows only: the softmax runs over
    j in sel, O~_i = sum_{j in sel} p_j c_j, o_i = W^UV_i O~_i."""
    sel = np.asarray(sel, dtype=np.int64)
    c_KV = np.asarray(c_KV)
    k_R = np.asarray(k_R)
    return attend_absorbed(q_C, q_R, pos_q, c_KV[sel], k_R[sel], W_UK, W_UV, base, scale)


def sparse_decode(q_C, q_R, pos_q, c_KV, k_R, W_UK, W_UV, base: float, scale: float, q_I, w_I, k_I, k: int):
    """Indexer scores, top-k selection, attention over the kept rows.
    Returns (out [n_h, d_h], lse [n_h], sel)."""
    sel = topk_select(indexer_scores(q_I, w_I, k_I), k)
    out, lse = attend_sparse(q_C, q_R, pos_q, c_KV, k_R, W_UK, W_UV, base, scale, sel)
    return out, lse, sel
