"""Host-side checks of the C ABI that run without a GPU: the library loads,
exports every function include/mla.h declares, and rejects bad arguments
with the documented status before launching anything; plus the work-split
arithmetic the kernels share (slot = split + sequence)."""
import ctypes
import os
import re

import numpy as np
import pytest

import compressed_kv_cache_mla_amd as mla

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mla.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared()
    assert set(names) >= {"mla_cache_append", "mla_decode", "mla_decode_workspace_size"}
    L = mla.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(mla.EXPORTED) == set(names)


def _dims(**kw):
    d = dict(n_h=128, d_h=128, d_c=512, d_hR=64, d_model=5120, page_size=64, softmax_scale=192 ** -0.5,
             rope_base=10000.0, dtype=mla.MLA_BF16)
    d.update(kw)
    return mla.mla_dims(**{k: d[k] for k, _ in mla.mla_dims._fields_})


def _decode(dims, ws_bytes=1 << 30, ptr=16, B=2, n_splits=8, stride=576):
    L = mla.lib()
    p = ctypes.c_void_p(ptr * 4096) if ptr else None
    return L.mla_decode(ctypes.byref(dims) if dims is not None else None, B, p, p, p, p, p, p, p, stride, 10, p, 4,
                        p, p, None, ctypes.c_void_p(1 << 20), ws_bytes, n_splits, None)


def test_decode_rejects_bad_arguments_before_launching():
    L = mla.lib()
    assert _decode(None) == mla.MLA_ERR_INVALID_ARG
    assert b"dims" in L.mla_last_error()
    assert _decode(_dims(d_c=256)) == mla.MLA_ERR_UNSUPPORTED
    assert _decode(_dims(d_hR=32)) == mla.MLA_ERR_UNSUPPORTED
    assert _decode(_dims(d_h=64)) == mla.MLA_ERR_UNSUPPORTED
    assert _decode(_dims(d_model=100)) == mla.MLA_ERR_UNSUPPORTED
    assert _decode(_dims(page_size=0)) == mla.MLA_ERR_INVALID_ARG
    assert _decode(_dims(dtype=7)) == mla.MLA_ERR_INVALID_ARG
    assert _decode(_dims(), B=0) == mla.MLA_ERR_INVALID_ARG
    assert _decode(_dims(), ptr=0) == mla.MLA_ERR_INVALID_ARG
    assert _decode(_dims(), stride=500) == mla.MLA_ERR_INVALID_ARG     # < 512
    assert _decode(_dims(), stride=580) == mla.MLA_ERR_INVALID_ARG     # 1160 B rows: not 16-byte multiples
    assert _decode(_dims(), ws_bytes=100) == mla.MLA_ERR_WORKSPACE
    assert b"workspace" in L.mla_last_error()


def test_decode_rejects_misaligned_pointers():
    L = mla.lib()
    p = ctypes.c_void_p(4096 + 8)
    d = _dims()
    st = L.mla_decode(ctypes.byref(d), 2, p, p, p, p, p, p, p, 576, 10, p, 4, p, p, None, ctypes.c_void_p(1 << 20),
                      1 << 30, 8, None)
    assert st == mla.MLA_ERR_INVALID_ARG


def test_append_rejects_bad_arguments():
    L = mla.lib()
    d = _dims()
    p = ctypes.c_void_p(1 << 16)
    args = [2, p, p, p, None, p, p, 2, 4, p, p, 576, 10, None, None]
    assert L.mla_cache_append(ctypes.byref(d), -1, *args[1:]) == mla.MLA_ERR_INVALID_ARG
    assert L.mla_cache_append(ctypes.byref(d), 0, *args[1:]) == mla.MLA_OK   # nothing to do
    bad = list(args)
    bad[1] = None
    assert L.mla_cache_append(ctypes.byref(d), *bad) == mla.MLA_ERR_INVALID_ARG
    bad = list(args)
    bad[0] = 5           # seq_id NULL with T > num_seqs
    assert L.mla_cache_append(ctypes.byref(d), *bad) == mla.MLA_ERR_INVALID_ARG
    assert L.mla_cache_append(ctypes.byref(_dims(d_c=128)), *args) == mla.MLA_ERR_UNSUPPORTED


def test_workspace_size_grows_with_batch_and_splits():
    L = mla.lib()
    d = _dims()
    a = L.mla_decode_workspace_size(ctypes.byref(d), 64, 256)
    b = L.mla_decode_workspace_size(ctypes.byref(d), 128, 256)
    c = L.mla_decode_workspace_size(ctypes.byref(d), 64, 512)
    assert 0 < a < b and a < c
    # partials (G + B slots) of n_h x 512 bf16 latents plus (m, l) in fp32 dominate
    assert a >= (256 + 64) * 128 * (512 * 2 + 8)
    f = L.mla_decode_workspace_size(ctypes.byref(_dims(dtype=mla.MLA_FP32)), 64, 256)
    assert f >= (256 + 64) * 128 * (512 * 4 + 8) > a
    assert L.mla_decode_workspace_size(ctypes.byref(_dims(d_c=1)), 64, 256) == 0


def _step(dims, ws_bytes=1 << 30, ptr=16, B=2, n_splits=8, stride=576, h_new=True):
    L = mla.lib()
    p = ctypes.c_void_p(ptr * 4096) if ptr else None
    h = p if h_new else None
    return L.mla_decode_step(ctypes.byref(dims) if dims is not None else None, B, h, p, p, p, p, p, p, p, p, p,
                             stride, 10, p, 4, p, p, None, ctypes.c_void_p(1 << 20), ws_bytes, n_splits, None, None)


def test_decode_step_rejects_bad_arguments_before_launching():
    L = mla.lib()
    assert _step(None) == mla.MLA_ERR_INVALID_ARG
    assert _step(_dims(d_c=256)) == mla.MLA_ERR_UNSUPPORTED
    assert _step(_dims(), B=0) == mla.MLA_ERR_INVALID_ARG
    assert _step(_dims(), h_new=False) == mla.MLA_ERR_INVALID_ARG
    assert b"h_new" in L.mla_last_error()
    assert _step(_dims(), stride=580) == mla.MLA_ERR_INVALID_ARG
    need = L.mla_decode_step_workspace_size(ctypes.byref(_dims()), 2, 8)
    assert _step(_dims(), ws_bytes=need - 1) == mla.MLA_ERR_WORKSPACE


def test_decode_step_workspace_holds_the_append_reduction():
    L = mla.lib()
    d = _dims()
    for B in (1, 16, 17, 64, 200):
        dec = L.mla_decode_workspace_size(ctypes.byref(d), B, 256)
        step = L.mla_decode_step_workspace_size(ctypes.byref(d), B, 256)
        # 8 fp32 chunk sums per output element (the tile counters sit in every layout)
        assert step >= dec + 8 * B * 576 * 4
        assert step - dec < 8 * B * 576 * 4 + 256
    assert L.mla_decode_step_workspace_size(ctypes.byref(_dims(d_c=1)), 4, 256) == 0


# ---- projections
COUNTER_BYTES = 1024 * 4          # split-K tile counters at the start of the workspace


def _a256(x):
    return (x + 255) // 256 * 256


def _splits_rows(M):
    return 16 if M <= 16 else 32 if M <= 32 else 64


def _splits_cols(M):
    return 16 if M <= 16 else 64           # four 16-column tiles per wave above 16 rows


def _splits(M, N, K):
    """K chunks of a bf16 projection, counted in 16-column tile units: none
    from 512 units on, else double while below 1024 units (2048 for the
    64-column tiles), up to 16, while 128 * 2S divides K."""
    rows, cols = _splits_rows(M), _splits_cols(M)
    units = (N // cols) * ((M + rows - 1) // rows) * (cols // 16)
    if units >= 512:
        return 1
    target = 1024 if cols == 16 else 2048
    S = 1
    while S < 16 and units * S < target and K % (2 * S * 128) == 0:
        S *= 2
    return S


@pytest.mark.parametrize("B,d_cq,n_h,d_model", [(32, 1536, 128, 5120), (64, 1536, 128, 5120), (1, 512, 16, 1024),
                                                (5, 256, 16, 1024), (40, 0, 16, 1024), (300, 1536, 128, 5120),
                                                (9, 128, 16, 1024), (17, 256, 16, 1024), (33, 256, 16, 1024)])
def test_query_project_workspace_size(B, d_cq, n_h, d_model):
    L = mla.lib()
    d = _dims(n_h=n_h, d_model=d_model)
    N1 = (d_cq if d_cq else n_h * 128) + n_h * 64
    S1 = _splits(B, N1, d_model)
    part = S1 * B * N1 * 4 if S1 > 1 else 0
    if d_cq:
        S2 = _splits(B, n_h * 128, d_cq)
        part = max(part, S2 * B * n_h * 128 * 4 if S2 > 1 else 0)
    packed = B > 8                         # activations packed above 8 rows, padded to 64
    rows = (B + 63) // 64 * 64 if packed else B
    h = _a256(rows * d_model * 2) if packed and not 16 < B <= 32 else 0   # 17..32 rows: h read row-major
    cq = _a256(rows * d_cq * 2)
    assert L.mla_query_project_workspace_size(ctypes.byref(d), B, d_cq) == COUNTER_BYTES + h + cq + _a256(part)
    f = _dims(n_h=n_h, d_model=d_model, dtype=mla.MLA_FP32)
    assert L.mla_query_project_workspace_size(ctypes.byref(f), B, d_cq) == COUNTER_BYTES + _a256(B * d_cq * 4)


def test_split_products_fit_the_tile_counters():
    """A product is split only while it has fewer than 1024 tiles."""
    for M in (1, 7, 16, 17, 32, 33, 64, 100, 500):
        for N, K in ((9728, 5120), (16384, 1536), (5120, 16384), (576, 5120), (1280, 1024), (2048, 256)):
            S = _splits(M, N, K)
            rows, cols = _splits_rows(M), _splits_cols(M)
            assert S == 1 or (N // cols) * ((M + rows - 1) // rows) <= 1024


def test_output_project_workspace_size():
    L = mla.lib()
    for B, n_h, d_model in ((32, 128, 5120), (64, 128, 5120), (1, 16, 1024), (37, 16, 1024), (128, 128, 5120),
                            (8, 16, 1024), (9, 16, 1024)):
        d = _dims(n_h=n_h, d_model=d_model)
        K = n_h * 128
        S = _splits(B, d_model, K)
        o = _a256((B + 63) // 64 * 64 * K * 2) if B > 8 else 0
        want = COUNTER_BYTES + o + (_a256(S * B * d_model * 4) if S > 1 else 0)
        assert L.mla_output_project_workspace_size(ctypes.byref(d), B) == want
        f = _dims(n_h=n_h, d_model=d_model, dtype=mla.MLA_FP32)
        assert L.mla_output_project_workspace_size(ctypes.byref(f), B) == COUNTER_BYTES


def test_pack_weight_rejects_bad_shapes():
    L = mla.lib()
    p = ctypes.c_void_p(16 * 4096)
    d = _dims()
    assert L.mla_pack_weight(ctypes.byref(d), 24, 64, p, p, None) == mla.MLA_ERR_INVALID_ARG    # rows % 16
    assert L.mla_pack_weight(ctypes.byref(d), 32, 48, p, p, None) == mla.MLA_ERR_INVALID_ARG    # K % 32
    assert L.mla_pack_weight(ctypes.byref(d), 0, 64, p, p, None) == mla.MLA_ERR_INVALID_ARG
    assert L.mla_pack_weight(ctypes.byref(d), 32, 64, None, p, None) == mla.MLA_ERR_INVALID_ARG
    assert L.mla_pack_weight(ctypes.byref(d), 32, 64, p, ctypes.c_void_p(16 * 4096 + 2), None) == \
        mla.MLA_ERR_INVALID_ARG
    assert L.mla_pack_weight(None, 32, 64, p, p, None) == mla.MLA_ERR_INVALID_ARG


def _query(dims, B=4, d_cq=512, ptr=16, wdq=True, ws_bytes=1 << 30, ws=1 << 20):
    L = mla.lib()
    p = ctypes.c_void_p(ptr * 4096) if ptr else None
    return L.mla_query_project(ctypes.byref(dims) if dims is not None else None, B, d_cq, p, p if wdq else None, p,
                               p, p, p, ctypes.c_void_p(ws), ws_bytes, None)


def test_query_project_rejects_bad_arguments_before_launching():
    L = mla.lib()
    assert _query(None) == mla.MLA_ERR_INVALID_ARG
    assert _query(_dims(d_c=256)) == mla.MLA_ERR_UNSUPPORTED
    assert _query(_dims(), B=0) == mla.MLA_ERR_INVALID_ARG
    assert _query(_dims(), d_cq=100) == mla.MLA_ERR_UNSUPPORTED      # not a multiple of 128
    assert _query(_dims(), d_cq=-128) == mla.MLA_ERR_UNSUPPORTED
    assert _query(_dims(d_model=5056)) == mla.MLA_ERR_UNSUPPORTED    # bf16 needs d_model % 128 == 0
    assert _query(_dims(), wdq=False) == mla.MLA_ERR_INVALID_ARG     # d_cq > 0 without W_DQ
    assert b"W_DQ" in L.mla_last_error()
    assert _query(_dims(), d_cq=0) == mla.MLA_ERR_INVALID_ARG        # W_DQ given with d_cq == 0
    assert _query(_dims(), ptr=0) == mla.MLA_ERR_INVALID_ARG
    assert _query(_dims(), ws=(1 << 20) + 16) == mla.MLA_ERR_INVALID_ARG   # workspace not 256-aligned
    assert _query(_dims(), ws_bytes=100) == mla.MLA_ERR_WORKSPACE
    assert _query(_dims(), ptr=0) == mla.MLA_ERR_INVALID_ARG
    L2 = mla.lib()
    p = ctypes.c_void_p(16 * 4096)
    bad = ctypes.c_void_p(16 * 4096 + 8)
    d = _dims()
    assert L2.mla_query_project(ctypes.byref(d), 4, 512, bad, p, p, p, p, p, ctypes.c_void_p(1 << 20), 1 << 30,
                                None) == mla.MLA_ERR_INVALID_ARG   # h misaligned


def test_output_project_rejects_bad_arguments_before_launching():
    L = mla.lib()
    p = ctypes.c_void_p(16 * 4096)
    ws = ctypes.c_void_p(1 << 20)
    d = _dims()
    assert L.mla_output_project(None, 4, p, p, p, ws, 1 << 30, None) == mla.MLA_ERR_INVALID_ARG
    assert L.mla_output_project(ctypes.byref(d), 0, p, p, p, ws, 1 << 30, None) == mla.MLA_ERR_INVALID_ARG
    assert L.mla_output_project(ctypes.byref(d), 4, None, p, p, ws, 1 << 30, None) == mla.MLA_ERR_INVALID_ARG
    assert L.mla_output_project(ctypes.byref(d), 4, p, p, ctypes.c_void_p(16 * 4096 + 4), ws, 1 << 30,
                                None) == mla.MLA_ERR_INVALID_ARG
    assert L.mla_output_project(ctypes.byref(d), 4, p, p, p, ws, 10, None) == mla.MLA_ERR_WORKSPACE
    assert L.mla_output_project(ctypes.byref(_dims(d_h=64)), 4, p, p, p, ws, 1 << 30, None) == \
        mla.MLA_ERR_UNSUPPORTED


# ---- the split arithmetic the decode and combine kernels share
def _split_begin(w, N, G):
    return (w * N) // G


def _split_of(x, N, G):
    return ((x + 1) * G + N - 1) // N - 1


@pytest.mark.parametrize("seed", range(20))
def test_split_slots_are_unique_and_contiguous(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    n = rng.integers(0, 300, size=B)
    G = int(rng.integers(1, 300))
    prefix = np.r_[0, np.cumsum(n)]
    N = int(prefix[-1])
    if N == 0:
        return
    for x in range(0, N, max(1, N // 50)):
        w = _split_of(x, N, G)
        assert _split_begin(w, N, G) <= x < _split_begin(w + 1, N, G)
    seen = set()
    for b in range(B):
        if n[b] == 0:
            continue
        w0, w1 = _split_of(prefix[b], N, G), _split_of(prefix[b + 1] - 1, N, G)
        ws = [w for w in range(G) if max(prefix[b], _split_begin(w, N, G)) < min(prefix[b + 1],
                                                                                  _split_begin(w + 1, N, G))]
        assert ws == list(range(w0, w1 + 1))
        for w in ws:
            assert w + b not in seen
            seen.add(w + b)
    assert max(seen) < G + B


def test_append_workspace_size():
    L = mla.lib()
    d = _dims()
    n = L.mla_cache_append_workspace_size(ctypes.byref(d), 32)
    assert n == 8 * 32 * 576 * 4
    assert L.mla_cache_append_workspace_size(ctypes.byref(d), 1024) == 8 * 1024 * 576 * 4
    assert L.mla_cache_append_workspace_size(ctypes.byref(d), 1025) == 0         # up to 1024 rows
    assert L.mla_cache_append_workspace_size(ctypes.byref(_dims(dtype=mla.MLA_FP32)), 32) == 0
    assert L.mla_cache_append_workspace_size(ctypes.byref(_dims(d_model=1536)), 32) == 0


def test_prefill_rejects_bad_arguments_before_launching():
    L = mla.lib()
    p = ctypes.c_void_p(16 * 4096)
    ws = ctypes.c_void_p(1 << 20)
    d = _dims()

    def call(dims=d, T=4, ptr=p, stride=576, ws_bytes=1 << 30, work=ws, num_seqs=2, max_pages=4):
        return L.mla_prefill(ctypes.byref(dims) if dims is not None else None, T, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                             ptr, ptr, ptr, ptr, stride, 10, ptr, num_seqs, max_pages, ptr, None, work, ws_bytes, 8,
                             None)
    assert call(None) == mla.MLA_ERR_INVALID_ARG
    assert call(_dims(d_c=256)) == mla.MLA_ERR_UNSUPPORTED
    assert call(T=0) == mla.MLA_ERR_INVALID_ARG
    assert call(ptr=None) == mla.MLA_ERR_INVALID_ARG
    assert call(ptr=ctypes.c_void_p(16 * 4096 + 2)) == mla.MLA_ERR_INVALID_ARG
    assert call(stride=500) == mla.MLA_ERR_INVALID_ARG
    assert call(num_seqs=0) == mla.MLA_ERR_INVALID_ARG
    assert call(work=ctypes.c_void_p((1 << 20) + 64)) == mla.MLA_ERR_INVALID_ARG
    assert call(ws_bytes=1000) == mla.MLA_ERR_WORKSPACE


def test_prefill_workspace_is_the_decode_layout_plus_query_tables():
    L = mla.lib()
    d = _dims()
    for T, max_pages in ((1, 1), (17, 5), (512, 70)):
        dec = L.mla_decode_workspace_size(ctypes.byref(d), T, 64)
        pre = L.mla_prefill_workspace_size(ctypes.byref(d), T, max_pages, 64)
        assert pre == dec + _a256(T * max_pages * 4) + _a256(T * 4)
    assert L.mla_prefill_workspace_size(ctypes.byref(d), 0, 4, 64) == 0


def test_decode_layer_workspace_is_its_parts():
    L = mla.lib()
    d = _dims()
    for B, d_cq in ((1, 1536), (32, 1536), (64, 0)):
        step = L.mla_decode_step_workspace_size(ctypes.byref(d), B, 256)
        q = L.mla_query_project_workspace_size(ctypes.byref(d), B, d_cq)
        o = L.mla_output_project_workspace_size(ctypes.byref(d), B)
        want = step + _a256(q) + _a256(B * 128 * 128 * 2) + _a256(B * 128 * 64 * 2) + _a256(B * 128 * 128 * 4) + \
            _a256(o)
        assert L.mla_decode_layer_workspace_size(ctypes.byref(d), B, d_cq, 256) == want
    assert L.mla_decode_layer_workspace_size(ctypes.byref(d), 4, 100, 256) == 0


def test_decode_layer_rejects_bad_arguments_before_launching():
    L = mla.lib()
    p = ctypes.c_void_p(16 * 4096)
    ws = ctypes.c_void_p(1 << 20)

    def call(dims=None, B=4, d_cq=512, wdq=p, ptr=p, ws_bytes=1 << 30, work=ws, stride=576):
        dd = _dims() if dims is None else dims
        return L.mla_decode_layer(ctypes.byref(dd), B, d_cq, ptr, ptr, ptr, wdq, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                                  stride, 10, ptr, 4, ptr, ptr, None, work, ws_bytes, 8, None, None)
    assert call(_dims(d_c=256)) == mla.MLA_ERR_UNSUPPORTED
    assert call(B=0) == mla.MLA_ERR_INVALID_ARG
    assert call(wdq=None) == mla.MLA_ERR_INVALID_ARG
    assert call(d_cq=0) == mla.MLA_ERR_INVALID_ARG
    assert call(ptr=None) == mla.MLA_ERR_INVALID_ARG
    assert call(ptr=ctypes.c_void_p(16 * 4096 + 2)) == mla.MLA_ERR_INVALID_ARG
    assert call(stride=500) == mla.MLA_ERR_INVALID_ARG
    assert call(work=ctypes.c_void_p((1 << 20) + 16)) == mla.MLA_ERR_INVALID_ARG
    assert call(ws_bytes=4096) == mla.MLA_ERR_WORKSPACE
