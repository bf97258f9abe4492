"""MI355X (gfx950) MLA decode over the compressed latent KV cache.

A thin ctypes binding over libmla.so (the C ABI in include/mla.h): it only
marshals arguments -- torch tensors' device pointers, sizes and the current
HIP stream.  Every step of the path (cache append, query projection, query
absorption, split-KV decode, combine, W^UV epilogue, output projection) runs
in the library's HIP kernels.

Importing this package does not touch the GPU.  Loading fails loudly if
libmla.so has not been built (python -m compressed_kv_cache_mla_amd.build).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = range(5)
MLA_BF16, MLA_FP32 = 0, 1
FLAG_BAD_SEQ_LEN, FLAG_BAD_PAGE, FLAG_BAD_POSITION, FLAG_BAD_SEQ_ID = 1, 2, 4, 8

EXPORTED = ("mla_cache_append", "mla_cache_append_ws", "mla_cache_append_workspace_size",
            "mla_decode_workspace_size", "mla_decode", "mla_decode_ex",
            "mla_decode_step_workspace_size", "mla_decode_step", "mla_decode_step_noalloc",
            "mla_pack_weight", "mla_query_project_workspace_size", "mla_query_project",
            "mla_output_project_workspace_size", "mla_output_project",
            "mla_prefill_workspace_size", "mla_prefill",
            "mla_decode_layer_workspace_size", "mla_decode_layer",
            "mla_indexer_select_workspace_size", "mla_indexer_select",
            "mla_sparse_decode_workspace_size", "mla_sparse_decode",
            "mla_read_error_flags", "mla_last_error", "mla_device_cu_count")


class MlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"mla status {status}: {msg}")
        self.status = status


class mla_dims(ctypes.Structure):
    _fields_ = [("n_h", ctypes.c_int32), ("d_h", ctypes.c_int32), ("d_c", ctypes.c_int32),
                ("d_hR", ctypes.c_int32), ("d_model", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("rope_base", ctypes.c_float), ("dtype", ctypes.c_int32)]


class mla_decode_opts(ctypes.Structure):
    _fields_ = [("ev_start", ctypes.c_void_p), ("ev_stop", ctypes.c_void_p), ("impl", ctypes.c_int32)]


@dataclass(frozen=True)
class Dims:
    """MLA sizes in the pages' notation (DeepSeek-V2: n_h = 128, d_h = 128,
    d_c = 512, d_h^R = 64, d_model = 5120)."""
    n_h: int = 128
    d_h: int = 128
    d_c: int = 512
    d_hR: int = 64
    d_model: int = 5120
    page_size: int = 64
    rope_base: float = 10000.0
    dtype: torch.dtype = torch.bfloat16
    softmax_scale: float | None = None

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale is not None else 1.0 / (self.d_h + self.d_hR) ** 0.5

    def c(self) -> mla_dims:
        if self.dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("dtype must be torch.bfloat16 or torch.float32")
        return mla_dims(self.n_h, self.d_h, self.d_c, self.d_hR, self.d_model, self.page_size, self.scale,
                        self.rope_base, MLA_BF16 if self.dtype == torch.bfloat16 else MLA_FP32)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmla.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with python -m compressed_kv_cache_mla_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        pdims = ctypes.POINTER(mla_dims)
        L.mla_cache_append.argtypes = [pdims, i32, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, i64, i32, vp, vp]
        L.mla_cache_append.restype = ctypes.c_int
        L.mla_cache_append_ws.argtypes = [pdims, i32, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, i64, i32, vp, vp,
                                          sz, vp]
        L.mla_cache_append_ws.restype = ctypes.c_int
        L.mla_cache_append_workspace_size.argtypes = [pdims, i32]
        L.mla_cache_append_workspace_size.restype = sz
        L.mla_decode_workspace_size.argtypes = [pdims, i32, i32]
        L.mla_decode_workspace_size.restype = sz
        L.mla_decode.argtypes = [pdims, i32, vp, vp, vp, vp, vp, vp, vp, i64, i32, vp, i32, vp, vp, vp, vp, sz,
                                 i32, vp]
        L.mla_decode.restype = ctypes.c_int
        L.mla_decode_ex.argtypes = [pdims, i32, vp, vp, vp, vp, vp, vp, vp, i64, i32, vp, i32, vp, vp, vp, vp, sz,
                                    i32, ctypes.POINTER(mla_decode_opts), vp]
        L.mla_decode_ex.restype = ctypes.c_int
        L.mla_decode_step_workspace_size.argtypes = [pdims, i32, i32]
        L.mla_decode_step_workspace_size.restype = sz
        L.mla_decode_step.argtypes = [pdims, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, vp, i32, vp, vp,
                                      vp, vp, sz, i32, ctypes.POINTER(mla_decode_opts), vp]
        L.mla_decode_step.restype = ctypes.c_int
        L.mla_decode_step_noalloc.argtypes = [pdims, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, vp, i32,
                                              vp, vp, vp, vp, vp]
        L.mla_decode_step_noalloc.restype = ctypes.c_int
        L.mla_pack_weight.argtypes = [pdims, i32, i32, vp, vp, vp]
        L.mla_pack_weight.restype = ctypes.c_int
        L.mla_query_project_workspace_size.argtypes = [pdims, i32, i32]
        L.mla_query_project_workspace_size.restype = sz
        L.mla_query_project.argtypes = [pdims, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.mla_query_project.restype = ctypes.c_int
        L.mla_output_project_workspace_size.argtypes = [pdims, i32]
        L.mla_output_project_workspace_size.restype = sz
        L.mla_output_project.argtypes = [pdims, i32, vp, vp, vp, vp, sz, vp]
        L.mla_output_project.restype = ctypes.c_int
        L.mla_prefill_workspace_size.argtypes = [pdims, i32, i32, i32]
        L.mla_prefill_workspace_size.restype = sz
        L.mla_prefill.argtypes = [pdims, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, vp, i32, i32, vp,
                                  vp, vp, sz, i32, vp]
        L.mla_prefill.restype = ctypes.c_int
        L.mla_decode_layer_workspace_size.argtypes = [pdims, i32, i32, i32]
        L.mla_decode_layer_workspace_size.restype = sz
        L.mla_decode_layer.argtypes = [pdims, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, vp,
                                       i32, vp, vp, vp, vp, sz, i32, ctypes.POINTER(mla_decode_opts), vp]
        L.mla_decode_layer.restype = ctypes.c_int
        L.mla_indexer_select_workspace_size.argtypes = [i32, i32, i32, i32]
        L.mla_indexer_select_workspace_size.restype = sz
        L.mla_indexer_select.argtypes = [i32, i32, i32, i32, vp, vp, vp, i64, i32, i32, vp, i32, vp, vp, vp, vp, vp,
                                         vp, sz, vp]
        L.mla_indexer_select.restype = ctypes.c_int
        L.mla_sparse_decode_workspace_size.argtypes = [pdims, i32, i32, i32, i32]
        L.mla_sparse_decode_workspace_size.restype = sz
        L.mla_sparse_decode.argtypes = [pdims, i32, vp, vp, vp, vp, vp, vp, vp, i64, i32, vp, i32, vp, i32, i32, i32,
                                        vp, vp, vp, i64, vp, vp, vp, vp, sz, i32, ctypes.POINTER(mla_decode_opts), vp]
        L.mla_sparse_decode.restype = ctypes.c_int
        L.mla_read_error_flags.argtypes = [vp, ctypes.POINTER(i32), vp]
        L.mla_read_error_flags.restype = ctypes.c_int
        L.mla_last_error.argtypes = []
        L.mla_last_error.restype = ctypes.c_char_p
        L.mla_device_cu_count.argtypes = []
        L.mla_device_cu_count.restype = i32
        _lib = L
    return _lib


def _check(status: int):
    if status != MLA_OK:
        raise MlaError(status, lib().mla_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def cu_count() -> int:
    return int(lib().mla_device_cu_count())


def cache_append(dims: Dims, h_t, W_DKV, W_KR, pos, page_table, c_KV, k_R, row_stride: int, num_pages: int,
                 seq_id=None, err_flag=None, stream=None, workspace=None):
    """mla_cache_append (mla_cache_append_ws when a workspace tensor is given):
    write c^KV = W^DKV h_t and k^R = RoPE(W^KR h_t) of T token rows into the
    paged pool (see include/mla.h)."""
    T = h_t.shape[0]
    num_seqs, max_pages = page_table.shape
    d = dims.c()
    args = (ctypes.byref(d), T, _ptr(h_t), _ptr(W_DKV), _ptr(W_KR), _ptr(seq_id), _ptr(pos), _ptr(page_table),
            num_seqs, max_pages, _ptr(c_KV), _ptr(k_R), row_stride, num_pages, _ptr(err_flag))
    if workspace is None:
        _check(lib().mla_cache_append(*args, _stream(stream)))
    else:
        _check(lib().mla_cache_append_ws(*args, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _stream(stream)))


def cache_append_workspace_size(dims: Dims, T: int) -> int:
    d = dims.c()
    return int(lib().mla_cache_append_workspace_size(ctypes.byref(d), T))


def decode_workspace_size(dims: Dims, B: int, n_splits: int = 0) -> int:
    d = dims.c()
    return int(lib().mla_decode_workspace_size(ctypes.byref(d), B, n_splits))


class HipEvent:
    """A HIP timing event created with hipEventDisableSystemFence: recording it
    between two kernels adds no system-scope release (cache write-back), so it
    can bracket one kernel without stretching the step.  Uses the HIP runtime
    that torch (and libmla.so) already loaded."""
    _hip = None

    def __init__(self):
        if HipEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            HipEvent._hip = hip
        self.handle = ctypes.c_void_p()
        st = HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.handle), ctypes.c_uint(0x20000000))
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self, stream=None):
        """Record on `stream` (default: torch's current stream)."""
        st = HipEvent._hip.hipEventRecord(self.handle, _stream(stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        st = HipEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return float(ms.value)

    def __del__(self):
        # only the class and the instance are used: module globals (ctypes
        # included) may already be gone at interpreter exit
        hip, handle = type(self)._hip, getattr(self, "handle", None)
        if handle and hip is not None:
            hip.hipEventDestroy(handle)
        self.handle = None


def _event_handle(ev):
    if ev is None:
        return None
    if isinstance(ev, HipEvent):
        return ev.handle
    if not ev.cuda_event:      # torch creates the HIP event on its first record
        ev.record()
    return ctypes.c_void_p(ev.cuda_event)


def decode(dims: Dims, q_C, q_R, pos_q, W_UK, W_UV, c_KV, k_R, row_stride: int, num_pages: int, page_table,
           seq_lens, out, lse=None, workspace=None, n_splits: int = 0, stream=None, ev_start=None, ev_stop=None,
           impl: int = 0):
    """mla_decode (mla_decode_ex when events or impl are given): one query per
    sequence against its cached latent rows; writes out [B, n_h, d_h] (fp32)
    and optionally lse [B, n_h].  ev_start / ev_stop (HipEvent or
    torch.cuda.Event) are recorded around the split-KV attention kernel."""
    B = q_C.shape[0]
    max_pages = page_table.shape[1]
    if workspace is None:
        workspace = torch.empty(decode_workspace_size(dims, B, n_splits), dtype=torch.uint8, device=q_C.device)
    d = dims.c()
    args = (ctypes.byref(d), B, _ptr(q_C), _ptr(q_R), _ptr(pos_q), _ptr(W_UK), _ptr(W_UV), _ptr(c_KV), _ptr(k_R),
            row_stride, num_pages, _ptr(page_table), max_pages, _ptr(seq_lens), _ptr(out), _ptr(lse),
            _ptr(workspace), workspace.numel(), n_splits)
    if ev_start is None and ev_stop is None and impl == 0:
        _check(lib().mla_decode(*args, _stream(stream)))
    else:
        o = mla_decode_opts(_event_handle(ev_start), _event_handle(ev_stop), impl)
        _check(lib().mla_decode_ex(*args, ctypes.byref(o), _stream(stream)))
    return workspace


def indexer_select_workspace_size(B: int, max_pages: int, page_size: int, top_k: int) -> int:
    return int(lib().mla_indexer_select_workspace_size(B, max_pages, page_size, top_k))


def indexer_select(q_I, w_I, k_I, idx_row_stride: int, num_pages: int, page_size: int, page_table, seq_lens,
                   top_k: int, scores, sel_tok, sel_row, err_flags, workspace=None, stream=None):
    """mla_indexer_select: the indexer's relevance scores of every cached
    token (scores [B, max_pages*page_size] fp32) and the top_k kept tokens of
    each sequence in ascending order with their pool rows (sel_tok, sel_row
    [B, top_k] int32; entries past min(seq_len, top_k) are left as they
    were).  err_flags: a device int32 word the kernels OR MLA_FLAG_* into."""
    B, H_I, d_I = q_I.shape
    max_pages = page_table.shape[1]
    if workspace is None:
        workspace = torch.empty(indexer_select_workspace_size(B, max_pages, page_size, top_k), dtype=torch.uint8,
                                device=q_I.device)
    _check(lib().mla_indexer_select(B, H_I, d_I, top_k, _ptr(q_I), _ptr(w_I), _ptr(k_I), idx_row_stride, num_pages,
                                    page_size, _ptr(page_table), max_pages, _ptr(seq_lens), _ptr(scores),
                                    _ptr(sel_tok), _ptr(sel_row), _ptr(err_flags), _ptr(workspace),
                                    workspace.numel(), _stream(stream)))
    return workspace


def sparse_decode_workspace_size(dims: Dims, B: int, max_pages: int, top_k: int, n_splits: int = 0) -> int:
    d = dims.c()
    return int(lib().mla_sparse_decode_workspace_size(ctypes.byref(d), B, max_pages, top_k, n_splits))


def sparse_decode(dims: Dims, q_C, q_R, pos_q, W_UK, W_UV, c_KV, k_R, row_stride: int, num_pages: int, page_table,
                  seq_lens, q_I, w_I, k_I, idx_row_stride: int, top_k: int, out, lse=None, sel_tok=None,
                  workspace=None, n_splits: int = 0, stream=None, ev_start=None, ev_stop=None):
    """mla_sparse_decode: the indexer picks each sequence's top_k cached
    tokens, then the MLA decode attends over those rows only.  sel_tok
    (optional [B, top_k] int32) receives the kept tokens; ev_start / ev_stop
    are recorded around the gather attention kernel."""
    B = q_C.shape[0]
    H_I, d_I = q_I.shape[1], q_I.shape[2]
    max_pages = page_table.shape[1]
    if workspace is None:
        workspace = torch.empty(sparse_decode_workspace_size(dims, B, max_pages, top_k, n_splits), dtype=torch.uint8,
                                device=q_C.device)
    d = dims.c()
    o = mla_decode_opts(_event_handle(ev_start), _event_handle(ev_stop), 0)
    _check(lib().mla_sparse_decode(ctypes.byref(d), B, _ptr(q_C), _ptr(q_R), _ptr(pos_q), _ptr(W_UK), _ptr(W_UV),
                                   _ptr(c_KV), _ptr(k_R), row_stride, num_pages, _ptr(page_table), max_pages,
                                   _ptr(seq_lens), H_I, d_I, top_k, _ptr(q_I), _ptr(w_I), _ptr(k_I), idx_row_stride,
                                   _ptr(out), _ptr(lse), _ptr(sel_tok), _ptr(workspace), workspace.numel(), n_splits,
                                   ctypes.byref(o), _stream(stream)))
    return workspace


def decode_step_workspace_size(dims: Dims, B: int, n_splits: int = 0) -> int:
    d = dims.c()
    return int(lib().mla_decode_step_workspace_size(ctypes.byref(d), B, n_splits))


def decode_step_workspace(dims: Dims, B: int, n_splits: int = 0, device="cuda"):
    """A zero-filled workspace for decode_step (the library needs it zeroed once)."""
    return torch.zeros(decode_step_workspace_size(dims, B, n_splits), dtype=torch.uint8, device=device)


def decode_step(dims: Dims, h_new, W_DKV, W_KR, q_C, q_R, pos_q, W_UK, W_UV, c_KV, k_R, row_stride: int,
                num_pages: int, page_table, seq_lens, out, lse, workspace, n_splits: int = 0, stream=None,
                ev_start=None, ev_stop=None, impl: int = 0):
    """mla_decode_step: append each sequence's newest token (h_new[b] at
    position pos_q[b]) to the pool, then decode; the workspace comes from
    decode_step_workspace() (zero-filled once, reused across calls)."""
    B = q_C.shape[0]
    max_pages = page_table.shape[1]
    d = dims.c()
    o = mla_decode_opts(_event_handle(ev_start), _event_handle(ev_stop), impl)
    _check(lib().mla_decode_step(ctypes.byref(d), B, _ptr(h_new), _ptr(W_DKV), _ptr(W_KR), _ptr(q_C), _ptr(q_R),
                                 _ptr(pos_q), _ptr(W_UK), _ptr(W_UV), _ptr(c_KV), _ptr(k_R), row_stride, num_pages,
                                 _ptr(page_table), max_pages, _ptr(seq_lens), _ptr(out), _ptr(lse), _ptr(workspace),
                                 workspace.numel(), n_splits, ctypes.byref(o), _stream(stream)))


def decode_step_noalloc(dims: Dims, h_new, W_DKV, W_KR, q_C, q_R, pos_q, W_UK, W_UV, c_KV, k_R, row_stride: int,
                        num_pages: int, page_table, seq_lens, out, lse=None, err_flags=None, stream=None):
    """mla_decode_step_noalloc: decode_step without a workspace (the library's
    own per-GPU scratch array; nothing is allocated).  err_flags: None or a
    one-element int32 device tensor that receives the step's FLAG_* bits."""
    B = q_C.shape[0]
    max_pages = page_table.shape[1]
    d = dims.c()
    _check(lib().mla_decode_step_noalloc(ctypes.byref(d), B, _ptr(h_new), _ptr(W_DKV), _ptr(W_KR), _ptr(q_C),
                                         _ptr(q_R), _ptr(pos_q), _ptr(W_UK), _ptr(W_UV), _ptr(c_KV), _ptr(k_R),
                                         row_stride, num_pages, _ptr(page_table), max_pages, _ptr(seq_lens),
                                         _ptr(out), _ptr(lse), _ptr(err_flags), _stream(stream)))


def pack_weight(dims: Dims, W, stream=None):
    """mla_pack_weight: a new tensor holding W [rows, K] in the packed layout
    the projection kernels stream (same dtype, same element count)."""
    if not W.is_contiguous():
        raise ValueError("pack_weight needs a contiguous row-major W")
    rows, K = W.shape
    out = torch.empty_like(W)
    d = dims.c()
    _check(lib().mla_pack_weight(ctypes.byref(d), rows, K, _ptr(W), _ptr(out), _stream(stream)))
    return out


def query_project_workspace_size(dims: Dims, B: int, d_cq: int) -> int:
    d = dims.c()
    return int(lib().mla_query_project_workspace_size(ctypes.byref(d), B, d_cq))


def query_project_workspace(dims: Dims, B: int, d_cq: int, device="cuda"):
    """A zero-filled workspace for query_project (the library needs it zeroed once)."""
    return torch.zeros(query_project_workspace_size(dims, B, d_cq), dtype=torch.uint8, device=device)


def query_project(dims: Dims, h, W_DQ, W_UQ, W_QR, q_C, q_R, workspace, stream=None):
    """mla_query_project: q^C = W^UQ (W^DQ h) and q^R = W^QR h (unrotated) for
    B token states h [B, d_model] into q_C [B, n_h, d_h], q_R [B, n_h, d_hR].
    The weights are packed (pack_weight); W_DQ None means no query
    down-projection (c^Q = h)."""
    B = h.shape[0]
    d_cq = 0 if W_DQ is None else W_DQ.shape[0]
    d = dims.c()
    _check(lib().mla_query_project(ctypes.byref(d), B, d_cq, _ptr(h), _ptr(W_DQ), _ptr(W_UQ), _ptr(W_QR),
                                   _ptr(q_C), _ptr(q_R), _ptr(workspace), workspace.numel(), _stream(stream)))


def output_project_workspace_size(dims: Dims, B: int) -> int:
    d = dims.c()
    return int(lib().mla_output_project_workspace_size(ctypes.byref(d), B))


def output_project_workspace(dims: Dims, B: int, device="cuda"):
    """A zero-filled workspace for output_project (the library needs it zeroed once)."""
    return torch.zeros(output_project_workspace_size(dims, B), dtype=torch.uint8, device=device)


def output_project(dims: Dims, o, W_O, u, workspace, stream=None):
    """mla_output_project: u [B, d_model] = W^O [o_1; ...; o_n_h] for the
    per-head outputs o [B, n_h, d_h] (fp32); W_O packed (pack_weight)."""
    B = o.shape[0]
    d = dims.c()
    _check(lib().mla_output_project(ctypes.byref(d), B, _ptr(o), _ptr(W_O), _ptr(u), _ptr(workspace),
                                    workspace.numel(), _stream(stream)))


def prefill_workspace_size(dims: Dims, T: int, max_pages: int, n_splits: int = 0) -> int:
    d = dims.c()
    return int(lib().mla_prefill_workspace_size(ctypes.byref(d), T, max_pages, n_splits))


def prefill(dims: Dims, h, W_DKV, W_KR, q_C, q_R, seq_id, pos, W_UK, W_UV, c_KV, k_R, row_stride: int,
            num_pages: int, page_table, out, lse=None, workspace=None, n_splits: int = 0, stream=None):
    """mla_prefill: append T new tokens (token t: sequence seq_id[t], position
    pos[t]) and let each attend causally over its sequence; writes out
    [T, n_h, d_h] (fp32) and optionally lse [T, n_h].  Returns the workspace
    (which holds the error flags)."""
    T = h.shape[0]
    num_seqs, max_pages = page_table.shape
    if workspace is None:
        workspace = torch.empty(prefill_workspace_size(dims, T, max_pages, n_splits), dtype=torch.uint8,
                                device=h.device)
    d = dims.c()
    _check(lib().mla_prefill(ctypes.byref(d), T, _ptr(h), _ptr(W_DKV), _ptr(W_KR), _ptr(q_C), _ptr(q_R),
                             _ptr(seq_id), _ptr(pos), _ptr(W_UK), _ptr(W_UV), _ptr(c_KV), _ptr(k_R), row_stride,
                             num_pages, _ptr(page_table), num_seqs, max_pages, _ptr(out), _ptr(lse), _ptr(workspace),
                             workspace.numel(), n_splits, _stream(stream)))
    return workspace


def decode_layer_workspace_size(dims: Dims, B: int, d_cq: int, n_splits: int = 0) -> int:
    d = dims.c()
    return int(lib().mla_decode_layer_workspace_size(ctypes.byref(d), B, d_cq, n_splits))


def decode_layer_workspace(dims: Dims, B: int, d_cq: int, n_splits: int = 0, device="cuda"):
    """A zero-filled workspace for decode_layer (the library needs it zeroed once)."""
    return torch.zeros(decode_layer_workspace_size(dims, B, d_cq, n_splits), dtype=torch.uint8, device=device)


def decode_layer(dims: Dims, h, W_DKV, W_KR, W_DQ, W_UQ, W_QR, W_UK, W_UV, W_O, pos_q, c_KV, k_R, row_stride: int,
                 num_pages: int, page_table, seq_lens, u, lse, workspace, n_splits: int = 0, stream=None,
                 ev_start=None, ev_stop=None, impl: int = 0):
    """mla_decode_layer: query projection, decode step (append + attention +
    combine + W^UV) and output projection for one new token per sequence;
    writes u [B, d_model] (fp32).  W_DQ, W_UQ, W_QR, W_O packed (pack_weight);
    W_DQ None means no query down-projection."""
    B = h.shape[0]
    d_cq = 0 if W_DQ is None else W_DQ.shape[0]
    max_pages = page_table.shape[1]
    d = dims.c()
    o = mla_decode_opts(_event_handle(ev_start), _event_handle(ev_stop), impl)
    _check(lib().mla_decode_layer(ctypes.byref(d), B, d_cq, _ptr(h), _ptr(W_DKV), _ptr(W_KR), _ptr(W_DQ), _ptr(W_UQ),
                                  _ptr(W_QR), _ptr(W_UK), _ptr(W_UV), _ptr(W_O), _ptr(pos_q), _ptr(c_KV), _ptr(k_R),
                                  row_stride, num_pages, _ptr(page_table), max_pages, _ptr(seq_lens), _ptr(u),
                                  _ptr(lse), _ptr(workspace), workspace.numel(), n_splits, ctypes.byref(o),
                                  _stream(stream)))


def read_error_flags(workspace_or_flag, stream=None) -> int:
    """Device error flags (FLAG_* bits) of a decode workspace or append flag word; clears them."""
    v = ctypes.c_int32(0)
    _check(lib().mla_read_error_flags(_ptr(workspace_or_flag), ctypes.byref(v), _stream(stream)))
    return int(v.value)
