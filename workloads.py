"""Synthetic MLA decode workloads shared by the GPU tests and bench.py.

Each workload fixes the shapes of one benchmark configuration (DeepSeek-V2
attention dims: n_h = 128, d_h = 128, d_c = 512, d_h^R = 64, d_model = 5120),
builds its inputs on the device from the seeded generator (seeded_inputs), and
can regenerate, on the CPU and without reading anything back from the GPU,
the fp64 inputs the oracle needs for any one sequence.

Conventions (the same as the library's and the oracle's):
* sequence b holds n_b cached tokens at positions 0 .. n_b-1; the decode query
  is the last of them (position n_b - 1), appended just before decoding;
* the pool is [num_pages, page_size, 576]: c^KV in columns 0..511, k^R in
  512..575; sequence b owns ceil(n_b / page_size) pages, assigned either in
  order or through a seeded random permutation of the whole pool;
* cache rows come either from the append kernel applied to seeded token
  states h ~ N(0, 1) ("append" mode) or straight from the generator as
  N(0, 1) latents ("direct" mode, used where building the context through
  append would take long, e.g. 60 layers x 128 x 8192 tokens);
* weights ~ N(0, 1/fan_in); q^C, q^R ~ N(0, 1) (the distribution of W^UQ h and
  W^QR h under those weights);
* "exact query" workloads (tests only) replace W^UK and q^C by values built
  from the same N(0, 1) draws with comparisons alone: W^UK entries in
  {0, +-1/4, +-1/2}, mostly 0, and q^C small integers, so that every element of
  q~ = W^UK^T q^C is a multiple of 1/4 below 64 in magnitude and exact in
  bf16; q^R is drawn small (N(0, 2^-16)) and the softmax scale is the fp32
  value of ln 2, whose product with fp32 log2(e) is exactly 1.  The scores
  the kernel sees are then the oracle's up to fp32 summation and the small
  RoPE'd q^R part, whatever their size.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

import seeded_inputs as si

D_C, D_R, D_H = 512, 64, 128
D_K = D_C + D_R


@dataclass
class Config:
    name: str
    n_h: int
    d_model: int
    B: int
    lens: object            # int (uniform prior context L) or (lo, hi) ragged range of L
    dtype: torch.dtype = torch.bfloat16
    page_size: int = 64
    permute_pages: bool = False
    cache_mode: str = "append"   # "append" | "direct"
    layers: int = 1
    seed: int = 1234
    query: str = "synthetic"     # "synthetic" | "projected" (q from W^UQ, W^QR; tests only)
    growth: int = 0              # direct mode: the row at position p of an n-token sequence is
                                 # scaled by 2^floor(growth * p / n) (scores that keep rising)
    exact_q: bool = False        # W^UK, q^C with q~ exact in bf16 (see the module docstring)

    def context_lengths(self) -> np.ndarray:
        """Prior context L_b per sequence (the decode token comes on top)."""
        if isinstance(self.lens, (tuple, list)):
            lo, hi = self.lens
            return si.uniform_ints(self.seed, self.name + "/lens", self.B, lo, hi)
        return np.full(self.B, int(self.lens), dtype=np.int64)


# The benchmark configurations (DeepSeek-V2 MLA decode shapes).
CONFIGS = {
    "tiny_fp32": Config("tiny_fp32", n_h=16, d_model=1024, B=1, lens=256, dtype=torch.float32,
                        cache_mode="append", seed=1235, query="projected"),
    "b32_l4096": Config("b32_l4096", n_h=128, d_model=5120, B=32, lens=4096, seed=1236),
    "b64_ragged": Config("b64_ragged", n_h=128, d_model=5120, B=64, lens=(1024, 16384), permute_pages=True,
                         seed=1237),
    "b4_l131072": Config("b4_l131072", n_h=128, d_model=5120, B=4, lens=131072, seed=1238),
    "l60_b128_l8192": Config("l60_b128_l8192", n_h=128, d_model=5120, B=128, lens=8192, layers=60,
                             cache_mode="direct", seed=1239),
    "b64_l8192": Config("b64_l8192", n_h=128, d_model=5120, B=64, lens=8192, seed=1240),
}


def scaled(cfg: Config, **kw) -> Config:
    """A copy of cfg with some fields replaced (smaller test variants)."""
    d = dict(cfg.__dict__)
    d.update(kw)
    return Config(**d)


def _key(cfg: Config, name: str, layer: int = 0) -> int:
    return si.stream_key(cfg.seed, name, layer)


# fp32 ln 2: times fp32 log2(e) it rounds to exactly 1.0 in fp32
LN2_F32 = float(np.float32(math.log(2.0)))


def _steps(x: torch.Tensor, thresholds, unit: float) -> torch.Tensor:
    """sign(x) * unit * #{t in thresholds : |x| >= t}, by comparisons only, so
    that the CPU and the GPU map the same draws to the same values."""
    a = x.abs()
    k = torch.zeros_like(x, dtype=torch.float32)
    for t in thresholds:
        k = k + (a >= t).to(torch.float32)
    return (torch.sign(x.to(torch.float32)) * k * unit).to(x.dtype)


def exact_W_UK(x: torch.Tensor) -> torch.Tensor:
    """Exact-query W^UK from N(0, 1) draws: 0 for |x| < 1.5, +-1/4 up to 3, +-1/2 beyond."""
    return _steps(x, (1.5, 3.0), 0.25)


def exact_q_C(x: torch.Tensor) -> torch.Tensor:
    """Exact-query q^C from N(0, 1) draws: integers in [-6, 6]."""
    return _steps(x, (0.5, 1.0, 1.5, 2.0, 2.5, 3.0), 1.0)


class Workload:
    """Device tensors of one configuration (one layer at a time)."""

    def __init__(self, cfg: Config, device="cuda", layer: int = 0, n_splits: int = 0):
        import compressed_kv_cache_mla_amd as mla
        self.mla = mla
        self.cfg = cfg
        self.layer = layer
        self.device = torch.device(device)
        self.dims = mla.Dims(n_h=cfg.n_h, d_model=cfg.d_model, page_size=cfg.page_size, dtype=cfg.dtype,
                             softmax_scale=LN2_F32 if cfg.exact_q else None)
        self.n_splits = n_splits
        L = cfg.context_lengths()
        self.n = (L + 1).astype(np.int64)                      # cached tokens incl. the decode token
        self.prefix = np.concatenate([[0], np.cumsum(self.n)]).astype(np.int64)
        ps = cfg.page_size
        self.pages_per_seq = (self.n + ps - 1) // ps
        self.max_pages = int(self.pages_per_seq.max())
        self.num_pages = int(self.pages_per_seq.sum())
        order = si.permutation(cfg.seed, cfg.name + "/pages", self.num_pages) if cfg.permute_pages \
            else np.arange(self.num_pages)
        pt = np.zeros((cfg.B, self.max_pages), dtype=np.int32)
        off = 0
        for b in range(cfg.B):
            k = int(self.pages_per_seq[b])
            pt[b, :k] = order[off:off + k]
            off += k
        self.page_table_np = pt
        dev = self.device
        self.page_table = torch.from_numpy(pt).to(dev)
        self.seq_lens = torch.from_numpy(self.n.astype(np.int32)).to(dev)
        self.pos_q = torch.from_numpy((self.n - 1).astype(np.int32)).to(dev)
        self.pool = torch.empty((self.num_pages * ps, D_K), dtype=cfg.dtype, device=dev)
        self.c_KV = self.pool[:, :D_C]
        self.k_R = self.pool[:, D_C:]
        self.row_stride = D_K
        self.out = torch.empty((cfg.B, cfg.n_h, D_H), dtype=torch.float32, device=dev)
        self.lse = torch.empty((cfg.B, cfg.n_h), dtype=torch.float32, device=dev)
        self._build_weights()
        self._build_queries()
        self._build_cache()
        self.workspace = torch.empty(mla.decode_workspace_size(self.dims, cfg.B, n_splits), dtype=torch.uint8,
                                     device=dev)

    # ---------------------------------------------------------------- inputs
    def _w(self, name, rows, cols, fan_in, device=None):
        return si.normal(_key(self.cfg, name, self.layer), (rows, cols), 1.0 / math.sqrt(fan_in), self.cfg.dtype,
                         device or self.device)

    def _W_UK(self, device=None):
        c = self.cfg
        if c.exact_q:
            return exact_W_UK(si.normal(_key(c, "W_UK", self.layer), (c.n_h * D_H, D_C), 1.0, c.dtype,
                                        device or self.device))
        return self._w("W_UK", c.n_h * D_H, D_C, D_C, device=device)

    def _q_rows(self, name, rows, width, device):
        c = self.cfg
        if name == "q_C" and c.exact_q:
            return exact_q_C(si.normal_rows(_key(c, name, self.layer), rows, width, 1.0, c.dtype, device))
        scale = 1.0 / 256 if (name == "q_R" and c.exact_q) else 1.0
        return si.normal_rows(_key(c, name, self.layer), rows, width, scale, c.dtype, device)

    def _build_weights(self):
        c, dm, nh = self.cfg, self.cfg.d_model, self.cfg.n_h
        self.W_DKV = self._w("W_DKV", D_C, dm, dm)
        self.W_KR = self._w("W_KR", D_R, dm, dm)
        self.W_UK = self._W_UK()
        self.W_UV = self._w("W_UV", nh * D_H, D_C, D_C)

    def _build_queries(self):
        c = self.cfg
        if c.query == "synthetic":
            rows = range(c.B * c.n_h)
            self.q_C = self._q_rows("q_C", rows, D_H, self.device).reshape(c.B, c.n_h, D_H)
            self.q_R = self._q_rows("q_R", rows, D_R, self.device).reshape(c.B, c.n_h, D_R)
        else:   # filled in by the caller (set_queries)
            self.q_C = torch.zeros((c.B, c.n_h, D_H), dtype=c.dtype, device=self.device)
            self.q_R = torch.zeros((c.B, c.n_h, D_R), dtype=c.dtype, device=self.device)

    def set_queries(self, q_C: torch.Tensor, q_R: torch.Tensor):
        self.q_C.copy_(q_C.to(self.device, self.cfg.dtype))
        self.q_R.copy_(q_R.to(self.device, self.cfg.dtype))

    def token_rows(self):
        """(seq_id, pos) of every cached token, in global token order."""
        B = self.cfg.B
        seq = np.repeat(np.arange(B), self.n)
        pos = np.arange(int(self.prefix[-1])) - np.repeat(self.prefix[:-1], self.n)
        return seq.astype(np.int32), pos.astype(np.int32)

    def h_rows(self, rows, device=None):
        """Token states h for global token ids ``rows`` (append mode)."""
        return si.normal_rows(_key(self.cfg, "h", self.layer), rows, self.cfg.d_model, 1.0, self.cfg.dtype,
                              device or self.device)

    def latent_rows(self, rows, device=None):
        """Direct-mode cache rows [c^KV ; k^R] for global token ids ``rows``."""
        x = si.normal_rows(_key(self.cfg, "latent", self.layer), rows, D_K, 1.0, self.cfg.dtype,
                           device or self.device)
        if self.cfg.growth:
            # power-of-two factors: the scaled rows are exact in any dtype
            g = np.asarray(rows.cpu() if torch.is_tensor(rows) else rows, dtype=np.int64)
            b = np.searchsorted(self.prefix, g, side="right") - 1
            k = (self.cfg.growth * (g - self.prefix[b])) // self.n[b]
            x = x * torch.from_numpy(np.ldexp(1.0, k).astype(np.float32)).to(x.device, x.dtype)[:, None]
        return x

    def pool_rows(self, seq: np.ndarray, pos: np.ndarray) -> np.ndarray:
        ps = self.cfg.page_size
        return self.page_table_np[seq, pos // ps].astype(np.int64) * ps + pos % ps

    def _build_cache(self, chunk: int = 65536):
        seq, pos = self.token_rows()
        N = seq.size
        if self.cfg.cache_mode == "direct":
            # all tokens but each sequence's last come straight from the generator;
            # the last (decode) token is appended through the library
            last = self.prefix[1:] - 1
            mask = np.ones(N, dtype=bool)
            mask[last] = False
            ids = np.nonzero(mask)[0]
            for i in range(0, ids.size, chunk):
                g = ids[i:i + chunk]
                rows = torch.from_numpy(self.pool_rows(seq[g], pos[g])).to(self.device)
                self.pool[rows] = self.latent_rows(torch.from_numpy(g).to(self.device))
            self.append_tokens(last)
        else:
            self.append_tokens(np.arange(N))

    def append_tokens(self, ids: np.ndarray, chunk: int = 65536):
        """Run the append kernel for global token ids ``ids``."""
        seq, pos = self.token_rows()
        for i in range(0, ids.size, chunk):
            g = ids[i:i + chunk]
            h = self.h_rows(torch.from_numpy(g).to(self.device))
            self.mla.cache_append(self.dims, h, self.W_DKV, self.W_KR,
                                  torch.from_numpy(pos[g]).to(self.device), self.page_table, self.c_KV, self.k_R,
                                  self.row_stride, self.num_pages,
                                  seq_id=torch.from_numpy(seq[g]).to(self.device))

    # ---------------------------------------------------------------- run
    def decode(self, stream=None, ev_start=None, ev_stop=None, impl=0):
        self.mla.decode(self.dims, self.q_C, self.q_R, self.pos_q, self.W_UK, self.W_UV, self.c_KV, self.k_R,
                        self.row_stride, self.num_pages, self.page_table, self.seq_lens, self.out, self.lse,
                        self.workspace, self.n_splits, stream, ev_start, ev_stop, impl)

    def _newest_token_states(self):
        if not hasattr(self, "_step_h"):
            last = self.prefix[1:] - 1
            self._step_h = self.h_rows(torch.from_numpy(last).to(self.device))
            self._step_pos = self.pos_q.clone()
        return self._step_h

    def append_step(self, stream=None, use_workspace: bool = True):
        """The decode step's append: each sequence's newest token (position
        n_b - 1) is written again from its token state (with the append
        workspace when the library has a split path for this size)."""
        self._newest_token_states()
        if not hasattr(self, "_append_ws"):
            nws = self.mla.cache_append_workspace_size(self.dims, self.cfg.B)
            self._append_ws = torch.empty(nws, dtype=torch.uint8, device=self.device) if nws > 0 else None
        self.mla.cache_append(self.dims, self._step_h, self.W_DKV, self.W_KR, self._step_pos, self.page_table,
                              self.c_KV, self.k_R, self.row_stride, self.num_pages, stream=stream,
                              workspace=self._append_ws if use_workspace else None)

    def step(self, stream=None, ev_start=None, ev_stop=None, impl: int = 0):
        """One whole decode step through mla_decode_step: each sequence's
        newest token (position n_b - 1) is appended again from its token
        state, then every sequence is decoded."""
        h = self._newest_token_states()
        if not hasattr(self, "_step_ws"):
            self._step_ws = self.mla.decode_step_workspace(self.dims, self.cfg.B, self.n_splits, self.device)
        self.mla.decode_step(self.dims, h, self.W_DKV, self.W_KR, self.q_C, self.q_R, self.pos_q, self.W_UK,
                             self.W_UV, self.c_KV, self.k_R, self.row_stride, self.num_pages, self.page_table,
                             self.seq_lens, self.out, self.lse, self._step_ws, self.n_splits, stream, ev_start,
                             ev_stop, impl)

    # ---------------------------------------------------------------- oracle side (CPU, generator only)
    def oracle_inputs(self, b: int) -> dict:
        """fp64 numpy inputs of sequence b, regenerated on the CPU."""
        c = self.cfg
        g0, g1 = int(self.prefix[b]), int(self.prefix[b + 1])
        f64 = lambda t: t.to(torch.float64).numpy()  # noqa: E731
        cpu = torch.device("cpu")
        d = dict(W_UK=f64(self._W_UK(device=cpu)), W_UV=f64(self._w("W_UV", c.n_h * D_H, D_C, D_C, device=cpu)),
                 n=g1 - g0, pos_q=g1 - g0 - 1)
        if c.cache_mode == "direct":
            lat = f64(self.latent_rows(range(g0, g1 - 1), device=cpu))
            d["prior_c"], d["prior_kR"] = lat[:, :D_C], lat[:, D_C:]
            d["h_new"] = f64(self.h_rows(range(g1 - 1, g1), device=cpu))
        else:
            d["h"] = f64(self.h_rows(range(g0, g1), device=cpu))
        d["W_DKV"] = f64(self._w("W_DKV", D_C, c.d_model, c.d_model, device=cpu))
        d["W_KR"] = f64(self._w("W_KR", D_R, c.d_model, c.d_model, device=cpu))
        if c.query == "synthetic":
            rows = range(b * c.n_h, (b + 1) * c.n_h)
            d["q_C"] = f64(self._q_rows("q_C", rows, D_H, cpu))
            d["q_R"] = f64(self._q_rows("q_R", rows, D_R, cpu))
        return d


# ---------------------------------------------------------------------------- sparse decode inputs
D_I = 128    # indexer key width


def exact_small_ints(x: torch.Tensor) -> torch.Tensor:
    """Integers in [-3, 3] from N(0, 1) draws, by comparisons only."""
    return _steps(x, (0.5, 1.25, 2.0), 1.0)


class IndexerInputs:
    """Indexer keys, queries and head weights of the sparse decode for one
    Workload (same pages and page table).  Keys: one row of D_I per cached
    token, N(0, 1) from the generator (by global token id), in a pool of its
    own laid out like the latent pool.  q^I ~ N(0, 1) per (sequence, head);
    w_h = min(|x| / 4, 1) for x ~ N(0, 1) (non-negative gates).  exact: keys
    and q^I integers in [-3, 3], w_h multiples of 1/4 in [0, 2]; every score
    is then exact in fp32 whatever the summation order."""

    def __init__(self, wl: Workload, H_I: int = 64, exact: bool = False, name: str = "idx"):
        self.wl, self.H_I, self.exact = wl, H_I, exact
        c = wl.cfg
        self.key = lambda part: si.stream_key(c.seed, f"{c.name}/{name}/{part}", wl.layer)  # noqa: E731
        dev = wl.device
        ps = c.page_size
        self.pool = torch.zeros((wl.num_pages * ps, D_I), dtype=torch.bfloat16, device=dev)
        self.row_stride = D_I
        seq, pos = wl.token_rows()
        N = seq.size
        for i in range(0, N, 65536):
            g = np.arange(i, min(N, i + 65536))
            rows = torch.from_numpy(wl.pool_rows(seq[g], pos[g])).to(dev)
            self.pool[rows] = self.key_rows(torch.from_numpy(g).to(dev))
        self.q_I = self.query_rows(range(c.B * H_I), dev).reshape(c.B, H_I, D_I)
        self.w_I = self.weight_rows(range(c.B), dev)

    def key_rows(self, rows, device=None):
        x = si.normal_rows(self.key("k"), rows, D_I, 1.0, torch.float32, device or self.wl.device)
        return (exact_small_ints(x) if self.exact else x).to(torch.bfloat16)

    def query_rows(self, rows, device):
        x = si.normal_rows(self.key("q"), rows, D_I, 1.0, torch.float32, device)
        return (exact_small_ints(x) if self.exact else x).to(torch.bfloat16)

    def weight_rows(self, rows, device):
        x = si.normal_rows(self.key("w"), rows, self.H_I, 1.0, torch.float32, device).abs()
        if self.exact:
            return _steps(x, (0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0), 0.25).to(torch.float32)
        return torch.clamp(x * 0.25, max=1.0)

    def oracle_inputs(self, b: int) -> dict:
        """fp64 q^I, w, and the keys of sequence b's tokens 0 .. n_b - 1 (CPU)."""
        wl, cpu = self.wl, torch.device("cpu")
        g0, g1 = int(wl.prefix[b]), int(wl.prefix[b + 1])
        f64 = lambda t: t.to(torch.float64).numpy()  # noqa: E731
        return dict(q_I=f64(self.query_rows(range(b * self.H_I, (b + 1) * self.H_I), cpu)),
                    w_I=f64(self.weight_rows(range(b, b + 1), cpu))[0],
                    k_I=f64(self.key_rows(range(g0, g1), cpu)))
