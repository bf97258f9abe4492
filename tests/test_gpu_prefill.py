"""GPU parity of the chunked prefill (mla_prefill) against the fp64 oracle.

A chunk of new tokens, in any order and any mix of sequences, is appended and
each token attends causally to its sequence's rows up to its own position
(oracle.attend_causal_chunk).  Sequences already hold a prior context,
written with mla_cache_append; pages are a seeded permutation of the pool.
Tolerance as for the decode: max|gpu - oracle| / max|oracle| <= 1e-2 (bf16),
<= 1e-5 (fp32), on the outputs and on the appended cache rows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from cases import lse_err, rel_err

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 1e-2, torch.float32: 1e-5}
D_C, D_R, D_H = 512, 64, 128


def _say(msg):
    print(msg, flush=True)


class Chunk:
    """Pool, weights and prior context of B sequences plus a chunk of new tokens."""

    def __init__(self, seed, n_h, d_model, dtype, prior, chunk, page_size=64, shuffle=True, n_splits=0):
        import compressed_kv_cache_mla_amd as mla
        self.mla, self.seed, self.dtype = mla, seed, dtype
        self.dims = mla.Dims(n_h=n_h, d_model=d_model, page_size=page_size, dtype=dtype)
        self.prior, self.chunk = np.asarray(prior), np.asarray(chunk)
        self.n = self.prior + self.chunk
        B = len(prior)
        pages = (self.n + page_size - 1) // page_size
        self.max_pages, self.num_pages = int(pages.max()), int(pages.sum())
        order = si.permutation(seed, "pages", self.num_pages)
        pt = np.zeros((B, self.max_pages), dtype=np.int32)
        off = 0
        for b in range(B):
            pt[b, :pages[b]] = order[off:off + pages[b]]
            off += pages[b]
        self.pt_np = pt
        dev = "cuda"
        self.page_table = torch.from_numpy(pt).to(dev)
        self.pool = torch.zeros((self.num_pages * page_size, D_C + D_R), dtype=dtype, device=dev)
        self.offs = np.concatenate([[0], np.cumsum(self.n)])
        self.W = {k: self._w(k, r, c, dev) for k, (r, c) in self._wshapes().items()}
        # prior context through the append kernel
        seq = np.concatenate([np.full(self.prior[b], b) for b in range(B)]).astype(np.int32)
        pos = np.concatenate([np.arange(self.prior[b]) for b in range(B)]).astype(np.int32)
        if seq.size:
            g = np.concatenate([self.offs[b] + np.arange(self.prior[b]) for b in range(B)])
            mla.cache_append(self.dims, self._h(g, dev), self.W["W_DKV"], self.W["W_KR"],
                             torch.from_numpy(pos).to(dev), self.page_table, self.pool[:, :D_C], self.pool[:, D_C:],
                             D_C + D_R, self.num_pages, seq_id=torch.from_numpy(seq).to(dev))
        # the chunk, in a seeded order across sequences
        cs = np.concatenate([np.full(self.chunk[b], b) for b in range(B)]).astype(np.int32)
        cp = np.concatenate([self.prior[b] + np.arange(self.chunk[b]) for b in range(B)]).astype(np.int32)
        if shuffle:
            perm = si.permutation(seed, "chunk order", cs.size)
            cs, cp = cs[perm], cp[perm]
        self.c_seq, self.c_pos = cs, cp
        self.T = cs.size
        self.c_glob = self.offs[cs] + cp
        self.q_C = si.normal(si.stream_key(seed, "q_C"), (self.T, n_h, D_H), 1.0, dtype, dev)
        self.q_R = si.normal(si.stream_key(seed, "q_R"), (self.T, n_h, D_R), 1.0, dtype, dev)
        self.out = torch.full((self.T, n_h, D_H), float("nan"), dtype=torch.float32, device=dev)
        self.lse = torch.full((self.T, n_h), float("nan"), dtype=torch.float32, device=dev)
        self.n_splits = n_splits

    def _wshapes(self):
        nh, dm = self.dims.n_h, self.dims.d_model
        return {"W_DKV": (D_C, dm), "W_KR": (D_R, dm), "W_UK": (nh * D_H, D_C), "W_UV": (nh * D_H, D_C)}

    def _w(self, name, rows, cols, dev):
        return si.normal(si.stream_key(self.seed, name), (rows, cols), cols ** -0.5, self.dtype, dev)

    def _h(self, rows, dev):
        return si.normal_rows(si.stream_key(self.seed, "h"), torch.as_tensor(rows, dtype=torch.int64), self.dims.d_model,
                              1.0, self.dtype, dev)

    def run(self, seq_override=None):
        dev = "cuda"
        seq = self.c_seq if seq_override is None else seq_override
        self.ws = self.mla.prefill(self.dims, self._h(self.c_glob, dev), self.W["W_DKV"], self.W["W_KR"], self.q_C,
                                   self.q_R, torch.from_numpy(seq.astype(np.int32)).to(dev),
                                   torch.from_numpy(self.c_pos).to(dev), self.W["W_UK"], self.W["W_UV"],
                                   self.pool[:, :D_C], self.pool[:, D_C:], D_C + D_R, self.num_pages,
                                   self.page_table, self.out, self.lse, n_splits=self.n_splits)
        torch.cuda.synchronize()

    def oracle_seq(self, b, reconstruct=False):
        """(token indices of the chunk in sequence b, out, lse, cache rows) from the oracle."""
        cpu = torch.device("cpu")
        f = lambda t: t.to(torch.float64).numpy()  # noqa: E731
        W = {k: f(self._w(k, r, c, cpu)) for k, (r, c) in self._wshapes().items()}
        h = f(self._h(self.offs[b] + np.arange(self.n[b]), cpu))
        c, kR = oracle.down_project(h, W["W_DKV"], W["W_KR"], np.arange(self.n[b]), self.dims.rope_base)
        idx = np.nonzero(self.c_seq == b)[0]
        qC = f(self.q_C.cpu())[idx]
        qR = f(self.q_R.cpu())[idx]
        out, lse = oracle.attend_causal_chunk(qC, qR, self.c_pos[idx], c, kR, W["W_UK"], W["W_UV"],
                                              self.dims.rope_base, self.dims.scale, reconstruct=reconstruct)
        return idx, out, lse, np.concatenate([c, kR], axis=1)

    def gpu_rows(self, b, positions):
        ps = self.dims.page_size
        rows = self.pt_np[b, positions // ps].astype(np.int64) * ps + positions % ps
        return self.pool[torch.from_numpy(rows).cuda()].to(torch.float64).cpu().numpy()

    def check(self, seqs=None, reconstruct=False):
        tol = TOL[self.dtype]
        out, lse = self.out.cpu().numpy(), self.lse.cpu().numpy()
        for b in (range(len(self.n)) if seqs is None else seqs):
            idx, ref, ref_lse, rows = self.oracle_seq(b, reconstruct)
            if idx.size == 0:
                continue
            e = rel_err(out[idx], ref)
            assert e <= tol, f"seq {b}: out rel err {e:.3e}"
            el = lse_err(lse[idx], ref_lse)
            assert el <= tol, f"seq {b}: lse rel err {el:.3e}"
            new = self.c_pos[idx]
            e = rel_err(self.gpu_rows(b, new), rows[new])
            assert e <= tol, f"seq {b}: appended rows rel err {e:.3e}"


CASES = [
    # (name, n_h, d_model, dtype, prior, chunk, page_size)
    ("mixed_bf16", 128, 1024, torch.bfloat16, [100, 0, 257], [17, 40, 1], 64),
    ("long_chunk_h32", 32, 1024, torch.bfloat16, [600, 33], [64, 130], 64),
    ("pages16_valu", 64, 512, torch.bfloat16, [50, 7], [20, 9], 16),
    ("tiny_fp32", 16, 1024, torch.float32, [256, 3], [8, 5], 64),
]


@pytest.mark.parametrize("name,n_h,d_model,dtype,prior,chunk,page_size", CASES)
def test_prefill_matches_oracle(name, n_h, d_model, dtype, prior, chunk, page_size):
    _say(f"case prefill {name}")
    c = Chunk(900 + len(name), n_h, d_model, dtype, prior, chunk, page_size)
    c.run()
    assert c.mla.read_error_flags(c.ws) == 0
    c.check()
    first = c.out.clone()
    c.run()                                         # same inputs (rows rewritten with the same values): same bits
    assert torch.equal(first, c.out)


def test_prefill_reconstruct_mode_sample():
    _say("case prefill reconstruct")
    c = Chunk(77, 128, 1024, torch.bfloat16, [300], [24], 64)
    c.run()
    c.check(reconstruct=True)


def test_prefill_deepseek_sizes_sampled():
    """d_model = 5120, n_h = 128: a 4096-token prior and a 128-token chunk of one
    sequence plus a 32-token chunk of a second; every token checked against the
    absorbed oracle."""
    _say("case prefill deepseek sizes")
    c = Chunk(78, 128, 5120, torch.bfloat16, [4096, 1000], [128, 32], 64)
    c.run()
    assert c.mla.read_error_flags(c.ws) == 0
    c.check()


@pytest.mark.parametrize("prior,chunk", [([300], [512]), ([300, 20], [400, 50])])
def test_prefill_long_chunk_shares_the_absorption_weights(prior, chunk):
    """512 (or 450, in two sequences) new tokens after a short prior (n_h =
    128): the absorption then lets each W^UK block serve several 64-token
    blocks, and the combine merges 64 queries per workgroup (450: a last
    block of 2); every token checked."""
    _say(f"case prefill long chunk {prior} {chunk}")
    c = Chunk(81, 128, 1024, torch.bfloat16, prior, chunk, 64)
    c.run()
    assert c.mla.read_error_flags(c.ws) == 0
    c.check()


def test_prefill_one_token_per_sequence_equals_decode():
    """One new token per sequence is the decode of that token: mla_prefill
    against mla_cache_append + mla_decode on the same inputs (within the bf16
    bound; the append kernels differ in summation order)."""
    import compressed_kv_cache_mla_amd as mla
    _say("case prefill vs decode")
    c = Chunk(79, 128, 1024, torch.bfloat16, [100, 300, 64], [1, 1, 1], 64, shuffle=False)
    c.run()
    pre = c.out.clone()
    out = torch.empty_like(c.out)
    seq_lens = torch.from_numpy((c.c_pos + 1).astype(np.int32)).cuda()
    mla.decode(c.dims, c.q_C, c.q_R, torch.from_numpy(c.c_pos).cuda(), c.W["W_UK"], c.W["W_UV"], c.pool[:, :D_C],
               c.pool[:, D_C:], D_C + D_R, c.num_pages, c.page_table, seq_lens, out)
    torch.cuda.synchronize()
    assert rel_err(pre.cpu().numpy(), out.cpu().numpy()) < 1e-2


def test_prefill_flags_a_bad_sequence_id():
    _say("case prefill bad sequence id")
    c = Chunk(80, 32, 1024, torch.bfloat16, [40, 70], [5, 6], 64)
    seq = c.c_seq.copy()
    bad = int(np.nonzero(seq == 1)[0][0])
    seq[bad] = 7                                    # no such sequence
    c.run(seq_override=seq)
    flags = c.mla.read_error_flags(c.ws)
    assert flags & c.mla.FLAG_BAD_SEQ_ID and flags & c.mla.FLAG_BAD_SEQ_LEN
    out = c.out.cpu().numpy()
    assert np.all(out[bad] == 0) and np.all(np.isneginf(c.lse.cpu().numpy()[bad]))
    c.check(seqs=[0])                               # the other sequence is untouched by the bad token


def test_prefill_rows_after_a_token_do_not_change_it():
    """Causality on the GPU: rewriting the pool rows after a token's position
    (here: the last 10 positions of the sequence) leaves that token's output
    bit for bit unchanged when the chunk is run again with the later tokens
    given other states."""
    _say("case prefill no future leak")
    c = Chunk(82, 32, 1024, torch.bfloat16, [200], [40], 64, shuffle=False)
    c.run()
    before = c.out.clone()
    # other token states for the last 10 new tokens: their rows (positions 230..239) change
    c.c_glob = c.c_glob.copy()
    c.c_glob[-10:] += 100000
    c.run()
    after = c.out
    assert torch.equal(before[:30], after[:30])
    assert not torch.equal(before[30:], after[30:])
