#!/usr/bin/env python3
"""Benchmark of the MLA decode hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input: the
append of each sequence's newest token (W^DKV down-projection + RoPE'd k^R
into the paged latent cache) followed by mla_decode (plan, absorb, split-KV
attention over the latent cache, combine, W^UV epilogue).  Inputs are
resident in HBM before timing starts.  To keep the 256 MB Infinity Cache from
serving repeated reads, steps rotate over several independent copies of the
workload (own weights, queries and cache) whose total size exceeds it.
Before its warm-up steps each measurement runs the same calls back to back,
untimed, for --settle seconds (default 0.5), so that the GPU, idle during
the workload's set-up, has reached its steady clocks when timing starts.

Prints one JSON line.  The headline workload is batch 64 at 8K context
(b64_l8192); `value` is its decode tokens/s (B sequences per step);
`roofline` is computed for the split-KV attention kernel from its algorithmic
bytes and its HIP-event duration measured in the timed region; `configs`
repeats the measurement on the other single-layer decode configurations
(batch 32 at 4K, batch 64 ragged over permuted pages, batch 4 at 128K);
`l60` times the 60-layer configuration (batch 128 at 8K, every layer's
append + decode) as one captured HIP graph; `projections` times the query
path (W^DQ, W^UQ, W^QR) and the output projection W^O, which sit outside the
step; `prefill` times chunked prefill (new tokens attending causally over
their sequences); `layer` times the whole attention layer (query path + step
+ W^O, h -> u); `sparse` times the sparse top-k decode (indexer, selection,
attention over the kept rows) at batch 4 x 128K and batch 64 x 8K with
top_k = 2048; `cpu_baseline` times the fp64 CPU oracle on one whole decode
step of the headline workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode tokens/s + latent-cache GB/s (% of HBM/MFMA roofline), 1 GPU"
PREFILL_CONFIGS = [(1, 4096, 512), (8, 2048, 64)]     # (sequences, prior tokens, new tokens per sequence)
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
COUNTERS = os.path.join(ROOT, "profiles", "decode_attention_counters.json")
KERNEL_SRC = os.path.join(ROOT, "compressed_kv_cache_mla_amd", "csrc", "decode_mfma.hip")


def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


COUNTER_WORKLOADS = ("b64_l8192", "b32_l4096", "b64_ragged", "b4_l131072")
PMC_CMD = ("cd /tmp && timeout -s KILL 120 rocprofv3 --pmc {ctr} --kernel-include-regex {regex} --output-format csv "
           "-d <out>/{name} -o run -- python3 <repo>/bench.py {args}")
PMC_BENCH_ARGS = "--no-cpu-baseline --no-extras --no-l60 --configs '' --workload {w} --steps 3 --warmup 1 --settle 0"


def write_counters(out_dir: str):
    """profiles/decode_attention_counters.json from rocprofv3 counter passes
    already run into out_dir (the commands recorded in the file): the copy
    calibration of FETCH_SIZE and WRITE_SIZE (a plain 1 GiB device copy) and
    both counters on the attention kernel of each workload.  Counter values
    are averaged over the kernel's dispatches."""
    import csv
    import glob

    def per_dispatch(name, counter, regex):
        files = glob.glob(os.path.join(out_dir, name, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter output under {out_dir}/{name}")
        vals = {}
        for row in csv.DictReader(open(files[0])):
            if row["Counter_Name"] == counter and regex in row["Kernel_Name"]:
                vals[row["Dispatch_Id"]] = vals.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
        if not vals:
            raise SystemExit(f"no {counter} values for {regex} in {files[0]}")
        return sum(vals.values()) / len(vals), len(vals)

    copy_bytes = 1 << 30
    cal = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        kib, _ = per_dispatch("copy_" + ctr.split("_")[0].lower(), ctr, "copyBuffer")
        cal[ctr] = {"copy_bytes": copy_bytes, "counter_kib_per_copy": round(kib, 1),
                    "bytes_per_counted_kib": round(copy_bytes / kib, 4)}
    wl = {}
    for w in COUNTER_WORKLOADS:
        f, n = per_dispatch(f"{w}_fetch", "FETCH_SIZE", "decode_mfma")
        wr, _ = per_dispatch(f"{w}_write", "WRITE_SIZE", "decode_mfma")
        rd = f * cal["FETCH_SIZE"]["bytes_per_counted_kib"]
        wb = wr * cal["WRITE_SIZE"]["bytes_per_counted_kib"]
        wl[w] = {"fetch_kib_per_launch": round(f, 1), "write_kib_per_launch": round(wr, 1),
                 "hbm_read_bytes": int(rd), "hbm_write_bytes": int(wb), "hbm_bytes_per_launch": int(rd + wb),
                 "launches": n}
    cmds = {}
    for w in COUNTER_WORKLOADS:
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            name = f"{w}_{ctr.split('_')[0].lower()}"
            cmds[name] = PMC_CMD.format(ctr=ctr, regex="decode_mfma", name=name, args=PMC_BENCH_ARGS.format(w=w))
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        name = "copy_" + ctr.split("_")[0].lower()
        cmds[name] = PMC_CMD.format(ctr=ctr, regex="copyBuffer", name=name, args="--copy-calibration")
    cmds["summary"] = f"python3 <repo>/bench.py --write-counters <out>"
    res = {"kernel": "decode_mfma_kernel<4> (split-KV attention)", "kernel_source_sha256_16": kernel_source_hash(),
           "calibration": cal, "workloads": wl, "commands": cmds}
    with open(COUNTERS, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res["workloads"]), flush=True)


def algorithmic(wl):
    """Algorithmic bytes and flops of one step and of one launch of the
    split-KV attention kernel."""
    c = wl.cfg
    N = int(wl.prefix[-1])
    B, nh, dm = c.B, c.n_h, c.d_model
    s = 2 if c.dtype.itemsize == 2 else 4
    cache = N * 576 * s
    attn_bytes = cache + B * nh * 576 * s + B * nh * (512 * 4 + 8)       # rows + q~ in, O~ + (m, l) out
    attn_flops = N * nh * (2 * 576 + 2 * 512)
    step_bytes = (cache + 2 * nh * 128 * 512 * s          # W^UK, W^UV
                  + 576 * dm * s + B * dm * s + B * 576 * s  # W^DKV|W^KR, h, new rows
                  + B * nh * (128 + 64) * s + B * nh * (128 + 1) * 4)   # q^C, q^R in; out, lse
    step_flops = attn_flops + B * 4 * nh * 128 * 512 + B * 2 * dm * 576
    return dict(N=N, cache=cache, attn_bytes=attn_bytes, attn_flops=attn_flops, step_bytes=step_bytes,
                step_flops=step_flops)


def measured_copy_gbps(torch) -> float:
    """A second denominator beside the spec peak: read + write bytes per
    second of a plain 1 GiB device-to-device copy on this GPU (best of 5)."""
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    best = float("inf")
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        y.copy_(x)
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    del x, y
    return 2 * n / (best * 1e-3) / 1e9


SETTLE_S = 0.5   # default; --settle


def settle(torch, fn, seconds: float) -> int:
    """Run fn(i) (one whole call of what is about to be timed) back to back
    for about `seconds` of wall time, before the warm-up and the timed calls.
    An MI355X coming from idle (workload set-up leaves it idle for seconds)
    takes some tens of milliseconds of load to reach its steady clocks: at
    B = 64, L = 8192 the first 50 steps after 6 warm-up steps averaged 224 us,
    later blocks of 50 fell to 194 us after about 400 steps, with or without
    events recorded inside them.  Untimed, like the warm-up; the timed region
    still holds exactly the requested steps.  Returns the calls made."""
    t0 = time.perf_counter()
    n = 0
    while seconds > 0:
        for _ in range(16):
            fn(n)
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break
    return n


def measure_projections(torch, mla, B: int, n_h: int = 128, d_model: int = 5120, d_cq: int = 1536, reps: int = 20):
    """The weight-streaming projections around the attention at batch B
    (DeepSeek-V2 sizes; d_cq = 1536, a choice: the pages give no query rank):
    mla_query_project (W^DQ, W^UQ, W^QR) and mla_output_project (W^O), each
    timed with fence-free HIP events per call over three rotating weight sets
    (about 1 GB, past the Infinity Cache).  Algorithmic bytes = weights +
    activations in and out."""
    import seeded_inputs as si
    dims = mla.Dims(n_h=n_h, d_model=d_model)
    bf = torch.bfloat16

    def w(seed, name, rows, cols):
        return mla.pack_weight(dims, si.normal(si.stream_key(seed, name), (rows, cols), cols ** -0.5, bf, "cuda"))

    sets = []
    for i in range(3):
        seed = 4242 + i
        sets.append(dict(h=si.normal(si.stream_key(seed, "h"), (B, d_model), 1.0, bf, "cuda"),
                         W_DQ=w(seed, "W_DQ", d_cq, d_model), W_UQ=w(seed, "W_UQ", n_h * 128, d_cq),
                         W_QR=w(seed, "W_QR", n_h * 64, d_model), W_O=w(seed, "W_O", d_model, n_h * 128),
                         o=si.normal(si.stream_key(seed, "o"), (B, n_h, 128), 1.0, torch.float32, "cuda")))
    q_C = torch.empty((B, n_h, 128), dtype=bf, device="cuda")
    q_R = torch.empty((B, n_h, 64), dtype=bf, device="cuda")
    u = torch.empty((B, d_model), dtype=torch.float32, device="cuda")
    wq = mla.query_project_workspace(dims, B, d_cq)
    wo = mla.output_project_workspace(dims, B)
    q_bytes = 2 * (d_cq * d_model + n_h * 128 * d_cq + n_h * 64 * d_model) + 2 * B * d_model + 2 * B * n_h * 192
    o_bytes = 2 * d_model * n_h * 128 + 4 * B * n_h * 128 + 4 * B * d_model
    out = {}
    for name, fn, nbytes in (
            ("query_project", lambda x: mla.query_project(dims, x["h"], x["W_DQ"], x["W_UQ"], x["W_QR"], q_C, q_R, wq),
             q_bytes),
            ("output_project", lambda x: mla.output_project(dims, x["o"], x["W_O"], u, wo), o_bytes)):
        settle(torch, lambda i: fn(sets[i % 3]), SETTLE_S)
        for i in range(6):
            fn(sets[i % 3])
        torch.cuda.synchronize()
        evs = [(mla.HipEvent(), mla.HipEvent()) for _ in range(reps)]
        for i, (a, b) in enumerate(evs):
            a.record()
            fn(sets[i % 3])
            b.record()
        torch.cuda.synchronize()
        us = float(np.median([1e3 * a.elapsed_ms(b) for a, b in evs]))
        gbps = nbytes / (us * 1e-6) / 1e9
        out[name] = {"B": B, "us_p50": round(us, 2), "alg_MB": round(nbytes / 1e6, 1), "GBps": round(gbps, 1),
                     "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
    del sets
    torch.cuda.empty_cache()
    return out


def measure_layer(torch, mla, W, name: str, d_cq: int = 1536, reps: int = 20, copies: int = 2):
    """One whole MLA attention layer per decode token (mla_decode_layer: query
    projection, decode step, output projection, h -> u) on a workload, over
    rotating copies with their own weights; HIP events per call, median."""
    import seeded_inputs as si
    cfg = W.CONFIGS[name]
    wls = [W.Workload(cfg, layer=i) for i in range(copies)]
    dims, nh, dm, B = wls[0].dims, cfg.n_h, cfg.d_model, cfg.B
    runs = []
    for i, wl in enumerate(wls):
        key = lambda nm: si.stream_key(cfg.seed + 77, nm, i)  # noqa: E731
        pw = lambda nm, r, c: mla.pack_weight(dims, si.normal(key(nm), (r, c), c ** -0.5, torch.bfloat16, "cuda"))  # noqa
        P = dict(W_DQ=pw("W_DQ", d_cq, dm), W_UQ=pw("W_UQ", nh * 128, d_cq), W_QR=pw("W_QR", nh * 64, dm),
                 W_O=pw("W_O", dm, nh * 128))
        u = torch.empty((B, dm), dtype=torch.float32, device="cuda")
        ws = mla.decode_layer_workspace(dims, B, d_cq)
        h = wl._newest_token_states()

        def call(wl=wl, P=P, u=u, ws=ws, h=h):
            mla.decode_layer(dims, h, wl.W_DKV, wl.W_KR, P["W_DQ"], P["W_UQ"], P["W_QR"], wl.W_UK, wl.W_UV, P["W_O"],
                             wl.pos_q, wl.c_KV, wl.k_R, wl.row_stride, wl.num_pages, wl.page_table, wl.seq_lens, u,
                             wl.lse, ws)
        runs.append(call)
    settle(torch, lambda i: runs[i % copies](), SETTLE_S)
    for i in range(4):
        runs[i % copies]()
    torch.cuda.synchronize()
    evs = [(mla.HipEvent(), mla.HipEvent()) for _ in range(reps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        runs[i % copies]()
        b.record()
    torch.cuda.synchronize()
    us = float(np.median([1e3 * a.elapsed_ms(b) for a, b in evs]))
    alg = algorithmic(wls[0])
    nbytes = alg["step_bytes"] + 2 * (d_cq * dm + nh * 128 * d_cq + nh * 64 * dm + dm * nh * 128) + 4 * B * dm
    del wls, runs
    torch.cuda.empty_cache()
    return {"workload": name, "B": B, "d_cq": d_cq, "us_p50": round(us, 1), "tokens_per_s": round(B / (us * 1e-6), 1),
            "alg_MB": round(nbytes / 1e6, 1), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}


def measure_prefill(torch, mla, B: int, L: int, T: int, n_h: int = 128, d_model: int = 5120, reps: int = 10):
    """Chunked prefill (mla_prefill) of T new tokens per sequence after an
    L-token prior, B sequences, DeepSeek-V2 sizes, 64-token pages in order.
    Each call appends the chunk again at the same positions (same values) and
    runs the causal attention; timed with fence-free HIP events per call.
    Algorithmic flops: the attention's n_h * (2*576 + 2*512) per (query,
    visible row) pair, plus the append (2 * d_model * 576 per token),
    absorption and W^UV (2 * 2 * n_h * 128 * 512 per token)."""
    import seeded_inputs as si
    bf = torch.bfloat16
    ps = 64
    dims = mla.Dims(n_h=n_h, d_model=d_model, page_size=ps)
    n = L + T
    max_pages = (n + ps - 1) // ps
    num_pages = B * max_pages
    pt = torch.arange(num_pages, dtype=torch.int32, device="cuda").reshape(B, max_pages)
    pool = torch.empty((num_pages * ps, 576), dtype=bf, device="cuda")
    key = lambda name: si.stream_key(4321, name)  # noqa: E731
    W_DKV = si.normal(key("W_DKV"), (512, d_model), d_model ** -0.5, bf, "cuda")
    W_KR = si.normal(key("W_KR"), (64, d_model), d_model ** -0.5, bf, "cuda")
    W_UK = si.normal(key("W_UK"), (n_h * 128, 512), 512 ** -0.5, bf, "cuda")
    W_UV = si.normal(key("W_UV"), (n_h * 128, 512), 512 ** -0.5, bf, "cuda")
    seq = torch.arange(B, dtype=torch.int32, device="cuda").repeat_interleave(n)
    pos = torch.arange(n, dtype=torch.int32, device="cuda").repeat(B)
    h = si.normal(key("h"), (B * n, d_model), 1.0, bf, "cuda")
    mla.cache_append(dims, h, W_DKV, W_KR, pos, pt, pool[:, :512], pool[:, 512:], 576, num_pages, seq_id=seq)
    last = (torch.arange(B * n, device="cuda") % n) >= L
    c_h, c_seq, c_pos = h[last].contiguous(), seq[last].contiguous(), pos[last].contiguous()
    q_C = si.normal(key("q_C"), (B * T, n_h, 128), 1.0, bf, "cuda")
    q_R = si.normal(key("q_R"), (B * T, n_h, 64), 1.0, bf, "cuda")
    out = torch.empty((B * T, n_h, 128), dtype=torch.float32, device="cuda")
    ws = torch.zeros(mla.prefill_workspace_size(dims, B * T, max_pages), dtype=torch.uint8, device="cuda")

    def call():
        mla.prefill(dims, c_h, W_DKV, W_KR, q_C, q_R, c_seq, c_pos, W_UK, W_UV, pool[:, :512], pool[:, 512:], 576,
                    num_pages, pt, out, workspace=ws)

    settle(torch, lambda i: call(), SETTLE_S)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    evs = [(mla.HipEvent(), mla.HipEvent()) for _ in range(reps)]
    for a, b in evs:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    us = float(np.median([1e3 * a.elapsed_ms(b) for a, b in evs]))
    pairs = B * (T * L + T * (T + 1) // 2)
    flops = pairs * n_h * (2 * 576 + 2 * 512) + B * T * (2 * d_model * 576 + 4 * n_h * 128 * 512)
    tf = flops / (us * 1e-6) / 1e12
    return {"B": B, "prior_tokens": L, "chunk_tokens": T, "us_p50": round(us, 1),
            "tokens_per_s": round(B * T / (us * 1e-6), 1), "TFLOPs": round(tf, 1),
            "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)}


def _host_threads():
    """Threads the fp64 oracle's BLAS calls use, and the host's CPU counts."""
    from threadpoolctl import threadpool_info
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return threads, os.cpu_count(), len(os.sched_getaffinity(0))


def cpu_baseline(W, name: str, seconds: float, step_us_gpu: float | None = None):
    """The fp64 oracle as it stands, timed on the host on the work of one
    decode step of workload `name`: for every sequence b, append its newest
    token (oracle.down_project) and decode it (oracle.attend_absorbed) over
    n_b cached rows.  Its inputs are one sequence's regenerated seeded inputs
    (queries, W^DKV, W^KR, W^UK, W^UV, the newest token's h) and n_max
    seeded N(0, 1) latent rows (numpy PCG64), each sequence of the batch
    taking the first n_b of them: the oracle's cost depends only on the
    shapes.  Steps are repeated while the time budget lasts (at least one);
    value = B / median step time.  reconstruct: the definition (K and V
    rebuilt per head) on one sequence of the workload for two heads, reported
    per cached token and head."""
    import oracle
    cfg = W.CONFIGS[name]
    L = cfg.context_lengths()
    n = (L + 1).astype(np.int64)
    n_max = int(n.max())
    wl_cpu = W.Workload.__new__(W.Workload)     # generator side only: no device tensors
    wl_cpu.cfg, wl_cpu.layer = cfg, 0
    import torch
    cpu = torch.device("cpu")
    f64 = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    W_UK = f64(wl_cpu._W_UK(device=cpu))
    W_UV = f64(wl_cpu._w("W_UV", cfg.n_h * 128, 512, 512, device=cpu))
    W_DKV = f64(wl_cpu._w("W_DKV", 512, cfg.d_model, cfg.d_model, device=cpu))
    W_KR = f64(wl_cpu._w("W_KR", 64, cfg.d_model, cfg.d_model, device=cpu))
    q_C = f64(wl_cpu._q_rows("q_C", range(cfg.n_h), 128, cpu))
    q_R = f64(wl_cpu._q_rows("q_R", range(cfg.n_h), 64, cpu))
    h_new = f64(wl_cpu.h_rows(range(1), device=cpu))
    rng = np.random.default_rng(cfg.seed)
    c_all = rng.standard_normal((n_max, 512))
    k_all = rng.standard_normal((n_max, 64))
    base, scale = 10000.0, 1.0 / math.sqrt(192.0)
    threads, nproc, affinity = _host_threads()

    def step():
        for b in range(cfg.B):
            nb = int(n[b])
            c1, k1 = oracle.down_project(h_new, W_DKV, W_KR, np.array([nb - 1]), base)
            c = c_all[:nb].copy()
            k = k_all[:nb].copy()
            c[nb - 1:], k[nb - 1:] = c1, k1
            oracle.attend_absorbed(q_C, q_R, nb - 1, c, k, W_UK, W_UV, base, scale)

    times, t_end = [], time.perf_counter() + seconds
    while True:
        t0 = time.perf_counter()
        step()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() + times[-1] > t_end or len(times) >= 5:
            break
    t_step = float(np.median(times))
    # the definition: per-head K, V rebuilt from the latent
    nr = min(n_max, 8193)
    t0 = time.perf_counter()
    oracle.attend_reconstruct(q_C, q_R, nr - 1, c_all[:nr], k_all[:nr], W_UK, W_UV, base, scale, heads=[0, 1])
    t_rec = time.perf_counter() - t0
    res = {"value": round(cfg.B / t_step, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"fp64 absorbed-form oracle on the whole of one decode step of {name} "
                     f"(B={cfg.B}, {int(n.sum())} cached tokens, n_h={cfg.n_h}): append of each newest token "
                     f"then decode; {len(times)} step(s), median {t_step:.2f} s; inputs: one sequence's seeded "
                     f"queries and weights and {n_max} seeded latent rows shared by the batch",
           "step_s": round(t_step, 3), "steps_timed": len(times), "host_nproc": nproc, "host_affinity": affinity,
           "reconstruct": {"us_per_cached_token_per_head": round(1e6 * t_rec / (nr * 2), 3),
                           "tokens_per_s_all_heads": round(1.0 / (t_rec / 2 * cfg.n_h), 4),
                           "sample": f"oracle.attend_reconstruct, one sequence of {nr} cached tokens, 2 heads, "
                                     f"{t_rec:.2f} s; tokens/s extrapolated to n_h={cfg.n_h}"}}
    if step_us_gpu:
        res["gpu_over_cpu"] = round(t_step / (step_us_gpu * 1e-6), 1)
    return res


SPARSE_CONFIGS = [("b4_l131072", 2048), ("b64_l8192", 2048)]   # (workload, top_k)


def measure_sparse(torch, mla, W, name: str, top_k: int, H_I: int = 64, reps: int = 20, copies: int = 3):
    """The sparse top-k decode (mla_sparse_decode) on a decode workload: the
    indexer scores every cached token (H_I heads, 128-wide bf16 keys), each
    sequence keeps its top_k, and the attention runs over the kept latent
    rows.  Copies rotate as for the dense steps (the 134 MB of indexer keys of
    one copy would fit the Infinity Cache).  Each call is timed with fence-free
    HIP events; the gather attention kernel with the events the library
    records around it; the selection alone (mla_indexer_select) separately."""
    cfg = W.CONFIGS[name]
    t0 = time.perf_counter()
    wls = [W.Workload(cfg, layer=i) for i in range(copies)]
    idxs = [W.IndexerInputs(wl, H_I=H_I) for wl in wls]
    B, dev = cfg.B, wls[0].device
    wss = [torch.empty(mla.sparse_decode_workspace_size(wl.dims, B, wl.max_pages, top_k), dtype=torch.uint8,
                       device=dev) for wl in wls]
    torch.cuda.synchronize()
    build_s = time.perf_counter() - t0

    def run(i, ev=(None, None)):
        wl, ix = wls[i % copies], idxs[i % copies]
        mla.sparse_decode(wl.dims, wl.q_C, wl.q_R, wl.pos_q, wl.W_UK, wl.W_UV, wl.c_KV, wl.k_R, wl.row_stride,
                          wl.num_pages, wl.page_table, wl.seq_lens, ix.q_I, ix.w_I, ix.pool, ix.row_stride, top_k,
                          wl.out, wl.lse, workspace=wss[i % copies], ev_start=ev[0], ev_stop=ev[1])

    settle(torch, run, SETTLE_S)
    for i in range(3):
        run(i)
    torch.cuda.synchronize()
    sev = [mla.HipEvent() for _ in range(reps + 1)]
    kev = [(mla.HipEvent(), mla.HipEvent()) for _ in range(reps)]
    for i in range(reps):
        sev[i].record()
        run(i, kev[i])
    sev[reps].record()
    torch.cuda.synchronize()
    step_us = [1e3 * sev[i].elapsed_ms(sev[i + 1]) for i in range(reps)]
    attn_us = [1e3 * a.elapsed_ms(b) for a, b in kev]
    # the selection alone
    max_tokens = wls[0].max_pages * cfg.page_size
    scores = torch.empty((B, max_tokens), dtype=torch.float32, device=dev)
    st = torch.empty((B, top_k), dtype=torch.int32, device=dev)
    sr = torch.empty((B, top_k), dtype=torch.int32, device=dev)
    fl = torch.zeros(1, dtype=torch.int32, device=dev)
    sws = torch.empty(mla.indexer_select_workspace_size(B, wls[0].max_pages, cfg.page_size, top_k),
                      dtype=torch.uint8, device=dev)

    def sel(i):
        wl, ix = wls[i % copies], idxs[i % copies]
        mla.indexer_select(ix.q_I, ix.w_I, ix.pool, ix.row_stride, wl.num_pages, cfg.page_size, wl.page_table,
                           wl.seq_lens, top_k, scores, st, sr, fl, workspace=sws)

    for i in range(3):
        sel(i)
    sev2 = [mla.HipEvent() for _ in range(reps + 1)]
    torch.cuda.synchronize()
    for i in range(reps):
        sev2[i].record()
        sel(i)
    sev2[reps].record()
    torch.cuda.synchronize()
    sel_us = [1e3 * sev2[i].elapsed_ms(sev2[i + 1]) for i in range(reps)]
    N = int(wls[0].prefix[-1])
    kept = int(np.minimum(wls[0].n, top_k).sum())
    idx_bytes = N * (128 * 2 + 4)                       # keys in, scores out
    attn_bytes = kept * 576 * 2 + B * cfg.n_h * (576 * 2 + 512 * 2 + 8)
    t_step, t_attn, t_sel = (float(np.median(x)) for x in (step_us, attn_us, sel_us))
    res = {"workload": name, "B": B, "top_k": top_k, "H_I": H_I, "d_I": 128, "cached_tokens": N, "kept_tokens": kept,
           "us_per_step_p10_p50_p90": [round(float(x), 1) for x in np.percentile(step_us, [10, 50, 90])],
           "tokens_per_s": round(B / (t_step * 1e-6), 1),
           "select_us_p50": round(t_sel, 1), "select_GBps": round(idx_bytes / (t_sel * 1e-6) / 1e9, 1),
           "attention_us_p50": round(t_attn, 1),
           "attention_GBps": round(attn_bytes / (t_attn * 1e-6) / 1e9, 1),
           "alg_bytes": {"indexer_keys_and_scores": idx_bytes, "attention": attn_bytes},
           "copies_rotated": copies, "build_s": round(build_s, 1)}
    del wls, idxs, wss
    torch.cuda.empty_cache()
    return res


def measure_l60(torch, mla, W, steps: int, warmup: int, n_splits: int = 0):
    """The 60-layer configuration: B = 128 sequences of 8192 prior tokens, 60
    layers with their own seeded weights, queries and latent caches (72.5 GB
    of cache in all), one step = for every layer the append of each
    sequence's newest token and the decode (mla_decode_step).  The 60 layer
    steps are captured once in a HIP graph (three kernel launches per layer,
    no memset nodes) and the graph is replayed; each replay is timed with
    fence-free HIP events.  value: B / step time."""
    cfg = W.CONFIGS["l60_b128_l8192"]
    t0 = time.perf_counter()
    layers = []
    for i in range(cfg.layers):
        wl = W.Workload(W.scaled(cfg, layers=1), layer=i, n_splits=n_splits)
        wl.step()          # creates the zero-filled step workspace outside the capture
        layers.append(wl)
    torch.cuda.synchronize()
    build_s = time.perf_counter() - t0
    alg = [algorithmic(wl) for wl in layers]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for wl in layers:  # one eager pass on the capture stream first
            wl.step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref_out = layers[-1].out.clone()
    with torch.cuda.graph(g):
        for wl in layers:
            wl.step()
    settle(torch, lambda i: g.replay(), SETTLE_S)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(layers[-1].out, ref_out))
    evs = [(mla.HipEvent(), mla.HipEvent()) for _ in range(steps)]
    for a, b in evs:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    us = [1e3 * a.elapsed_ms(b) for a, b in evs]
    t = float(np.median(us))
    step_bytes = sum(a["step_bytes"] for a in alg)
    cache = sum(a["cache"] for a in alg)
    res = {"workload": cfg.name, "B": cfg.B, "layers": cfg.layers, "cached_tokens_per_layer": alg[0]["N"],
           "us_per_step_p10_p50_p90": [round(float(x), 1) for x in np.percentile(us, [10, 50, 90])],
           "tokens_per_s": round(cfg.B / (t * 1e-6), 1), "alg_GB_per_step": round(step_bytes / 1e9, 2),
           "cache_GB": round(cache / 1e9, 2), "step_GBps": round(step_bytes / (t * 1e-6) / 1e9, 1),
           "step_hbm_frac": round(step_bytes / (t * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
           "graph": "60 layer steps, 180 kernel nodes, captured once", "replay_equals_eager": same,
           "build_s": round(build_s, 1)}
    del layers, g
    torch.cuda.empty_cache()
    return res


def main():
    global SETTLE_S
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed back-to-back calls before each warm-up, so that the GPU runs at its "
                         "steady clocks (0 = none)")
    ap.add_argument("--workload", default="b64_l8192",
                    help="headline workload (default: batch 64, 8K context, the shape the target is stated on)")
    ap.add_argument("--configs", default="b32_l4096,b64_ragged,b4_l131072",
                    help="comma-separated workloads timed the same way under `configs` ('' to skip)")
    ap.add_argument("--no-l60", action="store_true", help="skip the 60-layer configuration (HIP graph)")
    ap.add_argument("--copies", type=int, default=0, help="workload copies to rotate over (0 = enough to exceed "
                                                         "the 256 MB Infinity Cache twice)")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--impl", type=int, default=0, help="0 = MFMA attention kernel, 1 = VALU reference kernel")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the next rows' timings (query / output projections, prefill, whole layer)")
    ap.add_argument("--prefill-only", action="store_true", help="only time the chunked prefill configurations")
    ap.add_argument("--layer-only", default="", help="comma-separated workloads: only time the whole decode layer")
    ap.add_argument("--projections-only", default="",
                    help="comma-separated batch sizes: only time the query / output projections at them")
    ap.add_argument("--l60-only", action="store_true", help="only time the 60-layer configuration")
    ap.add_argument("--sparse-only", action="store_true", help="only time the sparse top-k decode configurations")
    ap.add_argument("--write-counters", default="", metavar="DIR",
                    help="write profiles/decode_attention_counters.json from the rocprofv3 counter passes in DIR "
                         "(the commands it records) and exit; needs no GPU")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (reference for the HBM "
                         "byte counters of rocprofv3)")
    args = ap.parse_args()
    SETTLE_S = args.settle
    if args.write_counters:
        write_counters(args.write_counters)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library and this benchmark run on one GPU; multi-GPU runs are not supported "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = 1 << 30
        x = torch.full((n,), 1, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)
        return
    import workloads as W
    import compressed_kv_cache_mla_amd as mla
    if args.layer_only:
        print(json.dumps({"layer": [measure_layer(torch, mla, W, n) for n in args.layer_only.split(",")]}), flush=True)
        return
    if args.prefill_only:
        print(json.dumps({"prefill": [measure_prefill(torch, mla, *cfg) for cfg in PREFILL_CONFIGS]}), flush=True)
        return
    if args.projections_only:
        print(json.dumps({f"B{b}": measure_projections(torch, mla, int(b))
                          for b in args.projections_only.split(",")}), flush=True)
        return
    if args.sparse_only:
        print(json.dumps({"sparse": [measure_sparse(torch, mla, W, n, k) for n, k in SPARSE_CONFIGS]}), flush=True)
        return
    if args.l60_only:
        print(json.dumps({"l60": measure_l60(torch, mla, W, args.steps, args.warmup, args.splits)}), flush=True)
        return

    def measure(name, steps, warmup):
        """Build rotating copies of a workload, run warmup + timed steps;
        returns (first workload, algorithmic sizes, copies, ms per step,
        mean attention-kernel us, wall s, percentiles)."""
        cfg = W.CONFIGS[name]
        if cfg.layers > 1:
            cfg = W.scaled(cfg, layers=1)
        t_build = time.perf_counter()
        first = W.Workload(cfg, layer=0, n_splits=args.splits)
        alg = algorithmic(first)
        per_copy = alg["step_bytes"] + first.workspace.numel()
        copies = args.copies or max(2, math.ceil(2 * 256e6 / per_copy))
        wls = [first] + [W.Workload(cfg, layer=i, n_splits=args.splits) for i in range(1, copies)]
        torch.cuda.synchronize()
        print(f"# built {copies} copies of {cfg.name} in {time.perf_counter() - t_build:.1f} s "
              f"({per_copy / 1e6:.0f} MB each)", file=sys.stderr, flush=True)

        def step(i, evs=None):
            # one mla_decode_step call: append of every sequence's newest token,
            # query absorption, plan, split-KV attention, combine + W^UV
            wl = wls[i % copies]
            if evs is None:
                wl.step(impl=args.impl)
            else:
                wl.step(ev_start=evs[0], ev_stop=evs[1], impl=args.impl)

        settled = settle(torch, step, args.settle)
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        # attention-kernel events: HIP events without the system-scope fence,
        # recorded on the decode stream by mla_decode_ex around that kernel
        kev = [(mla.HipEvent(), mla.HipEvent()) for _ in range(steps)]
        # step boundaries, also without the system fence (step i = sev[i] .. sev[i+1])
        sev = [mla.HipEvent() for _ in range(steps + 1)]
        t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        t_start.record()
        for i in range(steps):
            sev[i].record()
            step(i, kev[i])
        sev[steps].record()
        t_stop.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        kern_us = [1e3 * a.elapsed_ms(b) for a, b in kev]
        step_us = [1e3 * sev[i].elapsed_ms(sev[i + 1]) for i in range(steps)]
        dist = {"step_us_p10_p50_p90": [round(float(x), 2) for x in np.percentile(step_us, [10, 50, 90])],
                "kernel_us_p10_p50_p90": [round(float(x), 2) for x in np.percentile(kern_us, [10, 50, 90])]}
        del wls
        dist["settle_steps"] = settled
        return (first, alg, copies, t_start.elapsed_time(t_stop) / steps, sum(kern_us) / len(kern_us), wall,
                dist)

    def counter_traffic(name):
        """HBM bytes per attention launch from the committed rocprofv3 counter
        passes, if they were taken on the current kernel source."""
        if not os.path.exists(COUNTERS) or args.impl != 0:
            return None
        cnt = json.load(open(COUNTERS))
        rec = cnt.get("workloads", {}).get(name)
        if rec and cnt.get("kernel_source_sha256_16") == kernel_source_hash():
            return rec["hbm_bytes_per_launch"]
        return None

    first, alg, copies, ms_per_step, kern_us, wall, dist = measure(args.workload, args.steps, args.warmup)
    copy_gbps = measured_copy_gbps(torch)
    cfg = first.cfg
    B = cfg.B
    value = B / (ms_per_step * 1e-3)
    achieved = alg["attn_bytes"] / (kern_us * 1e-6) / 1e9
    del first
    torch.cuda.empty_cache()
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_s": args.settle, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if cfg.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "context_tokens_per_seq": int(cfg.lens) if not isinstance(
            cfg.lens, (tuple, list)) else list(cfg.lens), "cached_tokens": alg["N"], "n_h": cfg.n_h, "d_h": 128,
                   "d_c": 512, "d_hR": 64, "d_model": cfg.d_model, "page_size": cfg.page_size,
                   "copies_rotated": copies, "n_splits": args.splits or mla.cu_count()},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": counter_traffic(cfg.name),
                     "kernel": "split-KV attention (decode_mfma_kernel)" if args.impl == 0 else "decode_simple_kernel",
                     "alg_bytes_per_launch": alg["attn_bytes"], "kernel_us": round(kern_us, 2),
                     "mfma_tflops": round(alg["attn_flops"] / (kern_us * 1e-6) / 1e12, 1),
                     "mfma_frac": round(alg["attn_flops"] / (kern_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "measured_copy_GBps": round(copy_gbps, 1),
                     "frac_of_measured_copy": round(achieved / copy_gbps, 4)},
        **dist,
        "latent_cache_GBps": round(alg["cache"] / (ms_per_step * 1e-3) / 1e9, 1),
        "step_GBps": round(alg["step_bytes"] / (ms_per_step * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(alg["step_bytes"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "wall_s_timed": round(wall, 4),
    }
    print(f"# headline {cfg.name}: {ms_per_step * 1e3:.1f} us per step, attention {kern_us:.1f} us",
          file=sys.stderr, flush=True)
    # the other decode configurations, timed the same way
    confs = {}
    for name in [n for n in args.configs.split(",") if n and n != args.workload]:
        f2, a2, c2, ms2, k2, _, d2 = measure(name, max(10, args.steps // 2), args.warmup)
        confs[name] = {
            "B": f2.cfg.B, "cached_tokens": a2["N"], "ms_per_step": round(ms2, 5),
            "tokens_per_s": round(f2.cfg.B / (ms2 * 1e-3), 1), "kernel_us": round(k2, 2),
            "hbm_frac": round(a2["attn_bytes"] / (k2 * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "mfma_frac": round(a2["attn_flops"] / (k2 * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "step_hbm_frac": round(a2["step_bytes"] / (ms2 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": counter_traffic(name), "copies_rotated": c2, **d2}
        del f2
        torch.cuda.empty_cache()
        print(f"# {name}: {ms2 * 1e3:.1f} us per step, attention {k2:.1f} us", file=sys.stderr, flush=True)
    if confs:
        res["configs"] = confs
    if not args.no_l60:
        res["l60"] = measure_l60(torch, mla, W, max(5, args.steps // 4), 2, args.splits)
        print(f"# l60: {res['l60']['us_per_step_p10_p50_p90'][1]:.0f} us per 60-layer step", file=sys.stderr,
              flush=True)
    if not args.no_extras:
        # rows past the attention step: the query path and W^O at the headline batch
        res["projections"] = {f"B{B}": measure_projections(torch, mla, B)}
        # the chunked-prefill row: new tokens attending causally over their sequences
        res["prefill"] = [measure_prefill(torch, mla, *c) for c in PREFILL_CONFIGS]
        # the whole attention layer (query path + decode step + W^O) at the headline workload
        res["layer"] = [measure_layer(torch, mla, W, cfg.name)]
        # the sparse top-k decode row at the long-context and headline shapes
        res["sparse"] = [measure_sparse(torch, mla, W, n, k) for n, k in SPARSE_CONFIGS]
        print("# extras done", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(W, cfg.name, args.cpu_seconds, ms_per_step * 1e3)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
