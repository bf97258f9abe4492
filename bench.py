#!/usr/bin/env python3
"""Benchmark of the MLA decode hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input: the
append of each sequence's newest token (W^DKV down-projection + RoPE'd k^R
into the paged latent cache) followed by mla_decode (plan, absorb, split-KV
attention over the latent cache, combine, W^UV epilogue).  Inputs are
resident in HBM before timing starts.  To keep the 256 MB Infinity Cache from
serving repeated reads, steps rotate over several independent copies of the
workload (own weights, queries and cache) whose total size exceeds it.

Prints one JSON line.  `value` is decode tokens/s (B sequences per step);
`roofline` is computed for the split-KV attention kernel from its algorithmic
bytes and its HIP-event duration measured in the timed region; `projections`
times the query path (W^DQ, W^UQ, W^QR) and the output projection W^O, which
sit outside the step, at the same batch sizes; `prefill` times chunked
prefill (new tokens attending causally over their sequences); `layer` times
the whole attention layer (query path + step + W^O, h -> u); `cpu_baseline`
times the fp64 CPU oracle on a bounded sample of the same workload.
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


def cpu_baseline(wl, seconds: float):
    """The fp64 oracle (absorbed form) doing the same per-sequence work as a
    step -- append the newest token, then decode -- on a bounded sample."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    sample = [0, 1]
    prepared = []
    for b in sample:
        d = wl.oracle_inputs(b)
        n = d["n"]
        if "h" in d:
            c, kR = oracle.down_project(d["h"][:n - 1], d["W_DKV"], d["W_KR"], np.arange(n - 1), wl.dims.rope_base)
            h_new = d["h"][n - 1:]
        else:
            c, kR, h_new = d["prior_c"], d["prior_kR"], d["h_new"]
        prepared.append((d, c, kR, h_new))
    done, t0 = 0, time.perf_counter()
    while True:
        for d, c, kR, h_new in prepared:
            n = d["n"]
            c1, k1 = oracle.down_project(h_new, d["W_DKV"], d["W_KR"], np.array([n - 1]), wl.dims.rope_base)
            oracle.attend_absorbed(d["q_C"], d["q_R"], n - 1, np.concatenate([c, c1]), np.concatenate([kR, k1]),
                                   d["W_UK"], d["W_UV"], wl.dims.rope_base, wl.dims.scale)
            done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    n0 = int(wl.n[0])
    return {"value": done / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 absorbed-form oracle, append + decode of sequences {sample} ({n0} cached tokens, "
                      f"n_h={wl.cfg.n_h}) repeated {done} times in {el:.1f} s; 1 decode token per sequence"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="b32_l4096")
    ap.add_argument("--target-workload", default="b64_l8192",
                    help="second workload reported under target_shape ('' to skip)")
    ap.add_argument("--copies", type=int, default=0, help="workload copies to rotate over (0 = enough to exceed "
                                                         "the 256 MB Infinity Cache twice)")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--impl", type=int, default=0, help="0 = MFMA attention kernel, 1 = VALU reference kernel")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-projections", action="store_true", help="skip the query / output projection timings")
    ap.add_argument("--prefill-only", action="store_true", help="only time the chunked prefill configurations")
    ap.add_argument("--layer-only", default="", help="comma-separated workloads: only time the whole decode layer")
    ap.add_argument("--projections-only", default="",
                    help="comma-separated batch sizes: only time the query / output projections at them")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (reference for the HBM "
                         "byte counters of rocprofv3)")
    args = ap.parse_args()
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

    def measure(name, steps, warmup):
        """Build rotating copies of a workload, run warmup + timed steps;
        returns (first workload, copies, ms per step, attention-kernel us, wall s)."""
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
        return (first, alg, copies, t_start.elapsed_time(t_stop) / steps, sum(kern_us) / len(kern_us), wall,
                dist)

    first, alg, copies, ms_per_step, kern_us, wall, dist = measure(args.workload, args.steps, args.warmup)
    copy_gbps = measured_copy_gbps(torch)
    cfg = first.cfg
    B = cfg.B
    value = B / (ms_per_step * 1e-3)
    achieved = alg["attn_bytes"] / (kern_us * 1e-6) / 1e9
    traffic = None
    if os.path.exists(COUNTERS):
        cnt = json.load(open(COUNTERS))
        rec = cnt.get("workloads", {}).get(cfg.name)
        if rec and cnt.get("kernel_source_sha256_16") == kernel_source_hash() and args.impl == 0:
            traffic = rec["hbm_bytes_per_launch"]
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if cfg.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "context_tokens_per_seq": int(cfg.lens) if not isinstance(
            cfg.lens, (tuple, list)) else list(cfg.lens), "cached_tokens": alg["N"], "n_h": cfg.n_h, "d_h": 128,
                   "d_c": 512, "d_hR": 64, "d_model": cfg.d_model, "page_size": cfg.page_size,
                   "copies_rotated": copies, "n_splits": args.splits or first.mla.cu_count()},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "split-KV attention (decode_mfma_kernel)" if args.impl == 0 else "decode_simple_kernel",
                     "kernel_us": round(kern_us, 2),
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
    if args.target_workload and args.target_workload != args.workload:
        # the batch-64 / 8K-context decode shape the performance target is stated on
        f2, a2, c2, ms2, k2, _, d2 = measure(args.target_workload, max(5, args.steps // 2), args.warmup)
        res["target_shape"] = {
            "workload": f2.cfg.name, "B": f2.cfg.B, "cached_tokens": a2["N"], "ms_per_step": round(ms2, 5),
            "tokens_per_s": round(f2.cfg.B / (ms2 * 1e-3), 1), "kernel_us": round(k2, 2),
            "hbm_frac": round(a2["attn_bytes"] / (k2 * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "mfma_frac": round(a2["attn_flops"] / (k2 * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "hbm_frac_of_measured_copy": round(a2["attn_bytes"] / (k2 * 1e-6) / 1e9 / copy_gbps, 4),
            "copies_rotated": c2, **d2}
    if not args.no_projections:
        # rows past the attention step: the query path and W^O, at the batches reported above
        res["projections"] = {f"B{b}": measure_projections(torch, mla, b) for b in
                              sorted({B, res.get("target_shape", {}).get("B", B)})}
    if not args.no_projections:
        # the chunked-prefill row: new tokens attending causally over their sequences
        res["prefill"] = [measure_prefill(torch, mla, *cfg) for cfg in PREFILL_CONFIGS]
        # the whole attention layer (query path + decode step + W^O) at the step's workloads
        res["layer"] = [measure_layer(torch, mla, W, n) for n in
                        dict.fromkeys([cfg.name, res.get("target_shape", {}).get("workload", cfg.name)])]
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(first, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
