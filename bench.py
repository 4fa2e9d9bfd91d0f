#!/usr/bin/env python3
"""Benchmark of the hybrid GDN + sink/SWA layer on one MI355X.

Headline (the printed JSON line): prefill throughput of one layer with the
LLaMA3.1-8B attention shape (B=1, 32 query / 8 KV heads, d=128, T=4096,
budget 8 sinks + 56 window, bf16 inputs, fp32 state).  One step = one
layer pass over the sequence: one ABI call with both branches, which is one
kernel launch (chunk preparation, chunked GDN state scan and the sink+SWA
softmax tiles cooperating through per-chunk flags); HIP events around it on
its stream time it.  The same layer as two calls (linear, then softmax
adding its branch) is timed too, for reference.  Inputs are resident in HBM
before the timed region.

Secondary figures in "also": decode steps/s (B=256, 1000 consecutive steps),
long-context prefill (B=8, T=32768, budget 128, final state out), the
Qwen3-32B-shaped full stack (short conv + GDN, short conv + GLA, budget 896)
and its serving step (short-conv decode feeding the layer's decode step).

Roofline: algorithmic FLOPs (or bytes) per launch of the dominant kernel
divided by its mean event-timed duration, against the MI355X peaks (bf16
dense MFMA 2.5 PFLOP/s, HBM 8 TB/s); traffic from the committed rocprofv3
counter reading when it was taken on the current kernel sources.
cpu_baseline: the fp64 NumPy oracle timed on this host over the whole layer,
one thread, repeated to at least 10 s.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--only main|decode|...]
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # dense bf16 MFMA FLOP/s
PEAK_HBM = 8.0e12       # bytes/s
CHUNK = 64


def gdn_flops(w, T=None):
    """Algorithmic FLOPs of the chunked GDN linear branch (one layer)."""
    T = w.T if T is None else T
    stream = max(0, T - w.budget)
    d = w.d
    per = 6 * d * d + 2 * CHUNK * (3 * d + 2 * d)
    return w.B * w.H * stream * per


def gla_flops(w, T=None):
    T = w.T if T is None else T
    stream = max(0, T - w.budget)
    d = w.d
    per = 4 * d * d + 2 * CHUNK * (d + d)
    return w.B * w.H * stream * per


def swa_flops(w, T=None):
    T = w.T if T is None else T
    t = np.arange(T)
    return w.B * w.H * int(np.sum(4 * np.minimum(t + 1, w.budget))) * w.d


def prefill_bytes(w, elt=2, state=False):
    d = w.d
    b = w.B * w.T * (w.H * d * elt * 2 + 2 * w.Hkv * d * elt)      # q, o, k, v
    b += w.B * w.T * w.H * 4 * (d if w.update == "gla" else 2)     # gates
    if state:
        b += w.B * w.H * d * d * 4
    return b


def decode_bytes(w, elt=2):
    d, B, H, Hkv, N = w.d, w.B, w.H, w.Hkv, w.budget
    b = 2 * B * H * d * d * 4                 # state read + write
    b += B * Hkv * N * d * elt * 2            # cached K and V read
    b += B * Hkv * d * elt * 2 * 2            # new k, v read + written to the cache
    b += B * H * d * elt * 2                  # q in, o out
    b += B * H * 4 * 2 * 2                    # new a, b in; cached a, b of the evicted slot
    b += B * H * 4 * 2                        # new a, b stored
    b += B * 4 * 2                            # pos
    return b


def timed(fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


# ------------------------------------------------------------- headline

def bench_main(steps, warmup, split=True):
    import swa_chunked_gated_amd as gl
    from workloads import WORKLOADS, make_prefill_inputs

    w = WORKLOADS["llama8b_t4096"]
    inp = make_prefill_inputs(w, device="cuda")
    o = torch.empty(w.B, w.T, w.H, w.d, dtype=torch.bfloat16, device="cuda")
    q, k, v, a, b = (inp[x] for x in ("q", "k", "v", "a", "b"))
    both = gl.BRANCH_LINEAR | gl.BRANCH_SOFTMAX
    ws = torch.empty(gl.prefill_workspace_bytes(w.B, w.T, w.H, w.Hkv, w.d, w.n_sink, w.window,
                                                torch.bfloat16, flags=both),
                     dtype=torch.uint8, device="cuda")
    f_lin, f_swa = gdn_flops(w), swa_flops(w)

    # the layer: one call with both branches (one launch: preparation, state
    # scan and softmax tiles in the same kernel), events around it on its stream
    n = steps + warmup
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]

    def step(i):
        ev[i][0].record()
        gl.hybrid_prefill(q, k, v, a, b, w.n_sink, w.window, flags=both, o=o, workspace=ws)
        ev[i][1].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(warmup, n):
        step(i)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    layer_ms = float(np.mean([ev[i][0].elapsed_time(ev[i][1]) for i in range(warmup, n)]))

    # for reference, each branch alone: the linear call, then the softmax call
    # adding its branch (the two-launch form of the same layer)
    m_split = max(10, steps // 4)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(m_split + 3)]
    for i in range(m_split + 3 if split else 0):
        e = evs[i]
        e[0].record()
        gl.hybrid_prefill(q, k, v, a, b, w.n_sink, w.window, flags=gl.BRANCH_LINEAR, o=o, workspace=ws)
        e[1].record()
        gl.hybrid_prefill(q, k, v, a, b, w.n_sink, w.window, flags=gl.BRANCH_SOFTMAX | gl.ACCUMULATE, o=o)
        e[2].record()
    torch.cuda.synchronize()
    lin_ms = float(np.mean([evs[i][0].elapsed_time(evs[i][1]) for i in range(3, m_split + 3)])) if split else None
    swa_ms = float(np.mean([evs[i][1].elapsed_time(evs[i][2]) for i in range(3, m_split + 3)])) if split else None

    achieved = (f_lin + f_swa) / (layer_ms * 1e-3)
    res = {
        "w": w, "sec": sec,
        "kernels_ms": {LAYER_KERNEL: layer_ms,
                       "two-launch reference": {LINEAR_KERNELS: lin_ms, "swa_kernel": swa_ms}},
        "roofline": {
            "kernel": LAYER_KERNEL, "bound": "mfma", "achieved": achieved / 1e12, "peak": PEAK_BF16 / 1e12,
            "unit": "TFLOP/s", "frac": achieved / PEAK_BF16,
            "traffic": stored_traffic(LAYER_KERNEL, w.name, LAYER_SOURCES),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_flops_per_launch": f_lin + f_swa,
            "algorithmic_bytes_per_launch": prefill_bytes(w),
        },
        "layer_frac_mfma": (f_lin + f_swa) / sec / PEAK_BF16,
        "inputs": inp,
    }
    return res


def cpu_baseline(inp, w, min_seconds=10.0, max_reps=6):
    """fp64 oracle over the whole layer (all heads, whole T), one thread,
    repeated until at least `min_seconds` of CPU work; mean time per layer."""
    from threadpoolctl import threadpool_limits
    from oracle import hybrid as O

    f = {x: inp[x].double().cpu().numpy() for x in ("q", "k", "v", "a", "b")}
    times = []
    with threadpool_limits(1):
        while sum(times) < min_seconds and len(times) < max_reps:
            t0 = time.perf_counter()
            O.hybrid_prefill(f["q"], f["k"], f["v"], f["a"], f["b"], w.n_sink, w.window, flags=3)
            times.append(time.perf_counter() - t0)
    per = sum(times) / len(times)
    return {
        "value": w.B * w.T / per, "unit": "tokens/s", "cores": 1, "kind": "oracle",
        "sample": f"whole layer prefill (B={w.B}, T={w.T}, {w.H} query / {w.Hkv} KV heads, "
                  f"both branches), fp64 NumPy oracle on one thread, {len(times)} repetitions, "
                  f"{sum(times):.1f} s total, {per:.2f} s per layer",
        "cpu": _cpu_model(),
        "host_cores_allowed": len(os.sched_getaffinity(0)),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def kernel_sources_sha256(files):
    """Digest of the sources a kernel is compiled from; a stored counter
    reading only applies while this digest is unchanged."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


LINEAR_SOURCES = ("swa_chunked_gated_amd/csrc/gdn_prep.h", "swa_chunked_gated_amd/csrc/gdn_prep.hip",
                  "swa_chunked_gated_amd/csrc/gdn_scan_full.hip", "swa_chunked_gated_amd/csrc/linear_chunk.hip",
                  "swa_chunked_gated_amd/csrc/common.h")
# the linear launch of the LLaMA-shaped layer (32 chains): preparation and
# state scan in one kernel; with both branches the softmax tiles join it
LINEAR_KERNELS = "gdn_scan_full_kernel"
LAYER_KERNEL = "gdn_scan_full_kernel"
LAYER_SOURCES = ("swa_chunked_gated_amd/csrc/gdn_prep.h", "swa_chunked_gated_amd/csrc/gdn_scan_full.hip",
                 "swa_chunked_gated_amd/csrc/swa_tile.h", "swa_chunked_gated_amd/csrc/common.h")
SWA_SOURCES = ("swa_chunked_gated_amd/csrc/swa.hip", "swa_chunked_gated_amd/csrc/swa_tile.h",
               "swa_chunked_gated_amd/csrc/common.h")
DECODE_SOURCES = ("swa_chunked_gated_amd/csrc/decode.hip", "swa_chunked_gated_amd/csrc/common.h")
# one decode step is two launches: both branches and the state update, then the cache commit
DECODE_KERNELS = "decode_step_kernel+decode_commit_kernel"


def stored_traffic(kernel, workload, sources):
    """HBM bytes per launch from profiles/hbm_traffic.txt: rocprofv3 FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch) times the factors a plain device copy of
    known size gives.  None when no reading exists for the current sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    digest = kernel_sources_sha256(sources)
    fac = {}
    rows = []
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kv = dict(tok.split("=", 1) for tok in line.split() if "=" in tok)
            if kv.get("kind") == "copy":
                fac = {"fetch": float(kv["fetch_factor"]), "write": float(kv["write_factor"])}
            elif kv.get("kind") == "kernel":
                rows.append(kv)
    for kv in rows:
        if kv["kernel"] == kernel and kv["workload"] == workload and kv["sources_sha256"] == digest and fac:
            return (float(kv["fetch_kib"]) * fac["fetch"] + float(kv["write_kib"]) * fac["write"]) * 1024.0
    return None


# ------------------------------------------------------------ secondary

def bench_decode(steps=1000, warmup=10):
    import swa_chunked_gated_amd as gl
    from workloads import WORKLOADS, make_decode_inputs

    w = WORKLOADS["decode_b256"]
    inp = make_decode_inputs(w, device="cuda", steps=steps)
    keys = ("state", "k_cache", "v_cache", "a_cache", "b_cache", "pos")
    o = torch.empty(w.B, w.H, w.d, dtype=torch.bfloat16, device="cuda")

    def run(st, s):
        gl.hybrid_decode(inp["q"][s], inp["k"][s], inp["v"][s], inp["a"][s], inp["b"][s],
                         st["state"], st["k_cache"], st["v_cache"], st["a_cache"], st["b_cache"],
                         st["pos"], w.n_sink, w.window, o=o)

    scratch = {x: inp[x].clone() for x in keys}
    for s in range(warmup):
        run(scratch, s)
    del scratch
    st = {x: inp[x].clone() for x in keys}
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for s in range(steps):
        run(st, s)
    e1.record()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    ev_ms = e0.elapsed_time(e1) / steps
    byts = decode_bytes(w)
    return {
        "workload": "decode_b256 (B=256, H=32, Hkv=8, d=128, cache 8+56, t=4096..5095)",
        "steps": steps, "ms_per_step": sec * 1e3, "steps_per_s": 1.0 / sec,
        "tokens_per_s": w.B / sec, "event_ms_per_step": ev_ms,
        "roofline": {"kernel": DECODE_KERNELS, "bound": "hbm",
                     "achieved": byts / (ev_ms * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": byts / (ev_ms * 1e-3) / PEAK_HBM,
                     "algorithmic_bytes_per_step": byts,
                     "traffic": stored_traffic(DECODE_KERNELS, w.name, DECODE_SOURCES)},
    }


def shortconv_decode_bytes(w, elt=2):
    """One short-conv decode step: raw q, k, v in and prepared out, the conv
    weights, the ks-1 history rows read and one row written (fp32)."""
    C = (w.H + 2 * w.Hkv) * w.d
    ks = w.conv_ks
    return w.B * C * elt * 2 + C * ks * 4 + w.B * C * 4 * ks


def bench_qwen_decode(steps=200, warmup=10):
    """Serving step of the Qwen-shaped stack after its T=8192 prefill: the
    short-conv decode of the new raw q, k, v feeding the layer's decode step
    (budget 896), both on one stream; timed over consecutive steps."""
    import swa_chunked_gated_amd as gl
    from workloads import WORKLOADS, make_decode_inputs

    w = WORKLOADS["qwen32b_decode"]
    inp = make_decode_inputs(w, device="cuda", steps=steps)
    keys = ("state", "k_cache", "v_cache", "a_cache", "b_cache", "pos", "hist_q", "hist_k", "hist_v")
    o = torch.empty(w.B, w.H, w.d, dtype=torch.bfloat16, device="cuda")
    conv = tuple(torch.empty_like(inp[x][0]) for x in ("q", "k", "v"))

    def run(st, s):
        qc, kc, vc = gl.shortconv_decode(inp["q"][s], inp["k"][s], inp["v"][s], inp["wq"], inp["wk"],
                                         inp["wv"], st["hist_q"], st["hist_k"], st["hist_v"], st["pos"],
                                         w.rope_theta, 0, gl.ROPE | gl.L2NORM, out=conv)
        gl.hybrid_decode(qc, kc, vc, inp["a"][s], inp["b"][s], st["state"], st["k_cache"],
                         st["v_cache"], st["a_cache"], st["b_cache"], st["pos"], w.n_sink, w.window,
                         o=o)

    scratch = {x: inp[x].clone() for x in keys}
    for s in range(warmup):
        run(scratch, s)
    del scratch
    st = {x: inp[x].clone() for x in keys}
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for s in range(steps):
        run(st, s)
    e1.record()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    ev_ms = e0.elapsed_time(e1) / steps
    byts = decode_bytes(w) + shortconv_decode_bytes(w)
    return {
        "workload": "qwen32b_decode (B=2, H=64, Hkv=8, d=128, cache 8+888, short conv k=8, t=8192..)",
        "steps": steps, "ms_per_step": sec * 1e3, "steps_per_s": 1.0 / sec,
        "tokens_per_s": w.B / sec, "event_ms_per_step": ev_ms,
        "kernels": "shortconv_decode_kernel + decode_step_wide_kernel + decode_commit_kernel",
        "bound": "launch latency (8.4 MB of state per step)",
        "hbm_frac": byts / (ev_ms * 1e-3) / PEAK_HBM, "algorithmic_bytes_per_step": byts,
    }


def bench_copy(mib=1024, reps=3):
    """A plain device copy of known size: the reference the HBM byte counters
    (FETCH_SIZE, WRITE_SIZE) are scaled by, and the practical read+write roof."""
    n = mib * 2**20 // 4
    x = torch.randn(n, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"workload": f"device copy of {mib} MiB (fp32)", "bytes_read": 4 * n, "bytes_written": 4 * n,
            "us_per_copy": ms * 1e3, "read_plus_write_GBps": 8 * n / (ms * 1e-3) / 1e9}


def bench_prefill_cfg(name, steps=5, warmup=2):
    import swa_chunked_gated_amd as gl
    from workloads import WORKLOADS, make_prefill_inputs

    w = WORKLOADS[name]
    inp = make_prefill_inputs(w, device="cuda")
    flags = gl.BRANCH_LINEAR | gl.BRANCH_SOFTMAX | (gl.WRITE_STATE if w.write_state else 0)
    o = torch.empty(w.B, w.T, w.H, w.d, dtype=torch.bfloat16, device="cuda")
    st = torch.empty(w.B, w.H, w.d, w.d, dtype=torch.float32, device="cuda") if w.write_state else None
    if w.shortconv:
        qc, kc, vc = (torch.empty_like(inp[x]) for x in ("q", "k", "v"))
    nws = gl.prefill_workspace_bytes(w.B, w.T, w.H, w.Hkv, w.d, w.n_sink, w.window,
                                     torch.bfloat16, update=w.update, flags=flags)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None

    def layer():
        if w.shortconv:
            gl.shortconv_qkv(inp["q"], inp["k"], inp["v"], inp["wq"], inp["wk"], inp["wv"],
                             rope_theta=w.rope_theta, flags=gl.ROPE | gl.L2NORM, out=(qc, kc, vc))
            q, k, v = qc, kc, vc
        else:
            q, k, v = inp["q"], inp["k"], inp["v"]
        gl.hybrid_prefill(q, k, v, inp["a"], inp["b"], w.n_sink, w.window, update=w.update,
                          flags=flags, o=o, state_out=st, workspace=ws)

    sec = timed(layer, steps, warmup)
    f = (gdn_flops(w) if w.update == "gdn" else gla_flops(w)) + swa_flops(w)
    res = {"workload": name, "B": w.B, "T": w.T, "H": w.H, "Hkv": w.Hkv, "budget": w.budget,
           "update": w.update, "ms_per_step": sec * 1e3, "tokens_per_s": w.B * w.T / sec,
           "algorithmic_gflop": f / 1e9, "layer_frac_mfma": f / sec / PEAK_BF16}
    if w.shortconv:
        def conv():
            gl.shortconv_qkv(inp["q"], inp["k"], inp["v"], inp["wq"], inp["wk"], inp["wv"],
                             rope_theta=w.rope_theta, flags=gl.ROPE | gl.L2NORM, out=(qc, kc, vc))
        csec = timed(conv, steps, warmup)
        cbytes = 2 * sum(inp[x].numel() * inp[x].element_size() for x in ("q", "k", "v"))
        res["shortconv_ms"] = csec * 1e3
        res["shortconv_frac_hbm"] = cbytes / csec / PEAK_HBM
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", default="all",
                    choices=["all", "main", "decode", "longctx", "qwen32b", "qwen32b_decode", "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-split", action="store_true",
                    help="skip the two-launch reference timing of the headline layer (profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    if args.only == "decode":
        print(json.dumps(bench_decode(steps=args.steps, warmup=args.warmup)), flush=True)
        return
    if args.only == "qwen32b_decode":
        print(json.dumps(bench_qwen_decode(steps=args.steps, warmup=args.warmup)), flush=True)
        return
    if args.only == "copy":
        print(json.dumps(bench_copy()), flush=True)
        return
    if args.only in ("longctx", "qwen32b"):
        names = ["longctx_b8_t32768"] if args.only == "longctx" else \
            ["qwen32b_t8192_gdn", "qwen32b_t8192_gla"]
        for n in names:
            print(json.dumps(bench_prefill_cfg(n, steps=args.steps, warmup=args.warmup)), flush=True)
        return

    m = bench_main(args.steps, args.warmup, split=not args.no_split)
    w = m["w"]
    also = {}
    if args.only == "all":
        also["decode"] = bench_decode()
        also["longctx_b8_t32768"] = bench_prefill_cfg("longctx_b8_t32768")
        also["qwen32b_t8192_gdn"] = bench_prefill_cfg("qwen32b_t8192_gdn")
        also["qwen32b_t8192_gla"] = bench_prefill_cfg("qwen32b_t8192_gla")
        also["qwen32b_decode"] = bench_qwen_decode()
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(m["inputs"], w)
    line = {
        "metric": "hybrid GDN+sink/SWA layer prefill tokens/s (LLaMA3.1-8B attention shape)",
        "value": w.B * w.T / m["sec"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["sec"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the workload, no weights)",
        "config": {"workload": "llama8b_t4096 prefill", "B": w.B, "T": w.T, "H": w.H,
                   "Hkv": w.Hkv, "d": w.d, "n_sink": w.n_sink, "window": w.window,
                   "update": "gdn", "state": "fp32"},
        "roofline": m["roofline"],
        "cpu_baseline": cpu,
        "kernels_ms": m["kernels_ms"],
        "layer_frac_mfma": m["layer_frac_mfma"],
        "also": also,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
