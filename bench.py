#!/usr/bin/env python3
"""Benchmark of the hybrid GDN + sink/SWA layer on one MI355X.

Headline (the printed JSON line): prefill throughput of one layer on the
long-context workload, the largest one that fits one GPU: B=8 sequences of
T=32768 tokens, 32 query / 8 KV heads, d=128, budget 8 sinks + 120 window,
bf16 q/k/v/o, fp32 gates and state, final states written.  One step = one
layer pass over the batch: one ABI call with both branches and the state
output.  K steps are timed between device synchronisations (ms_per_step,
value = B*T / that time); each step is also bracketed by HIP events on its
stream (median reported).  Inputs are resident in HBM before timing.

Roofline: the layer's call is split into its branch calls (the linear branch
with the state, then the softmax branch adding onto it), each timed with
HIP events on the stream the kernels run on; the slowest is the dominant
kernel launch, whose algorithmic FLOPs divided by its median duration is
compared with the bf16 dense MFMA peak (2.5 PFLOP/s).  HBM traffic comes
from the committed rocprofv3 counter readings (profiles/hbm_traffic.txt)
while the kernel sources are the ones measured, else null.

cpu_baseline: the fp64 NumPy oracle, timed on this host before the GPU is
touched, on a bounded sample of the same workload, with its (sequence,
query head) chains spread over a pool of worker processes (one per allowed
core, at most 16).

"also" carries the other workloads, each with its own roofline and oracle
baseline: the tiny fp32 layer, the LLaMA3.1-8B-shaped layer (T=4096), decode
(B=256, 1000 consecutive steps, HBM roofline), the Qwen3-32B-shaped stack
(short conv + GDN, short conv + GLA, budget 896) and its serving step, and
the backward pass (the training path) at the LLaMA-shaped and long-context
shapes.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--only headline|...]
"""

from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # dense bf16 MFMA FLOP/s
PEAK_HBM = 8.0e12       # bytes/s
CHUNK = 64
HEADLINE = "longctx_b8_t32768"
WARM_S = 0.25           # seconds of untimed warm-up steps for the workloads besides the headline


# ------------------------------------------------------- algorithmic work

def gdn_flops(w, T=None):
    """Algorithmic FLOPs of the chunked GDN linear branch (one layer):
    6 dk dv + 2C(3dk + 2dv) per stream token and query head."""
    T = w.T if T is None else T
    stream = max(0, T - w.budget)
    d = w.d
    return w.B * w.H * stream * (6 * d * d + 2 * CHUNK * (3 * d + 2 * d))


def gla_flops(w, T=None):
    """GLA linear branch: 4 dk dv + 2C(dk + dv) per stream token and query head."""
    T = w.T if T is None else T
    stream = max(0, T - w.budget)
    d = w.d
    return w.B * w.H * stream * (4 * d * d + 2 * CHUNK * (d + d))


def linear_flops(w):
    """The delta rule with the diagonal gate does the scalar-gate rule's
    products (its gates scale operands instead of rows)."""
    return gla_flops(w) if w.update == "gla" else gdn_flops(w)


def gdn_prep_flops(w):
    """The part of gdn_flops the chunk preparation runs: the K K^T tiles of
    each chunk, 2 C dk per stream token and query head."""
    stream = max(0, w.T - w.budget)
    return w.B * w.H * stream * 2 * CHUNK * w.d


def swa_flops(w, T=None):
    """Softmax branch: 4 min(t+1, N) d per query row and head."""
    T = w.T if T is None else T
    t = np.arange(T)
    return w.B * w.H * int(np.sum(4 * np.minimum(t + 1, w.budget))) * w.d


def backward_flops(w):
    """The backward pass's algorithmic work (gated delta rule): per chunk
    and query head the gradient products of the chunk form, 6 C d^2 + 9 C^2 d
    + C^3 multiply-adds (dU, dS, dQ, dK^T terms over d^2; the score-shaped
    and UT-transform terms over C^2 d; the C^3 one for dL), twice the
    forward's chunk work; the softmax branch 10 min(t+1, N) d per query row
    and head (scores, dP, dQ, dK, dV: 2.5 times its forward)."""
    stream = max(0, w.T - w.budget)
    nch = -(-stream // CHUNK)
    lin = w.B * w.H * nch * 2 * (6 * CHUNK * w.d ** 2 + 9 * CHUNK ** 2 * w.d + CHUNK ** 3)
    return lin + 2.5 * swa_flops(w)


def prefill_bytes(w):
    """One read of q, k, v, a, b and one write of o (and the state)."""
    elt = 4 if w.dtype == "f32" else 2
    d = w.d
    b = w.B * w.T * (w.H * d * elt * 2 + 2 * w.Hkv * d * elt)      # q, o, k, v
    b += w.B * w.T * w.H * 4 * (d if w.update == "gla" else 2)     # gates
    if w.write_state:
        b += w.B * w.H * d * d * 4
    return b


def tb_bytes(w):
    """The chunk preparation's per-chunk results the layer reads back: TB
    [64][64] in the I/O type and g, gamma [2][64] fp32, per chunk and query
    head."""
    elt = 4 if w.dtype == "f32" else 2
    nch = -(-max(0, w.T - w.budget) // CHUNK)
    return w.B * w.H * nch * (CHUNK * CHUNK * elt + 2 * CHUNK * 4)


def shortconv_bytes(w):
    """Short conv: raw q, k, v read once, prepared q, k, v written once."""
    return 2 * 2 * w.B * w.T * (w.H + 2 * w.Hkv) * w.d


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


def shortconv_decode_bytes(w, elt=2):
    """One short-conv decode step: raw q, k, v in and prepared out, the conv
    weights, the ks-1 history rows read and one row written (fp32)."""
    C = (w.H + 2 * w.Hkv) * w.d
    ks = w.conv_ks
    return w.B * C * elt * 2 + C * ks * 4 + w.B * C * 4 * ks


# ------------------------------------------------------------- kernels

# Kernels each call launches, by workload (the library's launch choice:
# bf16 GDN at d = 128 with both branches, window <= 128 and at most 16
# sinks runs the light preparation, then the one-pass layer: one launch
# when the chains fill the GPU, and with at most 64 chains the segmented
# scan (segment maps, carry, then the layer kernel per segment); "prepare"
# and "layer2" are timed one by one through the two-phase flags.  Other
# bf16 GDN with B*H*d/64 < 256 runs preparation, scan and, with both
# branches, the softmax tiles as one launch; otherwise the light
# preparation, then the many-chain scan, and the softmax kernel).
SEGMENTED = "gdn_segmap_kernel+gdn_carry_kernel+gdn_layer_kernel"
CALL_KERNELS = {
    "longctx_b8_t32768": {"prepare": "gdn_prep_kernel", "layer2": "gdn_layer_kernel"},
    "llama8b_t4096": {"prepare": "gdn_prep_kernel", "layer2": SEGMENTED},
    "tiny_fp32": {"linear": "gdn_prep_kernel+linear_chunk_kernel", "softmax": "swa_kernel"},
    "qwen32b_t8192_gdn": {"shortconv": "shortconv_kernel",
                          "linear": "gdn_prep_kernel+gdn_linear_layer_kernel", "softmax": "swa_long_kernel"},
    "qwen32b_t8192_gla": {"shortconv": "shortconv_kernel",
                          "linear": "gla_prep_kernel+linear_chunk_kernel", "softmax": "swa_long_kernel"},
    "dgd_b8_t8192": {"linear": "gla_prep_kernel+linear_chunk_kernel", "softmax": "swa_ring_kernel"},
}
CSRC = "swa_chunked_gated_amd/csrc/"
KERNEL_SOURCES = {
    "gdn_layer_kernel": ("gdn_layer.hip", "common.h"),
    SEGMENTED: ("gdn_layer.hip", "common.h"),
    "gdn_prep_kernel": ("gdn_prep.h", "gdn_prep.hip", "common.h"),
    "gdn_prep_kernel+linear_chunk_kernel": ("gdn_prep.h", "gdn_prep.hip", "gdn_scan_full.hip",
                                            "linear_chunk.hip", "common.h"),
    "gla_prep_kernel+linear_chunk_kernel": ("gla_prep.hip", "linear_chunk.hip", "common.h"),
    "gdn_prep_kernel+gdn_linear_layer_kernel": ("gdn_prep.h", "gdn_prep.hip", "gdn_layer.hip", "common.h"),
    "gdn_scan_full_kernel": ("gdn_prep.h", "gdn_scan_full.hip", "swa_tile.h", "common.h"),
    "swa_ring_kernel": ("swa.hip", "swa_tile.h", "common.h"),
    "swa_kernel": ("swa.hip", "swa_tile.h", "common.h"),
    "swa_long_kernel": ("swa_long.hip", "swa_tile.h", "common.h"),
    "shortconv_kernel": ("shortconv.hip", "common.h"),
    "decode_step_kernel+decode_commit_kernel": ("decode.hip", "common.h"),
}


def kernel_sources_sha256(kernel):
    """Digest of the sources a kernel is compiled from; a stored counter
    reading only applies while this digest is unchanged."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, CSRC + f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(kernel, workload):
    """HBM bytes per launch from profiles/hbm_traffic.txt: rocprofv3 FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch) times the factors a plain device copy of
    known size gives.  None when no reading exists for the current sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    digest = kernel_sources_sha256(kernel)
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


# ----------------------------------------------------- oracle (CPU) leg

_CPU = {}   # inputs of the oracle sample, inherited by the forked workers


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _oracle_prefill_head(h):
    """Oracle layer (both branches, state) of query head h of the sample."""
    from oracle import hybrid as O
    w, f = _CPU["w"], _CPU["f"]
    G = w.H // w.Hkv
    g = h // G
    if w.shortconv:
        q, k, v = O.shortconv_qkv(f["q"][:, :, h:h + 1], f["k"][:, :, g:g + 1], f["v"][:, :, g:g + 1],
                                  f["wq"].reshape(w.H, w.d, -1)[h], f["wk"].reshape(w.Hkv, w.d, -1)[g],
                                  f["wv"].reshape(w.Hkv, w.d, -1)[g], w.rope_theta, 0, flags=3)
    else:
        q, k, v = f["q"][:, :, h:h + 1], f["k"][:, :, g:g + 1], f["v"][:, :, g:g + 1]
    b = f["b"][:, :, h:h + 1] if w.update != "gla" else None
    O.hybrid_prefill(q, k, v, f["a"][:, :, h:h + 1], b, w.n_sink, w.window, update=w.update)
    return h


def _oracle_backward_head(h):
    """Oracle backward (both branches, final-state gradient) of query head h
    of the sample."""
    from oracle import backward as OB
    w, f = _CPU["w"], _CPU["f"]
    g = h // (w.H // w.Hkv)
    OB.hybrid_prefill_backward(f["q"][:, :, h:h + 1], f["k"][:, :, g:g + 1], f["v"][:, :, g:g + 1],
                               f["a"][:, :, h:h + 1], f["b"][:, :, h:h + 1], w.n_sink, w.window,
                               f["d_o"][:, :, h:h + 1], f["d_state"][:, h:h + 1])
    return h


def _oracle_decode_seqs(sl):
    """Oracle decode steps of the sample's sequences sl[0]:sl[1]."""
    from oracle import hybrid as O
    w, f = _CPU["w"], _CPU["f"]
    s0, s1 = sl
    st = [f[x][s0:s1] for x in ("state", "k_cache", "v_cache", "a_cache", "b_cache", "pos")]
    for s in range(_CPU["steps"]):
        res = O.decode_step(*(f[x][s, s0:s1] for x in ("q", "k", "v", "a", "b")), *st,
                            w.n_sink, w.window, update=w.update)
        st = list(res[1:])
    return s1 - s0


def cpu_baseline(name, cores, T_sample=None, heads=None, steps=None, backward=False):
    """The oracle on a bounded sample of workload `name`: prefill runs
    sequence 0 (first T_sample tokens, the listed query heads), one task per
    head (with backward, the backward pass instead); decode runs `steps`
    steps of every sequence, one task per slice of sequences.  Rate in the
    workload's unit (tokens/s; steps/s)."""
    import torch
    from workloads import WORKLOADS, make_decode_inputs, make_prefill_inputs

    w = WORKLOADS[name]
    _CPU.clear()
    _CPU["w"] = w
    decode = w.T == 0
    if decode:
        inp = make_decode_inputs(w, steps=steps)
        _CPU["steps"] = steps
    else:
        inp = make_prefill_inputs(w, T=T_sample, B=1)
        if backward:
            inp.update(backward_grads(w, T_sample, 1))
    _CPU["f"] = {x: (t.to(torch.float64).numpy() if t.is_floating_point() else t.numpy())
                 for x, t in inp.items()}
    ctx = mp.get_context("fork")
    with ctx.Pool(cores) as pool:
        pool.map(abs, range(cores))          # workers started before timing
        t0 = time.perf_counter()
        if decode:
            per = max(1, w.B // (4 * cores))
            tasks = [(s, min(s + per, w.B)) for s in range(0, w.B, per)]
            pool.map(_oracle_decode_seqs, tasks, chunksize=1)
        else:
            pool.map(_oracle_backward_head if backward else _oracle_prefill_head, list(heads),
                     chunksize=1)
        wall = time.perf_counter() - t0
    _CPU.clear()
    res = {"kind": "oracle", "cores": cores, "cpu": _cpu_model(),
           "host_cores_allowed": len(os.sched_getaffinity(0)), "seconds": wall}
    if decode:
        res.update(value=steps / wall, unit="steps/s",
                   sample=f"{steps} consecutive decode steps of all {w.B} sequences x {w.H} heads "
                          f"(fp64 NumPy oracle, {len(tasks)} tasks of sequences over {cores} worker "
                          f"processes), {wall:.2f} s wall")
    else:
        conv = "short conv + " if w.shortconv else ""
        if backward:
            conv = "the backward pass (gradients of q, k, v, a, b) of "
        res.update(value=T_sample / wall, unit="tokens/s",
                   sample=f"sequence 0, tokens 0..{T_sample - 1}, {len(heads)} of {w.H} query heads"
                          f"{'' if len(heads) == w.H else ' (rate scaled to all heads)'}: {conv}both "
                          f"branches and the final state, fp64 NumPy oracle, one task per head over "
                          f"{cores} worker processes, {wall:.2f} s wall")
        if len(heads) != w.H:
            res["value"] *= len(heads) / w.H
    return res


def backward_grads(w, T=None, B=None, device="cpu"):
    """Seeded upstream gradients of the backward workloads: d_o ~ N(0, 0.5^2)
    in the I/O type and the final state's gradient ~ N(0, 0.05^2) fp32."""
    import torch
    T = w.T if T is None else T
    B = w.B if B is None else B
    g = torch.Generator(device="cpu").manual_seed(1234)
    d_o = (torch.randn(B, T, w.H, w.d, generator=g) * 0.5).to(w.torch_dtype)
    d_state = torch.randn(B, w.H, w.d, w.d, generator=g) * 0.05
    return {"d_o": d_o.to(device), "d_state": d_state.to(device)}


CPU_SAMPLES = {
    # prefill: (tokens of sequence 0, query heads); decode: steps of the whole batch
    "longctx_b8_t32768": dict(T_sample=8192, heads=range(32)),
    "tiny_fp32": dict(T_sample=256, heads=range(2)),
    "llama8b_t4096": dict(T_sample=4096, heads=range(32)),
    "qwen32b_t8192_gdn": dict(T_sample=4096, heads=range(32)),
    "qwen32b_t8192_gla": dict(T_sample=4096, heads=range(32)),
    "dgd_b8_t8192": dict(T_sample=8192, heads=range(32)),
    "decode_b256": dict(steps=20),
}
# backward pass: (tokens of sequence 0, query heads)
CPU_BWD_SAMPLES = {
    "llama8b_t4096": dict(T_sample=4096, heads=range(16)),
    "longctx_b8_t32768": dict(T_sample=4096, heads=range(16)),
}
BWD_KERNELS = ("gdn_prep_kernel+linear_chunk_kernel+gdn_bwd_rev_kernel+gdn_bwd_chunk_kernel+"
               "swa_bwd_dq_kernel+swa_bwd_dkdv_kernel+swa_bwd_sink_kernel")


# ------------------------------------------------------------- GPU legs

def _events(n):
    import torch
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def time_call(fn, reps, warmup):
    """Median and mean event-timed duration (ms) of fn on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    ev = _events(reps)
    for e in ev:
        e[0].record()
        fn()
        e[1].record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    return float(np.median(ms)), float(np.mean(ms))


def bench_prefill(name, steps, warmup, parts=True, warm_s=0.0):
    """One workload's layer: K timed steps (wall clock between
    synchronisations, and per-step events), then each call of the split
    layer event-timed on its own for the roofline.  Warm-up: `warmup` untimed
    steps, then (warm_s > 0) further untimed steps until warm_s seconds have
    passed, so that the GPU's clocks have ramped up before the timed steps of
    a short workload; the entry's "warmup" counts them all."""
    import torch
    import swa_chunked_gated_amd as gl
    from workloads import WORKLOADS, make_prefill_inputs

    w = WORKLOADS[name]
    inp = make_prefill_inputs(w, device="cuda")
    dt = w.torch_dtype
    st_flag = gl.WRITE_STATE if w.write_state else 0
    both = gl.BRANCH_LINEAR | gl.BRANCH_SOFTMAX | st_flag
    o = torch.empty(w.B, w.T, w.H, w.d, dtype=dt, device="cuda")
    st = torch.empty(w.B, w.H, w.d, w.d, dtype=torch.float32, device="cuda") if w.write_state else None
    if w.shortconv:
        qc, kc, vc = (torch.empty_like(inp[x]) for x in ("q", "k", "v"))
    nws = gl.prefill_workspace_bytes(w.B, w.T, w.H, w.Hkv, w.d, w.n_sink, w.window, dt,
                                     update=w.update, flags=both)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")

    def conv():
        gl.shortconv_qkv(inp["q"], inp["k"], inp["v"], inp["wq"], inp["wk"], inp["wv"],
                         rope_theta=w.rope_theta, flags=gl.ROPE | gl.L2NORM, out=(qc, kc, vc))

    def qkv():
        return (qc, kc, vc) if w.shortconv else (inp["q"], inp["k"], inp["v"])

    def layer():
        if w.shortconv:
            conv()
        gl.hybrid_prefill(*qkv(), inp["a"], inp["b"], w.n_sink, w.window, update=w.update,
                          flags=both, o=o, state_out=st, workspace=ws)

    for _ in range(warmup):
        layer()
    n_warm = warmup
    if warm_s > 0:
        torch.cuda.synchronize()
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < warm_s:
            for _ in range(4):
                layer()
            n_warm += 4
            torch.cuda.synchronize()
    ev = _events(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        layer()
        e[1].record()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    ev_ms = [a.elapsed_time(b) for a, b in ev]
    f_lin, f_swa = linear_flops(w), swa_flops(w)
    res = {"workload": name, "B": w.B, "T": w.T, "H": w.H, "Hkv": w.Hkv, "d": w.d,
           "n_sink": w.n_sink, "window": w.window, "update": w.update, "dtype": w.dtype,
           "state_out": w.write_state, "shortconv": w.shortconv,
           "steps": steps, "warmup": n_warm, "ms_per_step": sec * 1e3, "tokens_per_s": w.B * w.T / sec,
           "event_ms_median": float(np.median(ev_ms)), "event_ms_mean": float(np.mean(ev_ms)),
           "algorithmic_gflop": (f_lin + f_swa) / 1e9,
           "layer_frac_mfma": (f_lin + f_swa) / sec / PEAK_BF16}
    if not parts:
        return res

    # the layer's calls one by one, each event-timed (median of >= 20)
    reps = max(20, steps)
    calls = {}
    names = CALL_KERNELS[name]
    if w.shortconv:
        med, mean = time_call(conv, reps, 2)
        calls["shortconv"] = {"kernel": names["shortconv"], "ms_median": med, "ms_mean": mean,
                              "algorithmic_bytes": shortconv_bytes(w)}
    if w.shortconv:
        conv()
    q, k, v = qkv()

    def call(flags):
        return lambda: gl.hybrid_prefill(q, k, v, inp["a"], inp["b"], w.n_sink, w.window,
                                         update=w.update, flags=flags, o=o, state_out=st,
                                         workspace=ws)

    if "layer2" in names:
        # preparation alone, then the one-pass layer kernel alone (its
        # workspace filled by the first)
        med, mean = time_call(call(both | gl.PREPARE_ONLY), reps, 2)
        f_prep = gdn_prep_flops(w)
        calls["prepare"] = {"kernel": names["prepare"], "ms_median": med, "ms_mean": mean,
                            "algorithmic_flops": f_prep}
        med, mean = time_call(call(both | gl.PREPARED), reps, 2)
        calls["layer"] = {"kernel": names["layer2"], "ms_median": med, "ms_mean": mean,
                          "algorithmic_flops": f_lin + f_swa - f_prep}
    else:
        lin_flags = gl.BRANCH_LINEAR | st_flag
        med, mean = time_call(call(lin_flags), reps, 2)
        calls["linear"] = {"kernel": names["linear"], "ms_median": med, "ms_mean": mean,
                           "algorithmic_flops": f_lin}
        med, mean = time_call(call(gl.BRANCH_SOFTMAX | gl.ACCUMULATE), reps, 2)
        calls["softmax"] = {"kernel": names["softmax"], "ms_median": med, "ms_mean": mean,
                            "algorithmic_flops": f_swa}
    res["calls"] = calls

    # dominant kernel launch: the one-pass layer kernel; the whole layer when
    # it is one launch; else the slowest of the split calls' launches
    byts = None
    if "layer2" in names:
        kern, ms, flops = names["layer2"], calls["layer"]["ms_median"], calls["layer"]["algorithmic_flops"]
        byts = prefill_bytes(w) + tb_bytes(w)
    elif "layer" in names:
        kern, ms, flops = names["layer"], res["event_ms_median"], f_lin + f_swa
        byts = prefill_bytes(w)
    else:
        key = max(("linear", "softmax"), key=lambda c: calls[c]["ms_median"])
        kern, ms, flops = calls[key]["kernel"], calls[key]["ms_median"], calls[key]["algorithmic_flops"]
    achieved = flops / (ms * 1e-3)
    res["roofline"] = {
        "kernel": kern, "bound": "mfma", "achieved": achieved / 1e12, "peak": PEAK_BF16 / 1e12,
        "unit": "TFLOP/s", "frac": achieved / PEAK_BF16,
        "traffic": stored_traffic(kern, name),
        "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
        "algorithmic_flops_per_launch": flops, "launch_ms_median": ms,
    }
    if byts is not None:
        res["roofline"]["algorithmic_bytes_per_launch"] = byts
        res["roofline"]["hbm_view"] = {"achieved_GBps": byts / (ms * 1e-3) / 1e9,
                                       "frac": byts / (ms * 1e-3) / PEAK_HBM}
    if w.shortconv:
        c = calls["shortconv"]
        gbs = c["algorithmic_bytes"] / (c["ms_median"] * 1e-3)
        res["shortconv_roofline"] = {"kernel": c["kernel"], "bound": "hbm", "achieved": gbs / 1e9,
                                     "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": gbs / PEAK_HBM,
                                     "traffic": stored_traffic(c["kernel"], name),
                                     "algorithmic_bytes_per_launch": c["algorithmic_bytes"]}
    return res


def bench_backward(name, reps=20, warmup=3):
    """The backward pass at workload `name`'s shape (inputs, upstream
    gradients and the workspace resident), event-timed per call, median of
    `reps`."""
    import torch
    import swa_chunked_gated_amd as gl
    from workloads import WORKLOADS, make_prefill_inputs

    w = WORKLOADS[name]
    inp = make_prefill_inputs(w, device="cuda")
    gr = backward_grads(w, device="cuda")
    nws = gl.prefill_backward_workspace_bytes(w.B, w.T, w.H, w.Hkv, w.d, w.n_sink, w.window)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")

    def call():
        gl.hybrid_prefill_backward(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], w.n_sink,
                                   w.window, gr["d_o"], gr["d_state"], workspace=ws)

    med, mean = time_call(call, max(20, reps), warmup)
    flops = backward_flops(w)
    achieved = flops / (med * 1e-3)
    return {
        "workload": f"{name} backward (B={w.B}, T={w.T}, H={w.H}, Hkv={w.Hkv}, d={w.d}, "
                    f"budget {w.n_sink}+{w.window})",
        "ms_per_step": med, "event_ms_mean": mean, "tokens_per_s": w.B * w.T / (med * 1e-3),
        "algorithmic_gflop": flops / 1e9, "workspace_bytes": nws,
        "roofline": {"kernel": BWD_KERNELS, "bound": "mfma", "achieved": achieved / 1e12,
                     "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16,
                     "traffic": None, "algorithmic_flops_per_launch": flops,
                     "launch_ms_median": med},
    }


def bench_decode(steps=1000, warmup=10):
    import torch
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
    kern = "decode_step_kernel+decode_commit_kernel"
    return {
        "workload": "decode_b256 (B=256, H=32, Hkv=8, d=128, cache 8+56, t=4096..5095)",
        "steps": steps, "ms_per_step": sec * 1e3, "steps_per_s": 1.0 / sec,
        "tokens_per_s": w.B / sec, "event_ms_per_step": ev_ms,
        "roofline": {"kernel": kern, "bound": "hbm",
                     "achieved": byts / (ev_ms * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": byts / (ev_ms * 1e-3) / PEAK_HBM,
                     "algorithmic_bytes_per_step": byts,
                     "traffic": stored_traffic(kern, w.name)},
    }


def bench_qwen_decode(steps=200, warmup=10):
    """Serving step of the Qwen-shaped stack after its T=8192 prefill: the
    short-conv decode of the new raw q, k, v feeding the layer's decode step
    (budget 896), both on one stream; timed over consecutive steps."""
    import torch
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
    import torch
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


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", default="all",
                    choices=["all", "headline", "longctx", "llama", "tiny", "dgd", "decode", "qwen32b",
                             "qwen32b_decode", "copy", "backward"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bwd-workload", choices=["llama8b_t4096", "longctx_b8_t32768"], default=None,
                    help="with --only backward: one workload (default: both)")
    ap.add_argument("--no-parts", action="store_true",
                    help="time the layer only, not its calls one by one (profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    parts = not args.no_parts

    # single-workload legs (profiling and counter runs)
    single = {"longctx": HEADLINE, "llama": "llama8b_t4096", "tiny": "tiny_fp32", "dgd": "dgd_b8_t8192"}
    if args.only in single or args.only in ("decode", "qwen32b", "qwen32b_decode", "copy", "backward"):
        import torch
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(2)
        torch.cuda.set_device(0)
        if args.only in single:
            out = bench_prefill(single[args.only], args.steps, args.warmup, parts=parts, warm_s=WARM_S)
        elif args.only == "decode":
            out = bench_decode(steps=args.steps, warmup=args.warmup)
        elif args.only == "qwen32b_decode":
            out = bench_qwen_decode(steps=args.steps, warmup=args.warmup)
        elif args.only == "copy":
            out = bench_copy()
        elif args.only == "backward":
            for n in ([args.bwd_workload] if args.bwd_workload else list(CPU_BWD_SAMPLES)):
                print(json.dumps(bench_backward(n, args.steps, args.warmup)), flush=True)
            return
        else:
            for n in ("qwen32b_t8192_gdn", "qwen32b_t8192_gla"):
                print(json.dumps(bench_prefill(n, args.steps, args.warmup, parts=parts, warm_s=WARM_S)),
                      flush=True)
            return
        print(json.dumps(out), flush=True)
        return

    # the oracle first, before anything touches the GPU (its workers fork)
    cpu = {}
    if not args.no_cpu_baseline:
        todo = [HEADLINE] + ([] if args.only == "headline" else
                             ["tiny_fp32", "llama8b_t4096", "decode_b256", "qwen32b_t8192_gdn",
                              "qwen32b_t8192_gla", "dgd_b8_t8192"])
        for n in todo:
            cpu[n] = cpu_baseline(n, cores, **CPU_SAMPLES[n])
            print(f"# cpu_baseline {n}: {cpu[n]['value']:.1f} {cpu[n]['unit']} "
                  f"({cpu[n]['seconds']:.1f} s)", file=sys.stderr, flush=True)
        if args.only == "all":
            for n in CPU_BWD_SAMPLES:
                cpu[n + "_backward"] = cpu_baseline(n, cores, backward=True, **CPU_BWD_SAMPLES[n])
                print(f"# cpu_baseline {n} backward: {cpu[n + '_backward']['value']:.1f} tokens/s "
                      f"({cpu[n + '_backward']['seconds']:.1f} s)", file=sys.stderr, flush=True)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    m = bench_prefill(HEADLINE, args.steps, args.warmup, parts=True)
    print(f"# headline done: {m['ms_per_step']:.3f} ms per step", file=sys.stderr, flush=True)
    also = {}
    if args.only == "all":
        for n in ("tiny_fp32", "llama8b_t4096", "qwen32b_t8192_gdn", "qwen32b_t8192_gla", "dgd_b8_t8192"):
            also[n] = bench_prefill(n, args.steps, args.warmup, parts=True, warm_s=WARM_S)
            also[n]["cpu_baseline"] = cpu.get(n)
            print(f"# {n} done", file=sys.stderr, flush=True)
        for n in CPU_BWD_SAMPLES:
            also[n + "_backward"] = bench_backward(n)
            also[n + "_backward"]["cpu_baseline"] = cpu.get(n + "_backward")
            print(f"# {n} backward done", file=sys.stderr, flush=True)
        also["decode_b256"] = bench_decode()
        also["decode_b256"]["cpu_baseline"] = cpu.get("decode_b256")
        also["qwen32b_decode"] = bench_qwen_decode()
        also["copy"] = bench_copy()
    roof = dict(m.pop("roofline"))
    line = {
        "metric": "hybrid GDN+sink/SWA layer prefill tokens/s (long-context: B=8, T=32768, "
                  "32 query / 8 KV heads, d=128, budget 8+120, final state out)",
        "value": m["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the workload, no weights)",
        "config": {"workload": "longctx_b8_t32768 prefill", "B": m["B"], "T": m["T"], "H": m["H"],
                   "Hkv": m["Hkv"], "d": m["d"], "n_sink": m["n_sink"], "window": m["window"],
                   "update": "gdn", "state": "fp32, written"},
        "roofline": roof,
        "cpu_baseline": cpu.get(HEADLINE),
        "layer": m,
        "also": also,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
