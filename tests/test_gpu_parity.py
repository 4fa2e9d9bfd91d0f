"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Tolerances: fp32 inputs, max-abs error <= 1e-4; bf16 inputs with fp32
state, max-abs error <= 2e-2 * max|o_ref| over the compared outputs.  Index
masks are checked exactly (mask probe).  Full-size workloads are compared on
sampled (sequence, head) chains and rows that the oracle computes one by one.
"""

import math

import numpy as np
import pytest
import torch

import swa_chunked_gated_amd as gl
from oracle import hybrid as O
from workloads import WORKLOADS, Workload, make_decode_inputs, make_prefill_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"

ALL = gl.BRANCH_LINEAR | gl.BRANCH_SOFTMAX


def f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def assert_close(got, ref, fp32: bool, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.max(np.abs(got - ref)) if got.size else 0.0
    if fp32:
        bound = 1e-4
    else:
        bound = 2e-2 * max(np.max(np.abs(ref)), 1e-30)
    assert err <= bound, f"{what}: max abs err {err:.3e} > {bound:.3e}"
    return err


def to_dev(inp):
    return {k: v.to(DEV) for k, v in inp.items()}


def small(name="s", **kw):
    base = dict(name=name, B=2, H=4, Hkv=2, d=128, n_sink=8, window=56, T=257, sigma=0.5,
                dtype="bf16")
    base.update(kw)
    return Workload(**base)


def run_prefill(inp, w: Workload, flags=ALL | gl.WRITE_STATE):
    o, st = gl.hybrid_prefill(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], w.n_sink,
                              w.window, update=w.update, flags=flags)
    torch.cuda.synchronize()
    return o, st


def oracle_subset(inp, w: Workload, bsel, heads, rows=None, flags=ALL | gl.WRITE_STATE):
    """Oracle on sequences `bsel` and query heads `heads` (all in one KV group)."""
    G = w.H // w.Hkv
    g = heads[0] // G
    assert all(h // G == g for h in heads)
    q = f64(inp["q"][bsel][:, :, heads])
    k = f64(inp["k"][bsel][:, :, g:g + 1])
    v = f64(inp["v"][bsel][:, :, g:g + 1])
    a = f64(inp["a"][bsel][:, :, heads])
    b = f64(inp["b"][bsel][:, :, heads])
    o = np.zeros(q.shape)
    S = None
    if flags & (gl.BRANCH_LINEAR | gl.WRITE_STATE):
        if w.update == "gdn":
            o_lin, S = O.gdn_linear_branch(q, k, v, a, b, w.n_sink, w.window)
        else:
            o_lin, S = O.gla_linear_branch(q, k, v, a, w.n_sink, w.window)
        if flags & gl.BRANCH_LINEAR:
            o = o + o_lin
    if flags & gl.BRANCH_SOFTMAX:
        o = o + O.swa_branch(q, k, v, w.n_sink, w.window, rows=rows)
    return o, S


# ------------------------------------------------------------------ prefill

def test_tiny_fp32_layer_full():
    w = WORKLOADS["tiny_fp32"]
    inp = to_dev(make_prefill_inputs(w))
    o, st = run_prefill(inp, w)
    ref, S = O.hybrid_prefill(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["a"]),
                              f64(inp["b"]), w.n_sink, w.window)
    assert_close(f64(o), ref, True, "o")
    assert_close(f64(st), S, True, "state")


@pytest.mark.parametrize("T", [1, 7, 63, 64, 65, 100, 127, 128, 129, 257, 700])
def test_bf16_ragged_lengths(T):
    w = small(T=T)
    inp = to_dev(make_prefill_inputs(w, seed=T))
    o, st = run_prefill(inp, w)
    ref, S = O.hybrid_prefill(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["a"]),
                              f64(inp["b"]), w.n_sink, w.window)
    assert_close(f64(o), ref, False, "o")
    assert_close(f64(st), S, False, "state")


@pytest.mark.parametrize("T,n_sink,window", [(65, 8, 56), (257, 8, 56), (300, 3, 20), (200, 0, 64),
                                             (130, 8, 120)])
def test_fp32_d64_shapes(T, n_sink, window):
    w = small(T=T, d=64, dtype="f32", n_sink=n_sink, window=window, H=4, Hkv=1)
    inp = to_dev(make_prefill_inputs(w, seed=11))
    o, st = run_prefill(inp, w)
    ref, S = O.hybrid_prefill(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["a"]),
                              f64(inp["b"]), w.n_sink, w.window)
    assert_close(f64(o), ref, True, "o")
    assert_close(f64(st), S, True, "state")


@pytest.mark.parametrize("H,Hkv", [(4, 4), (8, 1), (16, 2)])
def test_head_groupings(H, Hkv):
    w = small(T=200, H=H, Hkv=Hkv, B=1)
    inp = to_dev(make_prefill_inputs(w, seed=5))
    o, st = run_prefill(inp, w)
    ref, S = O.hybrid_prefill(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["a"]),
                              f64(inp["b"]), w.n_sink, w.window)
    assert_close(f64(o), ref, False, "o")
    assert_close(f64(st), S, False, "state")


@pytest.mark.parametrize("flags", [gl.BRANCH_LINEAR, gl.BRANCH_SOFTMAX, gl.WRITE_STATE,
                                   gl.BRANCH_LINEAR | gl.WRITE_STATE])
def test_branch_flags(flags):
    w = small(T=300)
    inp = to_dev(make_prefill_inputs(w, seed=2))
    o, st = run_prefill(inp, w, flags=flags)
    ref, S = O.hybrid_prefill(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["a"]),
                              f64(inp["b"]), w.n_sink, w.window, flags=flags)
    if flags & ALL:
        assert_close(f64(o), ref, False, "o")
    else:
        assert o is None
    if flags & gl.WRITE_STATE:
        assert_close(f64(st), S, False, "state")


@pytest.mark.parametrize("n_sink,window,T", [(8, 56, 300), (8, 120, 400), (3, 20, 150), (0, 64, 200)])
def test_mask_probe_exact(n_sink, window, T):
    """Softmax-only with q = 0: weights are exactly uniform over A(t), and a
    one-hot v (dimension i mod d) turns every output row into exact counts of
    the attended positions per residue class."""
    d = 128
    B, H = 1, 1
    q = torch.zeros(B, T, H, d, dtype=torch.bfloat16, device=DEV)
    k = torch.randn(B, T, H, d, device=DEV).to(torch.bfloat16)
    v = torch.nn.functional.one_hot(torch.arange(T, device=DEV) % d, d).to(torch.bfloat16)
    v = v.view(1, T, 1, d).contiguous()
    a = torch.ones(B, T, H, device=DEV)
    b = torch.ones(B, T, H, device=DEV)
    o, _ = gl.hybrid_prefill(q, k, v, a, b, n_sink, window, flags=gl.BRANCH_SOFTMAX)
    torch.cuda.synchronize()
    o = f64(o)[0, :, 0]
    for t in range(T):
        A = O.softmax_index_set(t, n_sink, window)
        want = np.bincount(A % d, minlength=d)
        got = np.rint(o[t] * len(A)).astype(np.int64)
        assert np.array_equal(got, want), f"row {t}"


def test_llama8b_t4096_sampled_heads():
    w = WORKLOADS["llama8b_t4096"]
    inp = to_dev(make_prefill_inputs(w, device=DEV))
    o, st = run_prefill(inp, w)
    for heads in ([0, 1, 2, 3], [29, 31]):
        ref, S = oracle_subset(inp, w, [0], heads)
        assert_close(f64(o[:, :, heads]), ref, False, f"o heads {heads}")
        assert_close(f64(st[:, heads]), S, False, f"state heads {heads}")


def test_longctx_b8_t32768_sampled():
    w = WORKLOADS["longctx_b8_t32768"]
    inp = to_dev(make_prefill_inputs(w, device=DEV))
    o, st = run_prefill(inp, w)
    rng = np.random.default_rng(0)
    rows = sorted(set([0, 7, 8, 127, 128, 129, 255, 256, w.T - 1]) |
                  set(rng.integers(0, w.T, 40).tolist()))
    for bsel, heads in (([0], [0]), ([7], [31]), ([3], [13, 14])):
        ref, S = oracle_subset(inp, w, bsel, heads, rows=rows)
        got = f64(o[bsel][:, rows][:, :, heads])
        assert_close(got, ref[:, rows], False, f"o b{bsel} h{heads}")
        assert_close(f64(st[bsel][:, heads]), S, False, f"state b{bsel} h{heads}")


# ---------------------------------------------------------------- GLA

@pytest.mark.parametrize("T,dtype,d", [(257, "bf16", 128), (130, "bf16", 128), (700, "bf16", 64),
                                       (257, "f32", 64), (65, "f32", 64)])
def test_gla_prefill(T, dtype, d):
    w = small(T=T, d=d, dtype=dtype, update="gla")
    inp = to_dev(make_prefill_inputs(w, seed=3))
    o, st = run_prefill(inp, w)
    ref, S = O.hybrid_prefill(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["a"]),
                              None, w.n_sink, w.window, update="gla")
    assert_close(f64(o), ref, dtype == "f32", "o")
    assert_close(f64(st), S, dtype == "f32", "state")


@pytest.mark.parametrize("update,dtype,d,gate_mean", [("gla", "bf16", 128, 1.0), ("gla", "bf16", 128, 3.0),
                                                    ("gla", "f32", 64, 1.0), ("gdn", "bf16", 128, 1.0),
                                                    ("gdn", "f32", 64, 3.0)])
def test_strong_forget_gates(update, dtype, d, gate_mean):
    """Gates far below 1 (mean about 0.27 or 0.05 per token): a 64-token
    chunk then decays by e^-80 to e^-190, beyond the float range if the
    decay between two tokens were split into one factor per token."""
    w = small(T=300, d=d, dtype=dtype, update=update, gate_mean=gate_mean)
    inp = to_dev(make_prefill_inputs(w, seed=11))
    o, st = run_prefill(inp, w)
    ref, S = O.hybrid_prefill(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["a"]),
                              f64(inp["b"]) if update == "gdn" else None, w.n_sink, w.window,
                              update=update)
    assert_close(f64(o), ref, dtype == "f32", "o")
    assert_close(f64(st), S, dtype == "f32", "state")


# ------------------------------------------------------------- short conv

@pytest.mark.parametrize("dtype,d,T,flags,ks,H,Hkv", [
    ("bf16", 128, 200, 3, 8, 4, 2), ("f32", 64, 77, 3, 8, 4, 2), ("f32", 128, 70, 1, 8, 4, 2),
    ("bf16", 64, 130, 2, 8, 4, 2), ("f32", 64, 9, 0, 8, 4, 2), ("bf16", 128, 100, 3, 3, 4, 2),
    ("f32", 64, 64, 3, 1, 4, 2), ("bf16", 128, 16, 3, 8, 4, 2), ("f32", 128, 129, 3, 5, 4, 2),
    ("bf16", 128, 700, 3, 8, 3, 1), ("bf16", 64, 1000, 3, 8, 6, 3), ("f32", 128, 523, 3, 6, 3, 3)])
def test_shortconv_small(dtype, d, T, flags, ks, H, Hkv):
    """Tiles of 64 tokens with a causal halo (four consecutive tiles per
    workgroup), 8-token blocks, ragged ends, and head counts that leave part
    of a wave's head group empty."""
    w = small(T=T, d=d, dtype=dtype, shortconv=True, H=H, Hkv=Hkv, B=2, conv_ks=ks)
    inp = to_dev(make_prefill_inputs(w, seed=4))
    qo, ko, vo = gl.shortconv_qkv(inp["q"], inp["k"], inp["v"], inp["wq"], inp["wk"], inp["wv"],
                                  rope_theta=1e6, pos0=3, flags=flags)
    torch.cuda.synchronize()
    rq, rk, rv = O.shortconv_qkv(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["wq"]),
                                 f64(inp["wk"]), f64(inp["wv"]), 1e6, 3, flags=flags)
    fp32 = dtype == "f32"
    assert_close(f64(qo), rq, fp32, "q")
    assert_close(f64(ko), rk, fp32, "k")
    assert_close(f64(vo), rv, fp32, "v")


def test_qwen32b_full_stack_sampled():
    """Config with RoPE -> conv -> L2 norm, budget 896, GDN and GLA layers."""
    for name in ("qwen32b_t8192_gdn", "qwen32b_t8192_gla"):
        w = WORKLOADS[name]
        raw = to_dev(make_prefill_inputs(w, device=DEV))
        qc, kc, vc = gl.shortconv_qkv(raw["q"], raw["k"], raw["v"], raw["wq"], raw["wk"], raw["wv"],
                                      rope_theta=w.rope_theta, pos0=0, flags=gl.ROPE | gl.L2NORM)
        inp = dict(q=qc, k=kc, v=vc, a=raw["a"], b=raw["b"])
        o, st = run_prefill(inp, w)
        G = w.H // w.Hkv
        rows = [0, 7, 8, 895, 896, 897, 1000, 4095, 4096, w.T - 1]
        for bsel, heads, g in (([0], [0, 5], 0), ([1], [63], 7)):
            # short conv of the sampled channels
            cq = slice(heads[0], heads[-1] + 1)
            rq, rk, rv = O.shortconv_qkv(
                f64(raw["q"][bsel][:, :, cq]), f64(raw["k"][bsel][:, :, g:g + 1]),
                f64(raw["v"][bsel][:, :, g:g + 1]),
                f64(raw["wq"].view(w.H, w.d, -1)[cq].reshape(-1, w.conv_ks)),
                f64(raw["wk"].view(w.Hkv, w.d, -1)[g]), f64(raw["wv"].view(w.Hkv, w.d, -1)[g]),
                w.rope_theta, 0, flags=3)
            assert_close(f64(qc[bsel][:, :, cq]), rq, False, "conv q")
            assert_close(f64(kc[bsel][:, :, g:g + 1]), rk, False, "conv k")
            assert_close(f64(vc[bsel][:, :, g:g + 1]), rv, False, "conv v")
            # the layer on the GPU's conv outputs
            ref, S = oracle_subset(inp, w, bsel, heads, rows=rows)
            assert_close(f64(o[bsel][:, rows][:, :, heads]), ref[:, rows], False, f"{name} o")
            assert_close(f64(st[bsel][:, heads]), S, False, f"{name} state")
            assert heads[0] // G == g


# ---------------------------------------------------------- edge shapes

def test_many_chain_full_wave_scan():
    """B*H >= 256: one 8-wave scan workgroup per chain (light preparation),
    then the softmax launch; sampled chains against the oracle."""
    w = small(B=8, H=32, Hkv=8, d=128, T=300, sigma=1.0)
    inp = to_dev(make_prefill_inputs(w, seed=21))
    o, st = run_prefill(inp, w)
    for bsel, heads in (([0], [0, 1]), ([5], [17]), ([7], [31])):
        ref, S = oracle_subset(inp, w, bsel, heads)
        assert_close(f64(o[bsel][:, :, heads]), ref, False, "o")
        assert_close(f64(st[bsel][:, heads]), S, False, "state")


@pytest.mark.parametrize("B,H,Hkv,T,n_sink,window", [(8, 32, 8, 300, 8, 56), (16, 16, 4, 517, 8, 120),
                                                     (32, 8, 2, 400, 16, 128), (32, 8, 8, 250, 0, 1),
                                                     (64, 4, 1, 129, 3, 64), (16, 8, 2, 700, 0, 100),
                                                     (16, 16, 2, 200, 8, 120), (16, 8, 4, 193, 8, 120),
                                                     (16, 16, 4, 333, 5, 40), (32, 8, 2, 211, 16, 65)])
def test_one_pass_layer(B, H, Hkv, T, n_sink, window):
    """Both branches on many chains: the one-pass kernel (state scan and the
    softmax rows of each chunk in one workgroup per chain, o written once);
    ragged lengths, one-chunk streams, windows 1..128, 0..16 sinks; sampled
    chains against the oracle, output rows and final state."""
    w = small(B=B, H=H, Hkv=Hkv, d=128, T=T, n_sink=n_sink, window=window, sigma=1.0)
    inp = to_dev(make_prefill_inputs(w, seed=T * 7 + window))
    o, st = run_prefill(inp, w)
    G = H // Hkv
    for bsel, heads in (([0], [0]), ([B // 2], list(range(G * (Hkv - 1), G * Hkv))), ([B - 1], [H - 1])):
        ref, S = oracle_subset(inp, w, bsel, heads)
        assert_close(f64(o[bsel][:, :, heads]), ref, False, f"o b{bsel} h{heads}")
        assert_close(f64(st[bsel][:, heads]), S, False, f"state b{bsel} h{heads}")


@pytest.mark.parametrize("n_sink,window,flags,T", [(8, 120, ALL | gl.WRITE_STATE, 520), (0, 129, ALL, 520),
                                                    (64, 64, ALL, 520), (3, 20, gl.BRANCH_SOFTMAX, 520),
                                                    (0, 1, ALL, 257), (64, 65, ALL | gl.WRITE_STATE, 300)])
def test_resident_key_blocks(n_sink, window, flags, T):
    """Many sequences and groups of four query heads per KV head: the softmax
    launch keeps its key blocks resident across a workgroup's consecutive
    64-row tiles (nine, or five, per workgroup, the last one ragged); sampled
    (sequence, head) chains against the oracle."""
    w = small(B=256, H=16, Hkv=4, d=128, T=T, n_sink=n_sink, window=window, sigma=1.0)
    inp = to_dev(make_prefill_inputs(w, seed=window))
    o, st = run_prefill(inp, w, flags=flags)
    for bsel, heads in (([0], [0, 3]), ([77], [5, 6]), ([255], [12, 15])):
        ref, S = oracle_subset(inp, w, bsel, heads, flags=flags)
        assert_close(f64(o[bsel][:, :, heads]), ref, False, f"o b{bsel} h{heads}")
        if flags & gl.WRITE_STATE:
            assert_close(f64(st[bsel][:, heads]), S, False, f"state b{bsel} h{heads}")


@pytest.mark.parametrize("B,H,Hkv,T,n_sink,window,flags", [
    (4, 32, 8, 700, 8, 130, ALL | gl.WRITE_STATE), (2, 64, 8, 1100, 8, 888, ALL | gl.WRITE_STATE),
    (4, 32, 4, 333, 20, 56, ALL), (8, 16, 4, 515, 3, 300, ALL | gl.WRITE_STATE),
    (4, 32, 8, 700, 8, 130, gl.BRANCH_LINEAR | gl.WRITE_STATE), (4, 32, 8, 300, 8, 56, gl.BRANCH_LINEAR)])
def test_many_chain_linear_layer_kernel(B, H, Hkv, T, n_sink, window, flags):
    """Many chains (B*H*d/64 >= 256) with a window past the one-pass layer's
    ring (or more sinks than it holds), or the linear branch alone: the layer
    kernel runs the linear branch alone (its softmax waves form only the
    decayed score tile; rows t < n_sink + window are zeroed when no softmax
    launch follows), then the softmax launch adds its rows; sampled chains
    against the oracle, every row and the final state, ragged last chunks."""
    w = small(B=B, H=H, Hkv=Hkv, d=128, T=T, n_sink=n_sink, window=window, sigma=1.0)
    inp = to_dev(make_prefill_inputs(w, seed=T + window))
    o, st = run_prefill(inp, w, flags=flags)
    G = H // Hkv
    for bsel, heads in (([0], [0, 1]), ([B - 1], list(range(H - G, H)))):
        ref, S = oracle_subset(inp, w, bsel, heads, flags=flags)
        assert_close(f64(o[bsel][:, :, heads]), ref, False, f"o b{bsel} h{heads}")
        if flags & gl.WRITE_STATE:
            assert_close(f64(st[bsel][:, heads]), S, False, f"state b{bsel} h{heads}")


@pytest.mark.parametrize("H,Hkv,T,n_sink,window,flags", [
    (16, 2, 1300, 8, 888, ALL | gl.WRITE_STATE), (8, 2, 1000, 8, 888, gl.BRANCH_SOFTMAX),
    (4, 2, 777, 70, 300, ALL), (16, 2, 1500, 0, 256, gl.BRANCH_SOFTMAX | gl.ACCUMULATE),
    (2, 2, 900, 8, 400, ALL)])
def test_long_budget_softmax(H, Hkv, T, n_sink, window, flags):
    """Windows of 256 keys or more in bf16 at d = 128 (the long-budget softmax
    kernel): G = 8, 4, 2, 1, alone, added onto the linear branch's rows, and
    accumulated onto what o holds; every row of sampled chains against the
    oracle."""
    w = small(B=2, H=H, Hkv=Hkv, d=128, T=T, n_sink=n_sink, window=window, sigma=1.0)
    inp = to_dev(make_prefill_inputs(w, seed=window + T))
    if flags & gl.ACCUMULATE:
        base = torch.randn(w.B, w.T, w.H, w.d, device=DEV).to(torch.bfloat16)
        o = base.clone()
        gl.hybrid_prefill(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], n_sink, window,
                          flags=flags, o=o)
        torch.cuda.synchronize()
    else:
        o, st = run_prefill(inp, w, flags=flags)
    G = H // Hkv
    for bsel, heads in (([0], [0]), ([1], list(range(H - G, H)))):
        ref, S = oracle_subset(inp, w, bsel, heads, flags=flags & ~gl.ACCUMULATE)
        if flags & gl.ACCUMULATE:
            ref = ref + f64(base[bsel][:, :, heads])
        assert_close(f64(o[bsel][:, :, heads]), ref, False, f"o b{bsel} h{heads}")
        if flags & gl.WRITE_STATE:
            assert_close(f64(st[bsel][:, heads]), S, False, f"state b{bsel} h{heads}")


@pytest.mark.parametrize("dtype,d,n_sink,window,T", [("bf16", 128, 0, 1, 100), ("bf16", 128, 8, 1, 150),
                                                     ("f32", 64, 0, 1, 90), ("bf16", 64, 0, 64, 64)])
def test_degenerate_budgets(dtype, d, n_sink, window, T):
    """Window of one token, no sinks, and T equal to the budget."""
    w = small(B=1, H=4, Hkv=1, d=d, T=T, n_sink=n_sink, window=window, dtype=dtype)
    inp = to_dev(make_prefill_inputs(w, seed=T + window))
    o, st = run_prefill(inp, w)
    ref, S = O.hybrid_prefill(*(f64(inp[x]) for x in ("q", "k", "v", "a", "b")), n_sink, window)
    assert_close(f64(o), ref, dtype == "f32", "o")
    assert_close(f64(st), S, dtype == "f32", "state")


@pytest.mark.parametrize("n_sink,window,pos0", [(8, 56, 100), (8, 192, 300), (0, 1, 5), (2, 1, 1)])
def test_decode_largest_group_and_window_one(n_sink, window, pos0):
    """16 query heads per KV head (the largest group), narrow and wide cache
    passes; a one-token window, with and without sinks."""
    w = Workload("decg", B=3, H=16, Hkv=1, d=128, n_sink=n_sink, window=window, pos0=pos0, steps=3)
    inp = make_decode_inputs(w, device=DEV, seed=pos0 + window)
    st = {k: inp[k].clone() for k in ("state", "k_cache", "v_cache", "a_cache", "b_cache", "pos")}
    ref = {k: f64(st[k]) for k in st}
    ref["pos"] = st["pos"].cpu().numpy().astype(np.int64)
    for s_ in range(w.steps):
        step = {k: inp[k][s_] for k in ("q", "k", "v", "a", "b")}
        o = run_decode(step, st, w)
        ro, ref["state"], ref["k_cache"], ref["v_cache"], ref["a_cache"], ref["b_cache"], ref["pos"] = \
            O.decode_step(*(f64(step[x]) for x in ("q", "k", "v", "a", "b")), ref["state"], ref["k_cache"],
                          ref["v_cache"], ref["a_cache"], ref["b_cache"], ref["pos"], w.n_sink, w.window)
        assert_close(f64(o), ro, False, f"o step {s_}")
        assert_close(f64(st["state"]), ref["state"], False, f"state step {s_}")
        assert np.array_equal(f64(st["k_cache"]), ref["k_cache"])


# ------------------------------------------- weighted branches (hybridisation)

@pytest.mark.parametrize("B,H,Hkv,d,T,dtype,update", [
    (1, 4, 1, 128, 300, "bf16", "gdn"),     # few chains: one launch, linked softmax tiles
    (4, 32, 8, 128, 200, "bf16", "gdn"),    # many chains: preparation + scan, then softmax
    (2, 4, 2, 128, 260, "bf16", "gla"),
    (1, 2, 2, 64, 150, "f32", "gdn"),
    (256, 16, 4, 128, 520, "bf16", "gdn")])  # softmax with resident key blocks
def test_weighted_prefill(B, H, Hkv, d, T, dtype, update):
    w = small(B=B, H=H, Hkv=Hkv, d=d, T=T, dtype=dtype, update=update)
    inp = to_dev(make_prefill_inputs(w, seed=B * 100 + T))
    fp32 = dtype == "f32"
    plain, _ = run_prefill(inp, w, flags=ALL)
    same, _ = gl.hybrid_prefill(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], w.n_sink, w.window,
                                update=update, flags=ALL, weights=(1.0, 1.0))
    torch.cuda.synchronize()
    assert torch.equal(plain, same), "weights (1, 1) must equal the plain sum bitwise"
    wl, ws = 0.3, 1.7
    o, _ = gl.hybrid_prefill(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], w.n_sink, w.window,
                             update=update, flags=ALL, weights=(wl, ws))
    prior = torch.randn_like(o)
    acc = prior.clone()
    gl.hybrid_prefill(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], w.n_sink, w.window,
                      update=update, flags=ALL | gl.ACCUMULATE, o=acc, weights=(wl, ws))
    torch.cuda.synchronize()
    G = H // Hkv
    for bsel, heads in (([0], [0]), ([B - 1], [H - 1])):
        g = heads[0] // G
        qq = f64(inp["q"][bsel][:, :, heads])
        kk, vv = f64(inp["k"][bsel][:, :, g:g + 1]), f64(inp["v"][bsel][:, :, g:g + 1])
        aa, bb = f64(inp["a"][bsel][:, :, heads]), f64(inp["b"][bsel][:, :, heads])
        ref, _ = O.hybrid_prefill(qq, kk, vv, aa, bb, w.n_sink, w.window, update, ALL, wl, ws)
        assert_close(f64(o[bsel][:, :, heads]), ref, fp32, "weighted o")
        assert_close(f64(acc[bsel][:, :, heads]) - f64(prior[bsel][:, :, heads]), ref, fp32,
                     "weighted accumulate")


@pytest.mark.parametrize("dtype,n_sink,window,pos0", [("bf16", 3, 61, 70), ("bf16", 8, 300, 400),
                                                      ("f32", 3, 29, 40)])
def test_weighted_decode(dtype, n_sink, window, pos0):
    w = Workload("decw", B=2, H=8, Hkv=2, d=128 if dtype == "bf16" else 64, n_sink=n_sink,
                 window=window, pos0=pos0, steps=2, dtype=dtype)
    inp = make_decode_inputs(w, device=DEV, seed=pos0)
    fp32 = dtype == "f32"
    keys = ("state", "k_cache", "v_cache", "a_cache", "b_cache", "pos")
    st = {k: inp[k].clone() for k in keys}
    st1 = {k: inp[k].clone() for k in keys}
    ref = {k: f64(st[k]) for k in keys}
    ref["pos"] = st["pos"].cpu().numpy().astype(np.int64)
    for s_ in range(w.steps):
        step = {k: inp[k][s_] for k in ("q", "k", "v", "a", "b")}
        args = (step["q"], step["k"], step["v"], step["a"], step["b"])
        o = gl.hybrid_decode(*args, st["state"], st["k_cache"], st["v_cache"], st["a_cache"],
                             st["b_cache"], st["pos"], w.n_sink, w.window, weights=(-0.5, 2.0))
        o1 = gl.hybrid_decode(*args, st1["state"], st1["k_cache"], st1["v_cache"], st1["a_cache"],
                              st1["b_cache"], st1["pos"], w.n_sink, w.window, weights=(1.0, 1.0))
        if s_ == 0:   # the plain call from the same initial state
            o_plain = run_decode(step, {k: inp[k].clone() for k in keys}, w)
            assert torch.equal(o1, o_plain), "weights (1, 1) must equal the plain sum bitwise"
        torch.cuda.synchronize()
        ro, ref["state"], ref["k_cache"], ref["v_cache"], ref["a_cache"], ref["b_cache"], ref["pos"] = \
            O.decode_step(*(f64(x) for x in args), ref["state"], ref["k_cache"], ref["v_cache"],
                          ref["a_cache"], ref["b_cache"], ref["pos"], w.n_sink, w.window,
                          w_lin=-0.5, w_swa=2.0)
        assert_close(f64(o), ro, fp32, f"weighted decode step {s_}")
        assert_close(f64(st["state"]), ref["state"], fp32, f"state step {s_}")


# -------------------------------------------------------- short-conv decode

def assert_hist_close(got, ref, what):
    # histories are fp32 copies of rotated inputs: fp32 rounding of RoPE only
    got = f64(got)
    err = np.max(np.abs(got - ref)) if got.size else 0.0
    assert err <= 1e-5 * max(np.max(np.abs(ref)) if ref.size else 0.0, 1.0), f"{what}: {err:.3e}"


@pytest.mark.parametrize("dtype,d,ks,T0,flags,pos0", [
    ("bf16", 128, 8, 0, 3, 0), ("bf16", 128, 8, 5, 3, 0), ("bf16", 128, 8, 100, 3, 7),
    ("f32", 64, 8, 7, 3, 0), ("f32", 64, 4, 2, 1, 3), ("f32", 128, 1, 10, 3, 0),
    ("bf16", 64, 2, 9, 0, 0), ("f32", 128, 8, 300, 2, 1000)])
def test_shortconv_decode_steps(dtype, d, ks, T0, flags, pos0):
    """History after a prefill, then decode steps, for sequences at different
    positions: against the oracle's decode stepper, the oracle's prefill rows
    and the GPU prefill kernel's rows."""
    n = 10
    T0s = [T0, T0 + 3, max(T0 - 2, 0)]
    w = small(T=max(T0s) + n, d=d, dtype=dtype, shortconv=True, conv_ks=ks, H=4, Hkv=2, B=3)
    inp = to_dev(make_prefill_inputs(w, seed=11 + T0))
    theta = 1e4
    fp32 = dtype == "f32"
    m = ks - 1
    hist = [torch.zeros(w.B, m, nh * d, dtype=torch.float32, device=DEV) for nh in (w.H, w.Hkv, w.Hkv)]
    ref_hist = [np.zeros((w.B, m, nh * d)) for nh in (w.H, w.Hkv, w.Hkv)]
    for bi, t0 in enumerate(T0s):
        sl = slice(bi, bi + 1)
        hb = gl.shortconv_history_from_prefill(*(inp[x][sl, :t0].contiguous() for x in "qkv"), ks,
                                               theta, pos0, flags)
        rb = O.shortconv_history_from_prefill(*(f64(inp[x][sl, :t0]) for x in "qkv"), ks, theta,
                                              pos0, flags)
        for j in range(3):
            hist[j][sl] = hb[j]
            ref_hist[j][sl] = rb[j]
    torch.cuda.synchronize()
    for j, name in enumerate("qkv"):
        assert_hist_close(hist[j], ref_hist[j], f"history {name}")
    ref_pre = O.shortconv_qkv(*(f64(inp[x]) for x in ("q", "k", "v", "wq", "wk", "wv")), theta,
                              pos0, flags=flags)
    gpu_pre = gl.shortconv_qkv(inp["q"], inp["k"], inp["v"], inp["wq"], inp["wk"], inp["wv"],
                               rope_theta=theta, pos0=pos0, flags=flags)
    pos = torch.tensor(T0s, dtype=torch.int32, device=DEV)
    for s in range(n):
        ts = [t0 + s for t0 in T0s]
        idx = torch.tensor(ts, device=DEV)
        bsel = torch.arange(w.B, device=DEV)
        step = {x: inp[x][bsel, idx].contiguous() for x in "qkv"}
        out = gl.shortconv_decode(step["q"], step["k"], step["v"], inp["wq"], inp["wk"], inp["wv"],
                                  *hist, pos, theta, pos0, flags)
        torch.cuda.synchronize()
        ro = O.shortconv_decode_step(*(f64(step[x]) for x in "qkv"),
                                     *(f64(inp[x]) for x in ("wq", "wk", "wv")), *ref_hist,
                                     pos.cpu().numpy(), theta, pos0, flags)
        for j, name in enumerate("qkv"):
            rows_ref = ref_pre[j][np.arange(w.B), ts]
            assert_close(f64(out[j]), ro[j], fp32, f"{name} step {s} vs oracle step")
            assert_close(f64(out[j]), rows_ref, fp32, f"{name} step {s} vs oracle prefill")
            assert_close(f64(out[j]), f64(gpu_pre[j][bsel, idx]), fp32, f"{name} step {s} vs GPU prefill")
        pos += 1
    for j, name in enumerate("qkv"):
        assert_hist_close(hist[j], ref_hist[j], f"history {name} after the steps")


@pytest.mark.parametrize("name", ["qwen32b_t8192_gdn", "qwen32b_t8192_gla"])
def test_qwen32b_full_stack_decode(name):
    """Serving path of the Qwen-shaped stack: short-conv + layer prefill of T0
    tokens, then steps of short-conv decode feeding the layer's decode step
    (budget 896).  Each stage is checked against the oracle on sampled heads:
    the decode conv rows against the oracle conv of the raw inputs, the layer
    rows against the oracle layer on the GPU's conv outputs."""
    base = WORKLOADS[name]
    T0, n = 900, 4
    w = Workload(name, B=2, H=base.H, Hkv=base.Hkv, d=base.d, n_sink=base.n_sink,
                 window=base.window, T=T0 + n, sigma=base.sigma, update=base.update,
                 shortconv=True, rope_theta=base.rope_theta)
    raw = to_dev(make_prefill_inputs(w, seed=5))
    pre = {x: raw[x][:, :T0].contiguous() for x in ("q", "k", "v", "a", "b")}
    qc, kc, vc = gl.shortconv_qkv(pre["q"], pre["k"], pre["v"], raw["wq"], raw["wk"], raw["wv"],
                                  rope_theta=w.rope_theta, pos0=0, flags=gl.ROPE | gl.L2NORM)
    _, state = gl.hybrid_prefill(qc, kc, vc, pre["a"], pre["b"], w.n_sink, w.window,
                                 update=w.update, flags=gl.WRITE_STATE)
    kca, vca, aca, bca = gl.cache_from_prefill(kc, vc, pre["a"], pre["b"], w.H, w.n_sink, w.window,
                                               update=w.update)
    hist = gl.shortconv_history_from_prefill(pre["q"], pre["k"], pre["v"], w.conv_ks, w.rope_theta,
                                             0, gl.ROPE | gl.L2NORM)
    pos = torch.full((w.B,), T0, dtype=torch.int32, device=DEV)
    conv_rows = {x: [] for x in "qkv"}
    outs = []
    for t in range(T0, T0 + n):
        step = {x: raw[x][:, t].contiguous() for x in ("q", "k", "v", "a", "b")}
        sq, sk, sv = gl.shortconv_decode(step["q"], step["k"], step["v"], raw["wq"], raw["wk"],
                                         raw["wv"], *hist, pos, w.rope_theta, 0, gl.ROPE | gl.L2NORM)
        o = gl.hybrid_decode(sq, sk, sv, step["a"], step["b"], state, kca, vca, aca, bca, pos,
                             w.n_sink, w.window, update=w.update)
        for x, y in zip("qkv", (sq, sk, sv)):
            conv_rows[x].append(y)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.all(pos == T0 + n)
    G = w.H // w.Hkv
    full = {x: torch.cat([c, torch.stack(conv_rows[x], dim=1)], dim=1)
            for x, c in zip("qkv", (qc, kc, vc))}
    full.update(a=raw["a"], b=raw["b"])
    o_dec = torch.stack(outs, dim=1)                     # [B, n, H, d]
    rows = list(range(T0, T0 + n))
    for bsel, heads, g in (([0], [0, 3], 0), ([1], [61], 7)):
        cq = slice(heads[0], heads[-1] + 1)
        rq, rk, rv = O.shortconv_qkv(
            f64(raw["q"][bsel][:, :, cq]), f64(raw["k"][bsel][:, :, g:g + 1]),
            f64(raw["v"][bsel][:, :, g:g + 1]),
            f64(raw["wq"].view(w.H, w.d, -1)[cq].reshape(-1, w.conv_ks)),
            f64(raw["wk"].view(w.Hkv, w.d, -1)[g]), f64(raw["wv"].view(w.Hkv, w.d, -1)[g]),
            w.rope_theta, 0, flags=3)
        assert_close(f64(full["q"][bsel][:, rows][:, :, cq]), rq[:, rows], False, "decode conv q")
        assert_close(f64(full["k"][bsel][:, rows][:, :, g:g + 1]), rk[:, rows], False, "decode conv k")
        assert_close(f64(full["v"][bsel][:, rows][:, :, g:g + 1]), rv[:, rows], False, "decode conv v")
        ref, _ = oracle_subset(full, w, bsel, heads, rows=rows)
        assert_close(f64(o_dec[bsel][:, :, heads]), ref[:, rows], False, f"{name} decode o")
        assert heads[-1] // G == g


# ------------------------------------------------------------------ decode

def run_decode(step_inp, st, w, flags=ALL):
    o = gl.hybrid_decode(step_inp["q"], step_inp["k"], step_inp["v"], step_inp["a"],
                         step_inp.get("b"), st["state"], st["k_cache"], st["v_cache"],
                         st["a_cache"], st["b_cache"], st["pos"], w.n_sink, w.window,
                         update=w.update, flags=flags)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("update", ["gdn", "gla", "dgd"])
@pytest.mark.parametrize("pos0", [0, 2, 6, 60, 63, 64, 65, 500])
def test_decode_steps_small(update, pos0):
    w = Workload("dec", B=3, H=4, Hkv=2, d=128, n_sink=3, window=61, update=update, pos0=pos0,
                 steps=6)
    inp = make_decode_inputs(w, device=DEV, seed=pos0)
    st = {k: inp[k].clone() for k in ("state", "k_cache", "v_cache", "a_cache", "b_cache", "pos")}
    ref = {k: f64(st[k]) for k in st}
    ref["pos"] = st["pos"].cpu().numpy().astype(np.int64)
    for s in range(w.steps):
        step = {k: inp[k][s] for k in ("q", "k", "v", "a", "b")}
        o = run_decode(step, st, w)
        ro, ref["state"], ref["k_cache"], ref["v_cache"], ref["a_cache"], ref["b_cache"], ref["pos"] = \
            O.decode_step(f64(step["q"]), f64(step["k"]), f64(step["v"]), f64(step["a"]),
                          f64(step["b"]), ref["state"], ref["k_cache"], ref["v_cache"],
                          ref["a_cache"], ref["b_cache"], ref["pos"], w.n_sink, w.window,
                          update=update)
        assert_close(f64(o), ro, False, f"o step {s}")
        assert_close(f64(st["state"]), ref["state"], False, f"state step {s}")
        assert np.array_equal(st["pos"].cpu().numpy(), ref["pos"])
        # caches are copies of bf16 / fp32 inputs: exact
        assert np.array_equal(f64(st["k_cache"]), ref["k_cache"])
        assert np.array_equal(f64(st["v_cache"]), ref["v_cache"])
        assert np.array_equal(f64(st["a_cache"]), ref["a_cache"])
        if update != "gla":
            assert np.array_equal(f64(st["b_cache"]), ref["b_cache"])


@pytest.mark.parametrize("dtype,n_sink,window,pos0,update", [
    ("f32", 3, 61, 62, "gdn"), ("bf16", 8, 592, 5, "gdn"), ("bf16", 8, 592, 598, "gla"),
    ("bf16", 0, 300, 1000, "gdn"), ("f32", 8, 120, 130, "gla"), ("bf16", 8, 888, 4000, "gdn"),
    ("bf16", 8, 592, 598, "dgd"), ("f32", 3, 61, 62, "dgd")])
def test_decode_long_budgets(dtype, n_sink, window, pos0, update):
    """Budgets that take several staged passes of cached rows (online softmax
    across passes, a partial last pass), against the oracle's decode step."""
    w = Workload("decl", B=2, H=8, Hkv=2, d=128 if dtype == "bf16" else 64, n_sink=n_sink,
                 window=window, update=update, pos0=pos0, steps=3, dtype=dtype)
    inp = make_decode_inputs(w, device=DEV, seed=pos0 + window)
    st = {k: inp[k].clone() for k in ("state", "k_cache", "v_cache", "a_cache", "b_cache", "pos")}
    ref = {k: f64(st[k]) for k in st}
    ref["pos"] = st["pos"].cpu().numpy().astype(np.int64)
    fp32 = dtype == "f32"
    for s in range(w.steps):
        step = {k: inp[k][s] for k in ("q", "k", "v", "a", "b")}
        o = run_decode(step, st, w)
        ro, ref["state"], ref["k_cache"], ref["v_cache"], ref["a_cache"], ref["b_cache"], ref["pos"] = \
            O.decode_step(f64(step["q"]), f64(step["k"]), f64(step["v"]), f64(step["a"]),
                          f64(step["b"]), ref["state"], ref["k_cache"], ref["v_cache"],
                          ref["a_cache"], ref["b_cache"], ref["pos"], w.n_sink, w.window,
                          update=update)
        assert_close(f64(o), ro, fp32, f"o step {s}")
        assert_close(f64(st["state"]), ref["state"], fp32, f"state step {s}")
        assert np.array_equal(f64(st["k_cache"]), ref["k_cache"])
        assert np.array_equal(f64(st["v_cache"]), ref["v_cache"])


def test_decode_b256_sampled_sequences():
    w = WORKLOADS["decode_b256"]
    inp = make_decode_inputs(w, device=DEV, steps=3)
    st = {k: inp[k].clone() for k in ("state", "k_cache", "v_cache", "a_cache", "b_cache", "pos")}
    bsel = [0, 1, 128, 255]
    ref = {k: f64(st[k][bsel]) for k in st if k != "pos"}
    ref["pos"] = st["pos"][bsel].cpu().numpy().astype(np.int64)
    for s in range(3):
        step = {k: inp[k][s] for k in ("q", "k", "v", "a", "b")}
        o = run_decode(step, st, w)
        ro, ref["state"], ref["k_cache"], ref["v_cache"], ref["a_cache"], ref["b_cache"], ref["pos"] = \
            O.decode_step(*(f64(step[k][bsel]) for k in ("q", "k", "v", "a", "b")), ref["state"],
                          ref["k_cache"], ref["v_cache"], ref["a_cache"], ref["b_cache"],
                          ref["pos"], w.n_sink, w.window)
        assert_close(f64(o[bsel]), ro, False, f"o step {s}")
        assert_close(f64(st["state"][bsel]), ref["state"], False, f"state step {s}")
    assert torch.all(st["pos"] == w.pos0 + 3)


@pytest.mark.parametrize("update", ["gdn", "gla"])
@pytest.mark.parametrize("T0", [62, 63, 64, 65, 200])
def test_prefill_then_decode_matches_longer_prefill(update, T0):
    n = 9
    w = small(T=T0 + n, B=2, H=4, Hkv=2, update=update)
    inp = to_dev(make_prefill_inputs(w, seed=T0))
    o_full, _ = run_prefill(inp, w)
    pre = {k: inp[k][:, :T0].contiguous() for k in ("q", "k", "v", "a", "b")}
    _, state = run_prefill(pre, w)
    kc, vc, ac, bc = gl.cache_from_prefill(pre["k"], pre["v"], pre["a"], pre["b"], w.H,
                                           w.n_sink, w.window, update=update)
    st = dict(state=state, k_cache=kc, v_cache=vc, a_cache=ac, b_cache=bc,
              pos=torch.full((w.B,), T0, dtype=torch.int32, device=DEV))
    ref_full, _ = O.hybrid_prefill(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["a"]),
                                   f64(inp["b"]), w.n_sink, w.window, update=update)
    for t in range(T0, T0 + n):
        step = {k: inp[k][:, t].contiguous() for k in ("q", "k", "v", "a", "b")}
        o = run_decode(step, st, w)
        assert_close(f64(o), ref_full[:, t], False, f"decode t={t}")
        assert_close(f64(o), f64(o_full[:, t]), False, f"decode vs prefill t={t}")
    kc2, vc2, ac2, bc2 = gl.cache_from_prefill(inp["k"], inp["v"], inp["a"], inp["b"], w.H,
                                               w.n_sink, w.window, update=update)
    assert torch.equal(st["k_cache"], kc2) and torch.equal(st["v_cache"], vc2)
    assert torch.equal(st["a_cache"], ac2)
    if update == "gdn":
        assert torch.equal(st["b_cache"], bc2)


# ---------------------------------------------------------- invariants

def test_bitwise_deterministic_and_linear_in_v():
    w = WORKLOADS["llama8b_t4096"]
    inp = to_dev(make_prefill_inputs(w, device=DEV, seed=1))
    o1, s1 = run_prefill(inp, w)
    o2, s2 = run_prefill(inp, w)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    inp2 = dict(inp)
    inp2["v"] = inp["v"] * 2
    o3, s3 = run_prefill(inp2, w)
    assert torch.equal(o3, o1 * 2) and torch.equal(s3, s1 * 2)


def test_decode_bitwise_deterministic():
    w = WORKLOADS["decode_b256"]
    inp = make_decode_inputs(w, device=DEV, steps=1, B=32)
    outs = []
    for _ in range(2):
        st = {k: inp[k].clone() for k in ("state", "k_cache", "v_cache", "a_cache", "b_cache", "pos")}
        step = {k: inp[k][0] for k in ("q", "k", "v", "a", "b")}
        outs.append((run_decode(step, st, w), st["state"]))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("T,window,exact", [(250, 56, True), (333, 56, False), (333, 130, False)])
def test_split_calls_equal_fused_call_and_accumulate(T, window, exact):
    """LINEAR then SOFTMAX|ACCUMULATE reproduces the fused call, and
    ACCUMULATE adds the layer to what o holds.  With three stream chunks
    (T 250, window 56) the fused call runs the scan with softmax tiles adding
    onto its published rows, the same operations in the same order as the two
    split calls, and the two agree bit for bit.  With five chunks at window 56
    the fused call takes the segmented scan, whose layer kernel sums both
    branches in fp32 and rounds once; at window 130 the separate softmax
    launch takes 32-row query tiles where the linked ones take 64, so the
    keys' partial sums are combined in another order.  There the two agree to
    the bf16 tolerance."""
    w = small(T=T, B=2, H=8, Hkv=2, window=window)
    inp = to_dev(make_prefill_inputs(w, seed=9))
    fused, _ = run_prefill(inp, w, flags=ALL)
    o, _ = gl.hybrid_prefill(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], w.n_sink, w.window,
                             flags=gl.BRANCH_LINEAR)
    gl.hybrid_prefill(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], w.n_sink, w.window,
                      flags=gl.BRANCH_SOFTMAX | gl.ACCUMULATE, o=o)
    torch.cuda.synchronize()
    if exact:
        assert torch.equal(o, fused)
    else:
        assert_close(f64(o), f64(fused), False, "split vs fused")
    base = torch.randn_like(fused, dtype=torch.float32).to(fused.dtype)
    acc = base.clone()
    gl.hybrid_prefill(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], w.n_sink, w.window,
                      flags=ALL | gl.ACCUMULATE, o=acc)
    torch.cuda.synchronize()
    ref, _ = O.hybrid_prefill(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["a"]),
                              f64(inp["b"]), w.n_sink, w.window)
    assert_close(f64(acc), f64(base) + ref, False, "accumulate")
