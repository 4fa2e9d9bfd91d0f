"""GPU parity of the delta rule with a diagonal (per-channel) gate against
the fp64 oracle: prefill (per-channel-gate preparation with the
unit-lower-triangular solve, then the scan in its third mode), the cache
fill, and decode steps continuing from a prefill."""

import numpy as np
import pytest
import torch

import swa_chunked_gated_amd as gl
from oracle import hybrid as O
from workloads import Workload, make_prefill_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
ALL = gl.BRANCH_LINEAR | gl.BRANCH_SOFTMAX


def f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def assert_close(got, ref, fp32, what=""):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.max(np.abs(got - ref)) if got.size else 0.0
    bound = 1e-4 if fp32 else 2e-2 * max(np.max(np.abs(ref)), 1e-30)
    assert err <= bound, f"{what}: max abs err {err:.3e} > {bound:.3e}"


def dgd_workload(**kw):
    base = dict(name="dgd", B=2, H=4, Hkv=2, d=128, n_sink=8, window=56, T=257, sigma=0.5,
                dtype="bf16", update="dgd")
    base.update(kw)
    return Workload(**base)


@pytest.mark.parametrize("B,H,Hkv,d,T,n_sink,window,dtype,gate_mean", [
    (2, 4, 2, 128, 257, 8, 56, "bf16", -4.0),    # ragged last chunk
    (1, 2, 1, 128, 700, 0, 120, "bf16", 1.0),    # no sinks, many chunks, gates ~0.27
    (2, 4, 2, 64, 300, 8, 56, "bf16", 3.0),      # strong per-channel forgetting
    (1, 2, 2, 64, 200, 3, 20, "f32", -4.0),      # fp32 at d = 64
    (16, 16, 4, 128, 330, 8, 120, "bf16", -4.0), # 256 chains: the 8-wave scan
    (1, 2, 1, 128, 64 + 65, 8, 56, "bf16", -4.0),  # a single stream token past one chunk
])
def test_dgd_prefill(B, H, Hkv, d, T, n_sink, window, dtype, gate_mean):
    w = dgd_workload(B=B, H=H, Hkv=Hkv, d=d, T=T, n_sink=n_sink, window=window, dtype=dtype,
                     gate_mean=gate_mean)
    inp = {k: v.to(DEV) for k, v in make_prefill_inputs(w, seed=T + d).items()}
    print(f"dgd prefill B={B} H={H} d={d} T={T} {dtype}", flush=True)
    o, st = gl.hybrid_prefill(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], n_sink, window,
                              update="dgd", flags=ALL | gl.WRITE_STATE)
    torch.cuda.synchronize()
    # at most two sequences and the heads of one KV group against the oracle
    bsel = [0] if B <= 2 else [0, B - 1]
    G = H // Hkv
    heads = list(range(G))
    ref, S = O.hybrid_prefill(f64(inp["q"][bsel][:, :, heads]), f64(inp["k"][bsel][:, :, :1]),
                              f64(inp["v"][bsel][:, :, :1]), f64(inp["a"][bsel][:, :, heads]),
                              f64(inp["b"][bsel][:, :, heads]), n_sink, window, update="dgd")
    fp32 = dtype == "f32"
    assert_close(f64(o[bsel][:, :, heads]), ref, fp32, "o")
    assert_close(f64(st[bsel][:, heads]), S, fp32, "state")


def test_dgd_prefill_cache_then_decode_equals_longer_prefill():
    """prefill(T0) -> cache fill -> decode steps reproduce the oracle's
    prefill(T0 + n) rows, across evictions from the window into the state."""
    n_sink, window, T0, n = 4, 60, 150, 70
    w = dgd_workload(B=2, H=4, Hkv=2, d=128, n_sink=n_sink, window=window, T=T0 + n)
    inp = {k: v.to(DEV) for k, v in make_prefill_inputs(w, seed=5).items()}
    pre = {k: inp[k][:, :T0].contiguous() for k in ("q", "k", "v", "a", "b")}
    _, st = gl.hybrid_prefill(pre["q"], pre["k"], pre["v"], pre["a"], pre["b"], n_sink, window,
                              update="dgd", flags=ALL | gl.WRITE_STATE)
    kc, vc, ac, bc = gl.cache_from_prefill(pre["k"], pre["v"], pre["a"], pre["b"], w.H, n_sink,
                                           window, update="dgd")
    pos = torch.full((w.B,), T0, dtype=torch.int32, device=DEV)
    ref, _ = O.hybrid_prefill(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["a"]),
                              f64(inp["b"]), n_sink, window, update="dgd")
    for t in range(T0, T0 + n):
        o = gl.hybrid_decode(inp["q"][:, t].contiguous(), inp["k"][:, t].contiguous(),
                             inp["v"][:, t].contiguous(), inp["a"][:, t].contiguous(),
                             inp["b"][:, t].contiguous(), st, kc, vc, ac, bc, pos, n_sink, window,
                             update="dgd", flags=ALL)
        torch.cuda.synchronize()
        assert_close(f64(o), ref[:, t], False, f"o t={t}")
    assert bool((pos == T0 + n).all())


def test_dgd_b8_t8192_sampled():
    """The benchmarked shape (B = 8, T = 8192, 32 / 8 heads, budget 8 + 120,
    state out) in the launch configuration the bench times; sequence 0's
    first KV group against the oracle on every row and the final state."""
    from workloads import WORKLOADS
    w = WORKLOADS["dgd_b8_t8192"]
    inp = make_prefill_inputs(w, device=DEV)
    o, st = gl.hybrid_prefill(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], w.n_sink, w.window,
                              update="dgd", flags=ALL | gl.WRITE_STATE)
    torch.cuda.synchronize()
    heads = [0, 3]
    ref, S = O.hybrid_prefill(f64(inp["q"][:1][:, :, heads]), f64(inp["k"][:1][:, :, :1]),
                              f64(inp["v"][:1][:, :, :1]), f64(inp["a"][:1][:, :, heads]),
                              f64(inp["b"][:1][:, :, heads]), w.n_sink, w.window, update="dgd")
    assert_close(f64(o[:1][:, :, heads]), ref, False, "o")
    assert_close(f64(st[:1][:, heads]), S, False, "state")
