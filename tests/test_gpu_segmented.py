"""GPU parity of the segmented scan for few chains (bf16 GDN, d = 128, both
branches): the chunk preparation, the per-segment affine maps (N from the
zero state, M from the identity without values), the carry across segments
and the one-pass layer kernel run on every segment from its incoming state,
against the fp64 oracle.  Segment counts and lengths vary with the shape:
T = 4096 at 32 chains gives 8 segments of 8 chunks (the last one 7), T = 700
gives 5 of 2, T = 257 gives 4 of 1; ragged tails, sinks 0..16, windows
1..128, with and without the final state."""

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


def close(got, ref, what):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.max(np.abs(got - ref))
    bound = 2e-2 * np.max(np.abs(ref))
    assert err <= bound, f"{what}: max abs err {err:.3e} > {bound:.3e}"


def oracle_heads(inp, w, b, heads):
    G = w.H // w.Hkv
    g = heads[0] // G
    assert all(h // G == g for h in heads)
    q = f64(inp["q"][[b]][:, :, heads])
    k = f64(inp["k"][[b]][:, :, g:g + 1])
    v = f64(inp["v"][[b]][:, :, g:g + 1])
    a = f64(inp["a"][[b]][:, :, heads])
    bb = f64(inp["b"][[b]][:, :, heads])
    return O.hybrid_prefill(q, k, v, a, bb, w.n_sink, w.window)


@pytest.mark.parametrize("B,H,Hkv,T,n_sink,window,state", [
    (1, 32, 8, 4096, 8, 56, True),      # 8 segments x 8 chunks (last 7)
    (1, 32, 8, 700, 8, 56, True),       # 5 x 2
    (1, 32, 8, 257, 8, 56, True),       # 4 x 1
    (1, 32, 8, 1000, 8, 56, False),     # no final state: the last map is not formed
    (2, 16, 4, 1111, 0, 1, True),       # no sinks, one-token window, ragged tail
    (1, 64, 16, 900, 16, 128, True),    # 64 chains: 4 segments; largest budget
    (1, 8, 2, 2000, 3, 100, False),     # 8 chains: one chunk per segment
])
def test_segmented_scan(B, H, Hkv, T, n_sink, window, state):
    w = Workload("seg", B=B, H=H, Hkv=Hkv, d=128, n_sink=n_sink, window=window, T=T, sigma=0.5)
    inp = {x: t.to(DEV) for x, t in make_prefill_inputs(w, seed=T + window).items()}
    flags = ALL | (gl.WRITE_STATE if state else 0)
    print(f"segmented scan B={B} H={H} T={T} sinks={n_sink} window={window}", flush=True)
    o, st = gl.hybrid_prefill(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], n_sink, window,
                              flags=flags)
    torch.cuda.synchronize()
    G = H // Hkv
    picks = [(0, [0]), (B - 1, list(range(H - G, H))), (B // 2, [G + 1] if H > G else [0])]
    for b, heads in picks:
        ref, S = oracle_heads(inp, w, b, heads)
        close(f64(o[[b]][:, :, heads]), ref, f"o b{b} h{heads}")
        if state:
            close(f64(st[[b]][:, heads]), S, f"state b{b} h{heads}")


def test_segmented_two_phase_and_noalloc_agree():
    """The preparation as its own call (GDN_PREPARE_ONLY, then GDN_PREPARED)
    and the allocation-free entry point give the fused call's bits."""
    w = Workload("seg2", B=1, H=32, Hkv=8, d=128, n_sink=8, window=56, T=2100, sigma=0.5)
    inp = {x: t.to(DEV) for x, t in make_prefill_inputs(w, seed=5).items()}
    args = (inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], w.n_sink, w.window)
    flags = ALL | gl.WRITE_STATE
    o1, s1 = gl.hybrid_prefill(*args, flags=flags)
    ws = torch.empty(gl.prefill_workspace_bytes(w.B, w.T, w.H, w.Hkv, w.d, w.n_sink, w.window,
                                                torch.bfloat16, flags=flags),
                     dtype=torch.uint8, device=DEV)
    gl.hybrid_prefill(*args, flags=flags | gl.PREPARE_ONLY, workspace=ws)
    o2, s2 = gl.hybrid_prefill(*args, flags=flags | gl.PREPARED, workspace=ws)
    o3, s3 = gl.hybrid_prefill_noalloc(*args, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.equal(o1, o3) and torch.equal(s1, s3)
