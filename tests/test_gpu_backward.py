"""GPU parity of the backward pass (the training path) against the fp64
oracle's reverse-mode gradients (oracle/backward.py, itself pinned to finite
differences of the forward oracle): the gradients of
sum(d_o * o) + sum(d_state * S_final) with respect to q, k, v, a, b for bf16
GDN at d = 128, both branches, weighted or plain sum.

Tolerance: max-abs error <= 2e-2 * max|ref| + 1e-6 per gradient (bf16
operands, fp32 accumulation, as the forward; the absolute term covers
gradients that are exactly zero, such as da of a stream whose first token is
its only one)."""

import numpy as np
import pytest
import torch

import swa_chunked_gated_amd as gl
from oracle import backward as OB
from workloads import Workload, make_prefill_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def close(got, ref, what):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.max(np.abs(got - ref)) if got.size else 0.0
    bound = 2e-2 * np.max(np.abs(ref)) + 1e-6
    assert err <= bound, f"{what}: max abs err {err:.3e} > {bound:.3e}"


def run_case(B, H, Hkv, T, n_sink, window, weights=(1.0, 1.0), state_grad=True, seed=0):
    w = Workload("bwd", B=B, H=H, Hkv=Hkv, d=128, n_sink=n_sink, window=window, T=T, sigma=0.5)
    inp = {x: t.to(DEV) for x, t in make_prefill_inputs(w, seed=seed).items()}
    g = torch.Generator(device="cpu").manual_seed(seed + 1)
    d_o = (torch.randn(B, T, H, 128, generator=g) * 0.5).to(torch.bfloat16).to(DEV)
    d_state = (torch.randn(B, H, 128, 128, generator=g) * 0.05).to(DEV) if state_grad else None
    print(f"backward B={B} H={H} Hkv={Hkv} T={T} sinks={n_sink} window={window} w={weights}", flush=True)
    got = gl.hybrid_prefill_backward(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], n_sink, window,
                                     d_o, d_state, weights=weights)
    torch.cuda.synchronize()
    ref = OB.hybrid_prefill_backward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["a"]),
                                     f64(inp["b"]), n_sink, window, f64(d_o),
                                     None if d_state is None else f64(d_state),
                                     w_lin=weights[0], w_swa=weights[1])
    for name, x, y in zip(("dq", "dk", "dv", "da", "db"), got, ref):
        close(f64(x), y, name)


@pytest.mark.parametrize("B,H,Hkv,T,n_sink,window", [
    (1, 4, 1, 300, 8, 56),      # 4 chunks, the last one ragged
    (2, 8, 2, 257, 0, 1),       # no sinks, one-token window
    (1, 4, 2, 200, 16, 128),    # largest budget of the one-pass kernels
    (1, 2, 1, 700, 3, 100),     # 10 chunks
    (1, 4, 4, 64, 8, 56),       # T = budget: softmax branch only
    (1, 4, 1, 66, 64, 1),       # 64 sinks, one stream token
])
def test_backward_matches_oracle(B, H, Hkv, T, n_sink, window):
    run_case(B, H, Hkv, T, n_sink, window, seed=T + window)


@pytest.mark.parametrize("weights", [(1.0, 0.0), (0.0, 1.0), (0.7, 1.3)])
def test_backward_branch_weights(weights):
    run_case(1, 4, 2, 330, 8, 56, weights=weights, seed=7)


def test_backward_without_state_gradient():
    run_case(1, 4, 1, 260, 8, 56, state_grad=False, seed=11)
