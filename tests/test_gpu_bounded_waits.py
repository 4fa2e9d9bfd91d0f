"""The one-launch few-chain prefill hands chunks between workgroups through
flags, and every wait on a flag is bounded in time.  These tests force a
wait to run into its bound from the host (test-only fault injection: a
producer that never publishes, with a 200 us bound) and check that the
give-up is visible: the rows and states computed from the missing data are
NaN, the rows that do not depend on it are exact to tolerance, every kernel
exits, and the next call (faults cleared) is correct again."""

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
    err = np.max(np.abs(got - ref))
    bound = 2e-2 * np.max(np.abs(ref))
    assert np.all(np.isfinite(got)) and err <= bound, f"{what}: {err:.3e} > {bound:.3e}"


@pytest.mark.parametrize("faults", [1, 2])
def test_wait_give_up_poisons_dependent_rows(faults):
    # few chains, four query heads per KV head, both branches, a window
    # longer than 128 (no segmented scan): one launch
    w = Workload("waits", B=1, H=8, Hkv=2, d=128, n_sink=8, window=130, T=600, sigma=0.5)
    inp = {x: t.to(DEV) for x, t in make_prefill_inputs(w, seed=3).items()}
    args = (inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], w.n_sink, w.window)
    ref, S = O.hybrid_prefill(*(f64(inp[x]) for x in ("q", "k", "v", "a", "b")), w.n_sink, w.window)
    N = w.budget
    try:
        gl.set_test_faults(faults, 200)
        o, st = gl.hybrid_prefill(*args, flags=ALL | gl.WRITE_STATE)
        torch.cuda.synchronize()
    finally:
        gl.set_test_faults()
    o, st = f64(o), f64(st)
    # rows t >= N carry the linear branch: the scan computed them from chunk
    # tiles it never saw published (faults 1), or the softmax tiles never saw
    # the scan's rows published (faults 2)
    assert np.all(np.isnan(o[:, N:])), "rows depending on unpublished data must be NaN"
    close(o[:, :N], ref[:, :N], "softmax-only rows")
    if faults == 1:
        assert np.all(np.isnan(st)), "the state was computed from unpublished chunks"
    else:
        close(st, S, "state")
    # faults cleared: the same call is correct again
    o2, st2 = gl.hybrid_prefill(*args, flags=ALL | gl.WRITE_STATE)
    torch.cuda.synchronize()
    close(f64(o2), ref, "o after the faults are cleared")
    close(f64(st2), S, "state after the faults are cleared")
