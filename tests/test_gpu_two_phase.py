"""Two-phase prefill: PREPARE_ONLY (the state-independent chunk preparation
into the workspace) followed by PREPARED (the rest of the same call) gives
exactly what one call gives, on the three launch plans with a separate
preparation: the one-pass layer (both branches, d = 128, many chains), the
light preparation plus the many-chain scan (linear branch only), and GLA."""

import pytest
import torch

import swa_chunked_gated_amd as gl
from workloads import Workload, make_prefill_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("update,flags,T", [
    ("gdn", gl.BRANCH_LINEAR | gl.BRANCH_SOFTMAX | gl.WRITE_STATE, 700),
    ("gdn", gl.BRANCH_LINEAR | gl.WRITE_STATE, 700),
    ("gla", gl.BRANCH_LINEAR | gl.BRANCH_SOFTMAX | gl.WRITE_STATE, 457),
])
def test_prepare_then_prepared_equals_one_call(update, flags, T):
    w = Workload(name="two_phase", B=8, H=16, Hkv=4, d=128, n_sink=8, window=120, T=T, sigma=1.0,
                 dtype="bf16", update=update)
    inp = {k: v.to(DEV) for k, v in make_prefill_inputs(w, seed=T + len(update)).items()}
    args = (inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], w.n_sink, w.window)
    print(f"two-phase {update} flags={flags} T={T}", flush=True)
    o1, s1 = gl.hybrid_prefill(*args, update=update, flags=flags)
    nws = gl.prefill_workspace_bytes(w.B, w.T, w.H, w.Hkv, w.d, w.n_sink, w.window, torch.bfloat16,
                                     update=update, flags=flags)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    o2 = torch.full_like(o1, 7.0)
    s2 = torch.full_like(s1, 7.0)
    gl.hybrid_prefill(*args, update=update, flags=flags | gl.PREPARE_ONLY, o=o2, state_out=s2,
                      workspace=ws)
    torch.cuda.synchronize()
    assert bool((o2 == 7.0).all()) and bool((s2 == 7.0).all())     # outputs untouched
    gl.hybrid_prefill(*args, update=update, flags=flags | gl.PREPARED, o=o2, state_out=s2,
                      workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(s1, s2)
