"""The allocation-free prefill entry point against the regular one, through
the C ABI: the same kernels with the library's per-GPU workspace array in
place of a caller workspace, so the outputs must be bitwise equal.  Each
case makes two calls in a row on the shared array, the second with a smaller
input (the array then holds the first call's contents)."""

import pytest
import torch

import swa_chunked_gated_amd as gl
from workloads import Workload, make_prefill_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
ALL = gl.BRANCH_LINEAR | gl.BRANCH_SOFTMAX


def _inputs(w, seed):
    return {x: t.to(DEV) for x, t in make_prefill_inputs(w, seed=seed).items()}


def _both(w, inp, flags):
    args = (inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], w.n_sink, w.window)
    ref_o, ref_s = gl.hybrid_prefill(*args, update=w.update, flags=flags)
    o, s = gl.hybrid_prefill_noalloc(*args, update=w.update, flags=flags)
    torch.cuda.synchronize()
    return (ref_o, ref_s), (o, s)


def _equal(ref, got, flags):
    if flags & ALL:
        assert torch.equal(ref[0], got[0]), "o differs from the regular entry point"
    if flags & gl.WRITE_STATE:
        assert torch.equal(ref[1], got[1]), "state differs from the regular entry point"


# (first call, second smaller call): few chains (both branches: the
# segmented scan's maps and states in the array; linear only: the one-launch
# path, flags and hand-off epochs in the array), many-chain light
# preparation, GLA, fp32
CASES = [
    (dict(B=1, H=32, Hkv=8, d=128, T=2000), dict(B=1, H=8, Hkv=2, d=128, T=700)),
    (dict(B=8, H=32, Hkv=8, d=128, T=900), dict(B=4, H=32, Hkv=8, d=128, T=333)),
    (dict(B=2, H=8, Hkv=2, d=128, T=800, update="gla"), dict(B=1, H=4, Hkv=2, d=128, T=300, update="gla")),
    (dict(B=1, H=4, Hkv=2, d=64, T=500, dtype="f32"), dict(B=1, H=2, Hkv=2, d=64, T=200, dtype="f32")),
]


@pytest.mark.parametrize("first,second", CASES)
@pytest.mark.parametrize("flags", [ALL | gl.WRITE_STATE, gl.BRANCH_LINEAR])
def test_noalloc_equals_regular_entry_point(first, second, flags):
    for i, kw in enumerate((first, second)):
        w = Workload("na", n_sink=8, window=56, sigma=0.5, **kw)
        inp = _inputs(w, seed=10 * i + kw["T"])
        ref, got = _both(w, inp, flags)
        _equal(ref, got, flags)


def test_noalloc_rejects_workspace_beyond_the_array():
    w = Workload("big", B=64, H=32, Hkv=8, d=128, n_sink=8, window=56, T=8192)
    need = gl.prefill_workspace_bytes(w.B, w.T, w.H, w.Hkv, w.d, w.n_sink, w.window, torch.bfloat16)
    assert need > gl.noalloc_max_workspace()
    q = torch.zeros(w.B, w.T, w.H, w.d, dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros(w.B, w.T, w.Hkv, w.d, dtype=torch.bfloat16, device=DEV)
    g = torch.ones(w.B, w.T, w.H, device=DEV)
    o = torch.empty_like(q)
    with pytest.raises(gl.GdnError) as e:
        gl.hybrid_prefill_noalloc(q, kv, kv, g, g, w.n_sink, w.window, o=o)
    assert e.value.code == -3
