"""Exact index-set probes of every softmax code path, and long decode parity.

Mask probe: with q = 0 every logit is 0, so the softmax weights are exactly
1/|A(t)| over the attended keys, and with the linear branch's read-out
S^T q = 0 the linear branch contributes exactly 0.  With v one-hot (each key
carries a unit vector in one dimension), o[t] * |A(t)| is the exact count of
attended keys per dimension, and is compared as integers with the counts of
A(t) = { i <= t : i < n_sink or i > t - window } (page "The Key to Going
Linear", section 填补近似缺口的实用设计: 8 sink tokens always attended plus a
sliding window of the most recent tokens, current one included).  A single
dropped or extra key changes one count by one.

The prefill probes are placed on the shapes that reach each kernel path:
  * swa_kernel with one, two and four query heads per workgroup (G = 1, 2, 4
    with few sequences), bf16 and fp32 key blocks;
  * swa_ring_kernel (resident key blocks: bf16, four query heads per KV head,
    at least four 64-row tiles per workgroup, many sequences);
  * swa_long_kernel (bf16, d = 128, windows of 256 keys or more: key blocks
    by direct loads, 8 waves over 1 to 8 query heads);
  * the softmax tiles linked into the one-launch few-chain layer kernel,
    and the softmax waves of the one-pass layer kernel run per segment by
    the segmented scan
    (bf16, few chains, both branches, G a multiple of 4);
and the decode probe crosses the sink boundary, the full budget and several
wraps of the ring.
"""

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


def expected_counts(T, n_sink, window, d):
    """[T, d] int64: per row t, how many keys of A(t) carry each one-hot
    dimension (key i carries dimension i mod d), and [T] sizes |A(t)|."""
    cnt = np.zeros((T, d), np.int64)
    size = np.zeros(T, np.int64)
    for t in range(T):
        A = O.softmax_index_set(t, n_sink, window)
        cnt[t] = np.bincount(A % d, minlength=d)
        size[t] = len(A)
    return cnt, size


def probe_inputs(B, T, H, Hkv, d, dtype, seed=0, gates=False):
    """q = 0, random unit keys, v one-hot by token index mod d, gates in range."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.zeros(B, T, H, d, dtype=dtype, device=DEV)
    k = torch.randn(B, T, Hkv, d, generator=g)
    k = (k / k.norm(dim=-1, keepdim=True)).to(dtype).to(DEV)
    v = torch.nn.functional.one_hot(torch.arange(T) % d, d).to(dtype)
    v = v.view(1, T, 1, d).expand(B, T, Hkv, d).contiguous().to(DEV)
    if gates:
        a = torch.exp(-torch.nn.functional.softplus(torch.randn(B, T, H, generator=g) - 4)).to(DEV)
        b = torch.sigmoid(torch.randn(B, T, H, generator=g)).to(DEV)
    else:
        a = torch.ones(B, T, H, device=DEV)
        b = torch.ones(B, T, H, device=DEV)
    return q, k, v, a, b


def check_counts(o, n_sink, window):
    """o [B, T, H, d] from a probe: every (sequence, head) must reproduce the
    exact counts; compared on the GPU as integers."""
    B, T, H, d = o.shape
    cnt, size = expected_counts(T, n_sink, window, d)
    want = torch.from_numpy(cnt).to(DEV)
    sz = torch.from_numpy(size).to(DEV, torch.float64)
    got = torch.round(o.to(torch.float64) * sz.view(1, T, 1, 1)).to(torch.int64)
    bad = got != want.view(1, T, 1, d)
    if bool(bad.any()):
        bi, t, h, j = (int(x) for x in torch.nonzero(bad)[0])
        raise AssertionError(
            f"row {t} (seq {bi}, head {h}) dim {j}: {int(got[bi, t, h, j])} keys attended, "
            f"{cnt[t, j]} in A(t) (|A(t)| = {size[t]}); {int(bad.sum())} mismatches")


@pytest.mark.parametrize("n_sink,window", [(0, 1), (0, 120), (0, 129), (8, 1), (8, 120), (8, 129),
                                           (64, 1), (64, 120), (64, 129)])
def test_mask_probe_ring_kernel(n_sink, window):
    """Resident key blocks (many sequences, G = 4, nine 64-row tiles per
    sequence, one workgroup walking them all)."""
    B, T, H, Hkv, d = 256, 520, 16, 4, 128
    q, k, v, a, b = probe_inputs(B, T, H, Hkv, d, torch.bfloat16, seed=window)
    o, _ = gl.hybrid_prefill(q, k, v, a, b, n_sink, window, flags=gl.BRANCH_SOFTMAX)
    torch.cuda.synchronize()
    check_counts(o, n_sink, window)


@pytest.mark.parametrize("G,dtype,d", [(1, torch.bfloat16, 128), (2, torch.bfloat16, 128),
                                       (4, torch.bfloat16, 128), (2, torch.float32, 64),
                                       (4, torch.float32, 128), (4, torch.bfloat16, 64)])
@pytest.mark.parametrize("n_sink,window", [(8, 56), (0, 129), (3, 200), (8, 888)])
def test_mask_probe_swa_kernel(G, dtype, d, n_sink, window):
    """The two-buffer softmax kernel with 1, 2 or 4 query heads per
    workgroup, both key-block sizes, short and long budgets (window 888 in
    bf16 at d = 128 takes the long-budget kernel)."""
    B, Hkv = 2, 2
    T = 1100 if window == 888 else 400
    q, k, v, a, b = probe_inputs(B, T, G * Hkv, Hkv, d, dtype, seed=G * 7 + window)
    o, _ = gl.hybrid_prefill(q, k, v, a, b, n_sink, window, flags=gl.BRANCH_SOFTMAX)
    torch.cuda.synchronize()
    check_counts(o, n_sink, window)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("n_sink,window,T", [(8, 888, 1500), (0, 256, 1300), (70, 300, 1111), (3, 1000, 700)])
def test_mask_probe_long_budget_kernel(G, n_sink, window, T):
    """The long-budget softmax kernel (bf16, d = 128, window >= 256): key
    blocks by direct loads into a four-slot ring, 8 waves of 32 query rows
    over G = 8, 4, 2 or 1 query heads per KV head (tiles of 32 to 256 rows),
    runs of up to 8 tiles per workgroup, two sink blocks (70 sinks), and a
    sequence shorter than the budget."""
    B, Hkv, d = 2, 2, 128
    q, k, v, a, b = probe_inputs(B, T, G * Hkv, Hkv, d, torch.bfloat16, seed=G * 11 + window)
    o, _ = gl.hybrid_prefill(q, k, v, a, b, n_sink, window, flags=gl.BRANCH_SOFTMAX)
    torch.cuda.synchronize()
    check_counts(o, n_sink, window)


@pytest.mark.parametrize("B,H,Hkv,T,n_sink,window", [(1, 32, 8, 4096, 8, 56), (1, 8, 2, 1000, 8, 56),
                                                     (2, 8, 2, 700, 0, 64), (1, 16, 4, 900, 8, 120),
                                                     (1, 8, 1, 333, 8, 1), (1, 4, 1, 650, 3, 130),
                                                     (1, 8, 2, 1000, 20, 56), (2, 8, 2, 700, 17, 200)])
def test_mask_probe_linked_tiles(B, H, Hkv, T, n_sink, window):
    """Both branches on a few-chain bf16 shape with G a multiple of 4.  With
    window <= 128 and n_sink <= 16 (the first five cases) the segmented scan
    runs the one-pass layer kernel per segment, whose softmax waves form the
    rows; with a longer window or more sinks the softmax tiles run inside the
    one-launch layer kernel and add onto the scan's rows.  q = 0 makes the
    linear branch exactly 0, so o is the softmax branch alone."""
    q, k, v, a, b = probe_inputs(B, T, H, Hkv, 128, torch.bfloat16, seed=T, gates=True)
    o, st = gl.hybrid_prefill(q, k, v, a, b, n_sink, window, flags=ALL | gl.WRITE_STATE)
    torch.cuda.synchronize()
    check_counts(o, n_sink, window)
    assert bool(torch.isfinite(st).all())


def slot_of(i, n_sink, window):
    return i if i < n_sink else n_sink + (i - n_sink) % window


@pytest.mark.parametrize("dtype,d,H,Hkv,n_sink,window,update", [
    (torch.bfloat16, 128, 4, 1, 8, 56, "gdn"),      # narrow passes, G = 4
    (torch.bfloat16, 128, 16, 1, 3, 61, "gla"),     # largest group
    (torch.bfloat16, 128, 8, 2, 0, 64, "gdn"),      # no sinks
    (torch.bfloat16, 128, 8, 2, 8, 120, "gdn"),     # budget 128: two passes
    (torch.float32, 64, 4, 2, 5, 40, "gdn"),        # fp32 cache
    (torch.bfloat16, 128, 8, 1, 8, 300, "gdn"),     # wide passes
    (torch.bfloat16, 128, 8, 1, 1, 1, "gdn")])      # one-token window
def test_mask_probe_decode(dtype, d, H, Hkv, n_sink, window, update):
    """Decode from position 0 to beyond two ring wraps with q = 0 and the
    value of each token one-hot at dimension slot mod (d - 1), while every
    cache slot starts as a poison value one-hot at dimension d - 1: the
    output counts then name exactly which slots the step attended (the
    current token's slot included), and a slot not yet written never shows."""
    B = 2
    N = n_sink + window
    steps = min(N + 2 * window + 5, 1400)
    w = Workload("probe", B=B, H=H, Hkv=Hkv, d=d, n_sink=n_sink, window=window, update=update,
                 pos0=0, steps=steps, dtype="bf16" if dtype == torch.bfloat16 else "f32")
    inp = make_decode_inputs(w, device=DEV, seed=window + H)
    poison = torch.nn.functional.one_hot(torch.tensor(d - 1), d).to(dtype).to(DEV)
    st = {x: inp[x].clone() for x in ("state", "a_cache", "b_cache", "pos")}
    st["k_cache"] = inp["k_cache"].clone()
    st["v_cache"] = poison.expand(B, Hkv, N, d).contiguous()
    q0 = torch.zeros(B, H, d, dtype=dtype, device=DEV)
    outs = []
    for t in range(steps):
        vt = torch.nn.functional.one_hot(torch.tensor(slot_of(t, n_sink, window) % (d - 1)), d)
        vt = vt.to(dtype).to(DEV).expand(B, Hkv, d).contiguous()
        o = gl.hybrid_decode(q0, inp["k"][t], vt, inp["a"][t], inp["b"][t], st["state"],
                             st["k_cache"], st["v_cache"], st["a_cache"], st["b_cache"], st["pos"],
                             n_sink, window, update=update)
        outs.append(o)
    torch.cuda.synchronize()
    got_all = torch.stack(outs).to(torch.float64).cpu().numpy()      # [steps, B, H, d]
    assert np.all(st["pos"].cpu().numpy() == steps)
    for t in range(steps):
        A = O.softmax_index_set(t, n_sink, window)
        slots = np.array([slot_of(int(i), n_sink, window) for i in A])
        want = np.bincount(slots % (d - 1), minlength=d)
        got = np.rint(got_all[t] * len(A)).astype(np.int64)
        bad = np.argwhere(got != want[None, None])
        assert bad.size == 0, (f"step t={t}: seq {bad[0][0]} head {bad[0][1]} dim {bad[0][2]}: "
                               f"{got[tuple(bad[0])]} slots attended, {want[bad[0][2]]} expected")


# ------------------------------------- branch flags on the one-launch path

@pytest.mark.parametrize("flags", [gl.BRANCH_SOFTMAX | gl.WRITE_STATE, gl.BRANCH_SOFTMAX,
                                   gl.BRANCH_LINEAR | gl.WRITE_STATE, ALL])
def test_branch_flags_few_chain_group4(flags):
    """A few-chain bf16 shape with G a multiple of 4, where both branches run
    as one launch: each branch selection must give the oracle's output (the
    softmax branch alone must not be added onto rows the scan never wrote)."""
    w = Workload("fc", B=1, H=8, Hkv=2, d=128, n_sink=8, window=56, T=520, sigma=0.5)
    inp = {x: t.to(DEV) for x, t in make_prefill_inputs(w, seed=17).items()}
    o = torch.full((w.B, w.T, w.H, w.d), float("nan"), dtype=torch.bfloat16, device=DEV)
    o, st = gl.hybrid_prefill(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], w.n_sink, w.window,
                              flags=flags, o=o)
    torch.cuda.synchronize()
    ref, S = O.hybrid_prefill(*(f64(inp[x]) for x in ("q", "k", "v", "a", "b")), w.n_sink,
                              w.window, flags=flags)
    got = f64(o)
    assert np.all(np.isfinite(got)), "rows left unwritten"
    err = np.max(np.abs(got - ref))
    assert err <= 2e-2 * np.max(np.abs(ref)), err
    if flags & gl.WRITE_STATE:
        err = np.max(np.abs(f64(st) - S))
        assert err <= 2e-2 * np.max(np.abs(S)), err


# ----------------------------------------------- decode over 1000 steps

def test_decode_b256_1000_steps_sampled():
    """The decode workload (B = 256, 32 query / 8 KV heads, cache 8 + 56 at
    t = 4096..5095) over all 1000 steps, every step's output of 64 (sequence,
    head) chains (two whole sequences) against the oracle's stepper, and
    their state and caches after the last step."""
    w = WORKLOADS["decode_b256"]
    inp = make_decode_inputs(w, device=DEV)
    keys = ("state", "k_cache", "v_cache", "a_cache", "b_cache", "pos")
    st = {x: inp[x].clone() for x in keys}
    bsel = [3, 200]
    ref = {x: f64(st[x][bsel]) for x in keys if x != "pos"}
    ref["pos"] = st["pos"][bsel].cpu().numpy().astype(np.int64)
    outs = []
    for s in range(w.steps):
        o = gl.hybrid_decode(inp["q"][s], inp["k"][s], inp["v"][s], inp["a"][s], inp["b"][s],
                             st["state"], st["k_cache"], st["v_cache"], st["a_cache"], st["b_cache"],
                             st["pos"], w.n_sink, w.window)
        outs.append(o[bsel].clone())
    torch.cuda.synchronize()
    got = torch.stack(outs).to(torch.float64).cpu().numpy()
    step_in = {x: f64(inp[x][:, bsel]) for x in ("q", "k", "v", "a", "b")}
    worst = 0.0
    for s in range(w.steps):
        ro, ref["state"], ref["k_cache"], ref["v_cache"], ref["a_cache"], ref["b_cache"], ref["pos"] = \
            O.decode_step(*(step_in[x][s] for x in ("q", "k", "v", "a", "b")), ref["state"],
                          ref["k_cache"], ref["v_cache"], ref["a_cache"], ref["b_cache"], ref["pos"],
                          w.n_sink, w.window)
        err = np.max(np.abs(got[s] - ro))
        bound = 2e-2 * np.max(np.abs(ro))
        assert err <= bound, f"step {s}: max abs err {err:.3e} > {bound:.3e}"
        worst = max(worst, err / np.max(np.abs(ro)))
    S = f64(st["state"][bsel])
    assert np.max(np.abs(S - ref["state"])) <= 2e-2 * np.max(np.abs(ref["state"]))
    assert np.array_equal(f64(st["k_cache"][bsel]), ref["k_cache"])
    assert np.array_equal(f64(st["v_cache"][bsel]), ref["v_cache"])
    assert np.array_equal(f64(st["a_cache"][bsel]), ref["a_cache"])
    assert np.array_equal(f64(st["b_cache"][bsel]), ref["b_cache"])
    assert np.all(st["pos"].cpu().numpy() == w.pos0 + w.steps)
    print(f"worst relative error over 1000 steps: {worst:.3e}")


@pytest.mark.parametrize("B,H,Hkv,T,n_sink,window", [(32, 8, 2, 300, 8, 56), (16, 16, 4, 517, 8, 120),
                                                     (32, 8, 2, 400, 16, 128), (32, 8, 8, 250, 0, 1),
                                                     (64, 4, 1, 129, 3, 64), (32, 8, 2, 700, 0, 100),
                                                     (16, 16, 2, 137, 8, 120), (32, 8, 2, 333, 16, 63),
                                                     (32, 8, 2, 270, 5, 65)])
def test_mask_probe_one_pass_layer(B, H, Hkv, T, n_sink, window):
    """Both branches on many chains (B*H >= 128, window <= 128, n_sink <= 16):
    the layer runs as the one-pass kernel whose softmax rows read keys from a
    ring of three chunks; q = 0 makes the linear branch exactly 0."""
    q, k, v, a, b = probe_inputs(B, T, H, Hkv, 128, torch.bfloat16, seed=T + window, gates=True)
    o, st = gl.hybrid_prefill(q, k, v, a, b, n_sink, window, flags=ALL | gl.WRITE_STATE)
    torch.cuda.synchronize()
    check_counts(o, n_sink, window)
    assert bool(torch.isfinite(st).all())
