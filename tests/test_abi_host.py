"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function declared in
include/gdn_hybrid.h, and reject invalid arguments on the host with the
documented codes before anything is launched.  Only calls that fail
validation (or pure queries) are made here, so no GPU is touched.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn_hybrid.h")

from swa_chunked_gated_amd import _lib  # noqa: E402

OK, EINVAL, EUNSUP, EWS, ELAUNCH = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
DELTA, GLA = 0, 1
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ("gdn_hybrid_prefill", "gdn_hybrid_decode", "shortconv_qkv", "shortconv_qkv_decode",
              "shortconv_history_from_prefill",
              "gdn_hybrid_cache_from_prefill", "gdn_hybrid_prefill_workspace"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert names
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_version_and_strerror(lib):
    assert lib.gdn_hybrid_version() >= 10000
    for c in (OK, EINVAL, EUNSUP, EWS, ELAUNCH):
        assert lib.gdn_hybrid_strerror(c)
    assert lib.gdn_hybrid_strerror(123) == b"unknown error"


def ws(lib, *args):
    n = ctypes.c_size_t(99)
    rc = lib.gdn_hybrid_prefill_workspace(*args, ctypes.byref(n))
    return rc, n.value


def test_workspace_query(lib):
    # gated delta rule, per (sequence, head, 64-token chunk of the linear
    # stream): with few chains (B*H*(d/64) < 256) the full preparation,
    # Tm diag(b), -Wm, K^T 2^{g_C-g} and A; else Tm diag(b); plus 128 fp32
    # gate values
    def gdn_bytes(B, T, H, d, elt, n=64):
        nch = -(-(T - n) // 64)
        full = elt == 2 and B * H * (2 if d == 128 else 1) < 256     # bf16, few chains
        if full:    # -Wm, K^T, A in bf16; (TB V)^T in fp32; gates; ready and done flags
            per = (64 * d + d * 64 + 64 * 64) * elt + d * 64 * 4 + 512 + 8 + d // 16 * 8
        else:       # TB; gates
            per = 64 * 64 * elt + 512
        return B * H * nch * per
    # few chains, bf16 d = 128, both branches, window <= 128, <= 16 sinks:
    # the segmented scan's light preparation (TB, gates), then per (segment,
    # chain) M bf16, N and the incoming state fp32, [128][128] each (the
    # states with one spare segment); 32 chains over 63 chunks: 8 segments
    light = 2016 * (64 * 64 * 2 + 512)
    seg = 8 * 32 * 128 * 128 * (2 + 4 + 4) + 32 * 128 * 128 * 4
    assert ws(lib, 1, 4096, 32, 8, 128, 128, 8, 56, BF16, DELTA, 3) == (OK, light + seg)
    # the same shape, linear branch and state only: the one-launch path's
    # full preparation
    assert ws(lib, 1, 4096, 32, 8, 128, 128, 8, 56, BF16, DELTA, 5) == (OK, gdn_bytes(1, 4096, 32, 128, 2))
    assert gdn_bytes(1, 4096, 32, 128, 2) == 2016 * 74312
    assert ws(lib, 2, 300, 4, 2, 64, 64, 8, 56, F32, DELTA, 5) == (OK, gdn_bytes(2, 300, 4, 64, 4))
    assert ws(lib, 8, 4096, 32, 8, 128, 128, 8, 120, BF16, DELTA, 5) == (OK, gdn_bytes(8, 4096, 32, 128, 2, 128))
    nch = (4096 - 64 + 63) // 64
    assert ws(lib, 1, 4096, 32, 8, 128, 128, 8, 56, BF16, DELTA, 4)[1] > 0          # state only
    assert ws(lib, 1, 4096, 32, 8, 128, 128, 8, 56, BF16, DELTA, 2) == (OK, 0)     # softmax only
    # GLA: Q 2^G [64][d], (K 2^{G_C-G})^T [d][64], A [64][64] and 2^{G_C} [d] fp32
    assert ws(lib, 1, 4096, 32, 8, 128, 128, 8, 56, BF16, GLA, 3) == (OK, 32 * nch * (2 * 64 * 128 * 2 + 64 * 64 * 2 + 128 * 4))
    assert ws(lib, 1, 64, 32, 8, 128, 128, 8, 56, BF16, DELTA, 3) == (OK, 0)       # T <= budget
    assert ws(lib, 1, 65, 32, 8, 128, 128, 8, 56, BF16, DELTA, 3)[1] > 0
    assert ws(lib, 1, 4096, 32, 7, 128, 128, 8, 56, BF16, DELTA, 3)[0] == EINVAL   # H % Hkv
    assert ws(lib, 1, 4096, 32, 8, 96, 96, 8, 56, BF16, DELTA, 3)[0] == EINVAL     # d
    assert ws(lib, 1, 4096, 32, 8, 128, 64, 8, 56, BF16, DELTA, 3)[0] == EINVAL    # dk != dv
    assert ws(lib, 1, 4096, 32, 8, 128, 128, 8, 0, BF16, DELTA, 3)[0] == EINVAL    # window
    assert ws(lib, 1, 4096, 32, 8, 128, 128, -1, 56, BF16, DELTA, 3)[0] == EINVAL  # n_sink
    assert ws(lib, 1, 4096, 32, 8, 128, 128, 8, 56, 2, DELTA, 3)[0] == EINVAL      # dtype
    assert ws(lib, 1, 4096, 32, 8, 128, 128, 8, 56, BF16, 3, 3)[0] == EINVAL       # update
    # the diagonal-gate delta rule: the per-channel-gate tiles plus TB and Wm
    rc, n = ws(lib, 1, 4096, 32, 8, 128, 128, 8, 56, BF16, 2, 3)
    nch = (4096 - 64 + 63) // 64
    assert rc == OK and n >= 32 * nch * ((3 * 64 * 128 + 2 * 64 * 64) * 2 + 128 * 4)
    assert ws(lib, 1, 4096, 32, 8, 128, 128, 8, 56, BF16, DELTA, 0)[0] == EINVAL   # flags
    assert ws(lib, 1, 4096, 32, 8, 128, 128, 8, 56, BF16, DELTA, 8)[0] == EINVAL
    assert ws(lib, 1, 4096, 32, 8, 128, 128, 8, 56, BF16, DELTA, 16)[0] == EINVAL
    assert lib.gdn_hybrid_prefill_workspace(1, 64, 2, 2, 64, 64, 8, 56, 0, 0, 3, None) == EINVAL


def prefill(lib, q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, o=FAKE, st=FAKE, B=1, T=64, H=2,
            Hkv=2, dk=64, dv=64, ns=8, w=56, dt=BF16, up=DELTA, flags=3):
    return lib.gdn_hybrid_prefill(q, k, v, a, b, o, st, B, T, H, Hkv, dk, dv, ns, w, dt, up,
                                  flags, None, 0, None)


def test_prefill_validation(lib):
    assert prefill(lib, q=None) == EINVAL
    assert prefill(lib, k=None) == EINVAL
    assert prefill(lib, v=None) == EINVAL
    assert prefill(lib, o=None) == EINVAL
    assert prefill(lib, a=None) == EINVAL                       # linear branch needs a
    assert prefill(lib, b=None) == EINVAL                       # GDN needs b
    assert prefill(lib, b=None, up=2) == EINVAL                 # so does the diagonal-gate delta rule
    assert prefill(lib, st=None, flags=7) == EINVAL             # state requested
    assert prefill(lib, B=0) == EINVAL
    assert prefill(lib, T=-1) == EINVAL
    assert prefill(lib, H=3, Hkv=2) == EINVAL
    assert prefill(lib, dk=128, dv=64) == EINVAL
    assert prefill(lib, dk=32, dv=32) == EINVAL
    assert prefill(lib, w=0) == EINVAL
    assert prefill(lib, flags=0) == EINVAL
    assert prefill(lib, flags=8) == EINVAL                       # accumulate alone
    assert prefill(lib, flags=16) == EINVAL
    assert prefill(lib, dt=F32, dk=128, dv=128) == EUNSUP      # fp32 linear branch at d=128
    assert prefill(lib, dt=F32, dk=128, dv=128, flags=4) == EUNSUP
    # fp32 softmax-only at d=128 is supported, so only the missing pointer fails here
    assert prefill(lib, dt=F32, dk=128, dv=128, flags=2, q=None) == EINVAL
    assert prefill(lib, B=1 << 16, T=1 << 16) == EINVAL          # B*T overflows int


def test_two_phase_flags(lib):
    # both phases at once, unknown bits, or no branch: invalid
    assert prefill(lib, flags=3 | 16 | 32) == EINVAL
    assert prefill(lib, flags=3 | 64) == EINVAL
    assert prefill(lib, flags=16) == EINVAL
    assert ws(lib, 1, 4096, 32, 8, 128, 128, 8, 56, BF16, DELTA, 3 | 16 | 32)[0] == EINVAL
    assert ws(lib, 1, 4096, 32, 8, 128, 128, 8, 56, BF16, DELTA, 3 | 16)[0] == OK
    assert ws(lib, 1, 4096, 32, 8, 128, 128, 8, 56, BF16, DELTA, 3 | 32)[0] == OK
    # no stream chunk (T = n_sink + window): nothing to prepare
    assert prefill(lib, flags=3 | 16) == EUNSUP
    assert prefill(lib, flags=3 | 32) == EUNSUP
    # softmax only: no recurrence to prepare
    assert prefill(lib, T=200, flags=2 | 16) == EUNSUP
    # bf16, 2 chains: the one-launch path, whose preparation runs inside it
    big = ctypes.c_void_p(0x100000)
    for f in (3 | 16, 3 | 32):
        assert lib.gdn_hybrid_prefill(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 200, 2, 2, 64, 64,
                                      8, 56, BF16, DELTA, f, big, 1 << 30, None) == EUNSUP


def test_prefill_workspace_checks(lib):
    # T = 200 > budget: the gated delta rule needs its chunk workspace
    assert prefill(lib, T=200) == EWS
    big = ctypes.c_void_p(FAKE.value)
    assert lib.gdn_hybrid_prefill(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 200, 2, 2, 64, 64,
                                  8, 56, BF16, DELTA, 3, big, 16, None) == EWS    # too small
    assert lib.gdn_hybrid_prefill(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 200, 2, 2, 64, 64,
                                  8, 56, BF16, DELTA, 3, ctypes.c_void_p(FAKE.value + 8), 1 << 30,
                                  None) == EINVAL                                  # misaligned
    assert prefill(lib, T=200, up=GLA, b=None) == EWS
    # a softmax-only call needs none: with q missing it fails on q, not on the workspace
    assert prefill(lib, T=200, flags=2, q=None) == EINVAL


def test_misaligned_tensors_are_rejected(lib):
    # every tensor pointer must be 16-byte aligned; the check runs before any launch
    odd = ctypes.c_void_p(FAKE.value + 8)
    for name in ("q", "k", "v", "a", "b", "o", "st"):
        assert prefill(lib, T=0, flags=7, **{name: odd}) == EINVAL, name
    for name in ("q", "k", "v", "a", "b", "st", "kc", "vc", "ac", "bc", "pos", "o"):
        assert decode(lib, **{name: odd}) == EINVAL, name
    for name in ("q", "k", "v", "wq", "wk", "wv", "qo", "ko", "vo"):
        assert shortconv(lib, **{name: odd}) == EINVAL, name


def test_prefill_zero_length_is_a_noop(lib):
    # T = 0 with no state requested returns before any launch
    assert prefill(lib, T=0) == OK


def decode(lib, q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, st=FAKE, kc=FAKE, vc=FAKE, ac=FAKE,
           bc=FAKE, pos=FAKE, o=FAKE, B=2, H=4, Hkv=2, dk=128, dv=128, ns=8, w=56, dt=BF16,
           up=DELTA, flags=3):
    return lib.gdn_hybrid_decode(q, k, v, a, b, st, kc, vc, ac, bc, pos, o, B, H, Hkv, dk, dv,
                                 ns, w, dt, up, flags, None)


def test_decode_validation(lib):
    for name in ("q", "k", "v", "a", "st", "kc", "vc", "ac", "pos", "o"):
        assert decode(lib, **{name: None}) == EINVAL, name
    assert decode(lib, b=None) == EINVAL
    assert decode(lib, bc=None) == EINVAL
    assert decode(lib, flags=0) == EINVAL
    assert decode(lib, flags=4) == EINVAL                        # no state output in decode
    assert decode(lib, H=5, Hkv=2) == EINVAL
    assert decode(lib, H=34, Hkv=2) == EUNSUP                    # G = 17 > 16
    assert decode(lib, H=16, Hkv=1, w=1000) == EUNSUP            # G * N too large
    assert decode(lib, w=0) == EINVAL


def shortconv(lib, q=FAKE, k=FAKE, v=FAKE, wq=FAKE, wk=FAKE, wv=FAKE, qo=FAKE, ko=FAKE, vo=FAKE,
              B=1, T=16, H=2, Hkv=1, d=64, ks=8, theta=1e6, pos0=0, flags=3, dt=BF16):
    return lib.shortconv_qkv(q, k, v, wq, wk, wv, qo, ko, vo, B, T, H, Hkv, d, ks, theta, pos0,
                             flags, dt, None)


def test_shortconv_validation(lib):
    for name in ("q", "k", "v", "wq", "wk", "wv", "qo", "ko", "vo"):
        assert shortconv(lib, **{name: None}) == EINVAL, name
    assert shortconv(lib, ks=0) == EUNSUP
    assert shortconv(lib, ks=9) == EUNSUP
    assert shortconv(lib, d=96) == EINVAL
    assert shortconv(lib, theta=0.0) == EINVAL
    assert shortconv(lib, theta=0.0, flags=2, T=0) == OK           # no RoPE: theta unused
    assert shortconv(lib, flags=4) == EINVAL
    assert shortconv(lib, pos0=-1) == EINVAL
    assert shortconv(lib, T=0) == OK
    assert shortconv(lib, T=65535 * 64 + 1, H=1, Hkv=1) == EUNSUP   # 64-token tiles: a grid dimension
    assert shortconv(lib, B=65536, T=1, H=1, Hkv=1) == EUNSUP


def test_cache_fill_validation(lib):
    f = lib.gdn_hybrid_cache_from_prefill
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1, 8, 2, 2, 64, 64, 8, 56, BF16, DELTA, None) == EINVAL
    assert f(FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 2, 64, 64, 8, 56, BF16, DELTA, None) == EINVAL
    assert f(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 2, 64, 64, 8, 56, BF16, DELTA, None) == EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 3, 2, 64, 64, 8, 56, BF16, DELTA, None) == EINVAL


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError, match="not built"):
        _lib.load()


def test_shortconv_decode_validation(lib):
    f = lib.shortconv_qkv_decode

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, wq=FAKE, wk=FAKE, wv=FAKE, hq=FAKE, hk=FAKE, hv=FAKE,
                 pos=FAKE, qo=FAKE, ko=FAKE, vo=FAKE, B=1, H=4, Hkv=2, d=64, ks=8, theta=1e6,
                 pos0=0, flags=3, dt=BF16)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["wq"], a["wk"], a["wv"], a["hq"], a["hk"], a["hv"],
                 a["pos"], a["qo"], a["ko"], a["vo"], a["B"], a["H"], a["Hkv"], a["d"], a["ks"],
                 a["theta"], a["pos0"], a["flags"], a["dt"], None)

    for name in ("q", "k", "v", "wq", "wk", "wv", "pos", "qo", "ko", "vo", "hq", "hk", "hv"):
        assert call(**{name: None}) == EINVAL, name
    assert call(ks=0) == EUNSUP
    assert call(ks=9) == EUNSUP
    assert call(d=96) == EINVAL
    assert call(H=3) == EINVAL
    assert call(theta=0.0) == EINVAL
    assert call(flags=4) == EINVAL
    assert call(pos0=-1) == EINVAL
    assert call(B=65536) == EUNSUP
    assert call(q=ctypes.c_void_p(0x1004)) == EINVAL                # not 16-byte aligned


def test_shortconv_history_validation(lib):
    f = lib.shortconv_history_from_prefill

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, hq=FAKE, hk=FAKE, hv=FAKE, B=1, T=16, H=4, Hkv=2, d=64,
                 ks=8, theta=1e6, pos0=0, flags=3, dt=BF16)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["hq"], a["hk"], a["hv"], a["B"], a["T"], a["H"],
                 a["Hkv"], a["d"], a["ks"], a["theta"], a["pos0"], a["flags"], a["dt"], None)

    assert call(ks=1, hq=None, hk=None, hv=None) == OK             # no history: nothing launched
    assert call(ks=9) == EUNSUP
    for name in ("hq", "hk", "hv", "q", "k", "v"):
        assert call(**{name: None}) == EINVAL, name
    assert call(T=-1) == EINVAL
    assert call(theta=-1.0) == EINVAL
    assert call(pos0=-1) == EINVAL
    assert call(B=65536) == EUNSUP
    assert call(hq=ctypes.c_void_p(0x1008)) == EINVAL


def test_weighted_calls_reject_non_finite_weights(lib):
    import math
    for wl, ws in ((math.nan, 1.0), (1.0, math.inf)):
        assert lib.gdn_hybrid_prefill_weighted(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 8, 2, 2, 64,
                                               64, 8, 56, BF16, DELTA, 3, wl, ws, None, 0, None) == EINVAL
        assert lib.gdn_hybrid_decode_weighted(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                              FAKE, FAKE, 1, 2, 2, 64, 64, 8, 56, BF16, DELTA, 3, wl, ws,
                                              None) == EINVAL


def test_test_fault_setting_validation(lib):
    assert lib.gdn_hybrid_set_test_faults(-1, 100) == EINVAL
    assert lib.gdn_hybrid_set_test_faults(4, 100) == EINVAL
    assert lib.gdn_hybrid_set_test_faults(0, 0) == EINVAL
    assert lib.gdn_hybrid_set_test_faults(0, 1000001) == EINVAL
    assert lib.gdn_hybrid_set_test_faults(3, 50) == OK
    assert lib.gdn_hybrid_set_test_faults(0, 100000) == OK   # normal operation restored


def test_noalloc_prefill_validation(lib):
    """Rejected on the host before the device array is looked up."""
    cap = lib.gdn_hybrid_noalloc_max_workspace()
    assert cap == 256 << 20
    p = [FAKE] * 7
    # workspace beyond the array: B=64, H=32, T=8192 (light preparation, ~2.2 GB)
    ws = ctypes.c_size_t(0)
    assert lib.gdn_hybrid_prefill_workspace(64, 8192, 32, 8, 128, 128, 8, 56, BF16, DELTA, 3,
                                            ctypes.byref(ws)) == OK
    assert ws.value > cap
    assert lib.gdn_hybrid_prefill_noalloc(*p, 64, 8192, 32, 8, 128, 128, 8, 56, BF16, DELTA, 3,
                                          None) == EWS
    # the usual argument checks
    assert lib.gdn_hybrid_prefill_noalloc(*p, 1, 100, 3, 2, 128, 128, 8, 56, BF16, DELTA, 3,
                                          None) == EINVAL          # H % Hkv != 0
    assert lib.gdn_hybrid_prefill_noalloc(*p, 1, 100, 4, 2, 128, 128, 8, 56, BF16, DELTA, 0,
                                          None) == EINVAL          # no flag
    assert lib.gdn_hybrid_prefill_noalloc(None, *p[1:], 1, 100, 4, 2, 128, 128, 8, 56, BF16, DELTA,
                                          3, None) == EINVAL       # q NULL
    assert lib.gdn_hybrid_prefill_noalloc(*p, 1, 100, 4, 2, 128, 128, 8, 56, F32, DELTA, 1,
                                          None) == EUNSUP          # fp32 linear branch at d = 128


# ------------------------------------------------------------- backward pass

def bws(lib, B=1, T=300, H=4, Hkv=1, d=128, n_sink=8, window=56, dtype=BF16, update=DELTA):
    n = ctypes.c_size_t(99)
    rc = lib.gdn_hybrid_prefill_backward_workspace(B, T, H, Hkv, d, d, n_sink, window, dtype,
                                                   update, ctypes.byref(n))
    return rc, n.value


def bwd(lib, B=1, T=300, H=4, Hkv=1, d=128, n_sink=8, window=56, dtype=BF16, update=DELTA,
        ptrs=None, dstate=None, ws_ptr=None, ws_bytes=1 << 40, w=(1.0, 1.0)):
    p = ptrs if ptrs is not None else [FAKE] * 11
    q, k, v, a, b, do, dq, dk, dv, da, db = p
    return lib.gdn_hybrid_prefill_backward(q, k, v, a, b, do, dstate, dq, dk, dv, da, db, B, T, H,
                                           Hkv, d, d, n_sink, window, dtype, update, w[0], w[1],
                                           ws_ptr if ws_ptr is not None else ctypes.c_void_p(0x100000),
                                           ws_bytes, None)


def test_backward_workspace_query(lib):
    rc, n = bws(lib)
    assert rc == OK
    # light preparation (TB bf16 + 128 gate floats), Tm (bf16 64 x 64), the
    # states entering and the gradients leaving each chunk (bf16 128 x 128),
    # per-row softmax statistics (2 floats), sink partials (2 x n_sink x 128
    # floats per 64-row query tile), each part 256-byte aligned
    items = 1 * 4 * 4                      # T = 300, budget 64: 4 chunks
    up = lambda x: (x + 255) // 256 * 256
    want = up(items * (64 * 64 * 2 + 512)) + up(items * 64 * 64 * 2) + 2 * up(items * 128 * 128 * 2) \
        + up(4 * 300 * 2 * 4) + 2 * up(4 * 5 * 8 * 128 * 4)
    assert n == want
    assert bws(lib, dtype=F32)[0] == EUNSUP
    assert bws(lib, d=64)[0] == EUNSUP
    assert bws(lib, update=GLA)[0] == EUNSUP
    assert bws(lib, update=2)[0] == EUNSUP
    assert bws(lib, H=4, Hkv=3)[0] == EINVAL
    assert bws(lib, window=0)[0] == EINVAL
    assert lib.gdn_hybrid_prefill_backward_workspace(1, 300, 4, 1, 128, 128, 8, 56, BF16, DELTA, None) == EINVAL


def test_backward_validation(lib):
    assert bwd(lib, dtype=F32) == EUNSUP
    assert bwd(lib, d=64) == EUNSUP
    for i in range(11):
        p = [FAKE] * 11
        p[i] = None
        assert bwd(lib, ptrs=p) == EINVAL, i
    p = [FAKE] * 11
    p[3] = ctypes.c_void_p(0x1008)          # a misaligned
    assert bwd(lib, ptrs=p) == EINVAL
    assert bwd(lib, dstate=ctypes.c_void_p(0x1004)) == EINVAL
    assert bwd(lib, w=(float("nan"), 1.0)) == EINVAL
    assert bwd(lib, ws_bytes=16) == EWS
    assert bwd(lib, ws_ptr=ctypes.c_void_p(0x100008)) == EINVAL    # workspace not 256-aligned
