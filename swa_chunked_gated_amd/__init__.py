"""MI355X (gfx950) hybrid attention layer: gated delta rule over the tokens
outside a fixed budget + softmax over sinks and a sliding window, summed.

This module only marshals torch tensors into the C ABI of
``libgdn_hybrid.so`` (include/gdn_hybrid.h); every step of the layer runs in
the library's HIP kernels on the caller's current HIP stream.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import GdnError  # noqa: F401

BRANCH_LINEAR = 1
BRANCH_SOFTMAX = 2
WRITE_STATE = 4
ACCUMULATE = 8
# two-phase prefill: the state-independent chunk preparation alone, then the
# rest from a workspace that holds it (same arguments, k, a, b unchanged)
PREPARE_ONLY = 16
PREPARED = 32
ROPE = 1
L2NORM = 2

_DTYPES = {torch.float32: 0, torch.bfloat16: 1}
# "dgd": the delta rule with a diagonal (per-channel) gate
_UPDATES = {"gdn": 0, "gla": 1, "dgd": 2}

__all__ = [
    "hybrid_prefill", "hybrid_decode", "cache_from_prefill", "shortconv_qkv",
    "prefill_workspace_bytes", "hybrid_prefill_backward", "prefill_backward_workspace_bytes",
    "version", "GdnError", "BRANCH_LINEAR", "BRANCH_SOFTMAX", "WRITE_STATE", "ACCUMULATE",
    "PREPARE_ONLY", "PREPARED", "ROPE", "L2NORM",
]


def version() -> int:
    return _lib.load().gdn_hybrid_version()


def set_test_faults(faults: int = 0, wait_us: int = 100000) -> None:
    """Test-only: inject faults into the one-launch prefill's flag hand-offs
    (bit 0: no chunk-ready flags, bit 1: no row-done flags) with each bounded
    wait limited to ``wait_us``; the affected rows and states come out NaN.
    ``set_test_faults()`` restores normal operation."""
    _lib.check("gdn_hybrid_set_test_faults", _lib.load().gdn_hybrid_set_test_faults(faults, wait_us))


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _io_dtype(*ts):
    dt = ts[0].dtype
    for t in ts:
        if t.dtype != dt:
            raise ValueError("q, k, v (and outputs/caches) must share one dtype")
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    return _DTYPES[dt]


def _f32(*ts):
    for t in ts:
        if t is not None and t.dtype != torch.float32:
            raise ValueError("gates, states and conv weights must be float32")


def prefill_workspace_bytes(B: int, T: int, H: int, Hkv: int, d: int, n_sink: int, window: int,
                            dtype, update: str = "gdn",
                            flags: int = BRANCH_LINEAR | BRANCH_SOFTMAX) -> int:
    """Device workspace (bytes) ``hybrid_prefill`` needs for these arguments."""
    dt = _DTYPES[dtype]
    n = ctypes.c_size_t(0)
    rc = _lib.load().gdn_hybrid_prefill_workspace(B, T, H, Hkv, d, d, n_sink, window, dt,
                                                  _UPDATES[update], flags, ctypes.byref(n))
    _lib.check("gdn_hybrid_prefill_workspace", rc)
    return n.value


def hybrid_prefill(q, k, v, a, b, n_sink: int, window: int, update: str = "gdn",
                   flags: int = BRANCH_LINEAR | BRANCH_SOFTMAX, o=None, state_out=None,
                   workspace=None, weights=None):
    """Layer output for whole sequences starting at position 0.

    ``weights=(w_lin, w_swa)`` gives o = w_lin o_lin + w_swa o_swa (the
    weighted entry point); omitted, the plain sum.

    q [B,T,H,d], k/v [B,T,Hkv,d] (fp32 or bf16); a [B,T,H] (GLA: [B,T,H,d])
    and b [B,T,H] fp32.  Returns (o [B,T,H,d], state [B,H,d,d] fp32 or None).
    With ACCUMULATE in flags, ``o`` must be given and receives o += branches.
    ``workspace``: a uint8 device tensor of at least
    ``prefill_workspace_bytes(...)`` bytes; allocated here when omitted.
    PREPARE_ONLY fills the workspace with the chunk preparation alone;
    PREPARED (with that workspace) runs the rest of the same call.
    """
    if flags & ACCUMULATE and o is None:
        raise ValueError("ACCUMULATE needs an initialised output tensor o")
    if flags & PREPARED and workspace is None:
        raise ValueError("PREPARED needs the workspace a PREPARE_ONLY call filled")
    B, T, H, dk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    dt = _io_dtype(q, k, v)
    _f32(a, b)
    if o is None and flags & (BRANCH_LINEAR | BRANCH_SOFTMAX):
        o = torch.empty(B, T, H, dv, dtype=q.dtype, device=q.device)
    if state_out is None and flags & WRITE_STATE:
        state_out = torch.empty(B, H, dk, dv, dtype=torch.float32, device=q.device)
    if o is not None:
        _io_dtype(q, o)
    _f32(state_out)
    lib = _lib.load()
    need = ctypes.c_size_t(0)
    rc = lib.gdn_hybrid_prefill_workspace(B, T, H, Hkv, dk, dv, n_sink, window, dt,
                                          _UPDATES[update], flags, ctypes.byref(need))
    _lib.check("gdn_hybrid_prefill_workspace", rc)
    if need.value > 0 and workspace is None:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if weights is None:
        rc = lib.gdn_hybrid_prefill(_p(q), _p(k), _p(v), _p(a), _p(b), _p(o), _p(state_out),
                                    B, T, H, Hkv, dk, dv, n_sink, window, dt, _UPDATES[update],
                                    flags, _p(workspace), ws_bytes, _stream(q))
        _lib.check("gdn_hybrid_prefill", rc)
    else:
        rc = lib.gdn_hybrid_prefill_weighted(_p(q), _p(k), _p(v), _p(a), _p(b), _p(o),
                                             _p(state_out), B, T, H, Hkv, dk, dv, n_sink, window,
                                             dt, _UPDATES[update], flags, float(weights[0]),
                                             float(weights[1]), _p(workspace), ws_bytes, _stream(q))
        _lib.check("gdn_hybrid_prefill_weighted", rc)
    return o, state_out


def hybrid_prefill_noalloc(q, k, v, a, b, n_sink: int, window: int, update: str = "gdn",
                           flags: int = BRANCH_LINEAR | BRANCH_SOFTMAX, o=None, state_out=None):
    """``hybrid_prefill`` through the entry point that allocates nothing: its
    chunk workspace is the library's per-GPU array (see
    ``noalloc_max_workspace``); calls that may overlap on one GPU race.
    Outputs are allocated here with torch when not given."""
    if flags & ACCUMULATE and o is None:
        raise ValueError("ACCUMULATE needs an initialised output tensor o")
    B, T, H, dk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    dt = _io_dtype(q, k, v)
    _f32(a, b)
    if o is None and flags & (BRANCH_LINEAR | BRANCH_SOFTMAX):
        o = torch.empty(B, T, H, dv, dtype=q.dtype, device=q.device)
    if state_out is None and flags & WRITE_STATE:
        state_out = torch.empty(B, H, dk, dv, dtype=torch.float32, device=q.device)
    if o is not None:
        _io_dtype(q, o)
    _f32(state_out)
    rc = _lib.load().gdn_hybrid_prefill_noalloc(_p(q), _p(k), _p(v), _p(a), _p(b), _p(o),
                                                _p(state_out), B, T, H, Hkv, dk, dv, n_sink,
                                                window, dt, _UPDATES[update], flags, _stream(q))
    _lib.check("gdn_hybrid_prefill_noalloc", rc)
    return o, state_out


def noalloc_max_workspace() -> int:
    """Bytes of the per-GPU workspace array of ``hybrid_prefill_noalloc``."""
    return int(_lib.load().gdn_hybrid_noalloc_max_workspace())


def prefill_backward_workspace_bytes(B: int, T: int, H: int, Hkv: int, d: int, n_sink: int,
                                     window: int) -> int:
    """Device workspace (bytes) ``hybrid_prefill_backward`` needs."""
    n = ctypes.c_size_t(0)
    rc = _lib.load().gdn_hybrid_prefill_backward_workspace(B, T, H, Hkv, d, d, n_sink, window,
                                                           _DTYPES[torch.bfloat16],
                                                           _UPDATES["gdn"], ctypes.byref(n))
    _lib.check("gdn_hybrid_prefill_backward_workspace", rc)
    return n.value


def hybrid_prefill_backward(q, k, v, a, b, n_sink: int, window: int, d_o, d_state=None,
                            weights=(1.0, 1.0), workspace=None):
    """Gradients of sum(d_o * o) + sum(d_state * S_final) for the prefill
    o = w_lin o_lin + w_swa o_swa (gated delta rule, bf16, d = 128).

    q, d_o [B,T,H,d] and k, v [B,T,Hkv,d] bf16; a, b [B,T,H] fp32; d_state
    [B,H,d,d] fp32 or None.  Returns fp32 (dq, dk, dv, da, db) with the
    shapes of q, k, v, a, b.
    """
    B, T, H, d = q.shape
    Hkv = k.shape[2]
    dt = _io_dtype(q, k, v, d_o)
    _f32(a, b, d_state)
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    dq = torch.empty(B, T, H, d, **f32)
    dk = torch.empty(B, T, Hkv, d, **f32)
    dv = torch.empty(B, T, Hkv, d, **f32)
    da = torch.empty(B, T, H, **f32)
    db = torch.empty(B, T, H, **f32)
    lib = _lib.load()
    need = ctypes.c_size_t(0)
    rc = lib.gdn_hybrid_prefill_backward_workspace(B, T, H, Hkv, d, d, n_sink, window, dt,
                                                   _UPDATES["gdn"], ctypes.byref(need))
    _lib.check("gdn_hybrid_prefill_backward_workspace", rc)
    if workspace is None:
        workspace = torch.empty(max(need.value, 256), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = lib.gdn_hybrid_prefill_backward(_p(q), _p(k), _p(v), _p(a), _p(b), _p(d_o), _p(d_state),
                                         _p(dq), _p(dk), _p(dv), _p(da), _p(db), B, T, H, Hkv, d, d,
                                         n_sink, window, dt, _UPDATES["gdn"],
                                         float(weights[0]), float(weights[1]), _p(workspace),
                                         ws_bytes, _stream(q))
    _lib.check("gdn_hybrid_prefill_backward", rc)
    return dq, dk, dv, da, db


def hybrid_decode(q, k, v, a, b, state, k_cache, v_cache, a_cache, b_cache, pos,
                  n_sink: int, window: int, update: str = "gdn",
                  flags: int = BRANCH_LINEAR | BRANCH_SOFTMAX, o=None, weights=None):
    """One decode step for every sequence (state, caches and pos in place).

    ``weights=(w_lin, w_swa)``: o = w_lin o_lin + w_swa o_swa; omitted, the
    plain sum.

    q [B,H,d]; k/v [B,Hkv,d]; a [B,H] (GLA [B,H,d]); b [B,H]; state
    [B,H,d,d] fp32; k/v_cache [B,Hkv,n_sink+window,d]; a/b_cache
    [B,window,H] (GLA a: [B,window,H,d]); pos [B] int32.  Returns o [B,H,d].
    """
    B, H, dk = q.shape
    Hkv, dv = k.shape[1], v.shape[2]
    dt = _io_dtype(q, k, v, k_cache, v_cache)
    _f32(a, b, state, a_cache, b_cache)
    if pos.dtype != torch.int32:
        raise ValueError("pos must be int32")
    if o is None:
        o = torch.empty(B, H, dv, dtype=q.dtype, device=q.device)
    lib = _lib.load()
    ptrs = (_p(q), _p(k), _p(v), _p(a), _p(b), _p(state), _p(k_cache), _p(v_cache),
            _p(a_cache), _p(b_cache), _p(pos), _p(o))
    if weights is None:
        rc = lib.gdn_hybrid_decode(*ptrs, B, H, Hkv, dk, dv, n_sink, window, dt, _UPDATES[update],
                                   flags, _stream(q))
        _lib.check("gdn_hybrid_decode", rc)
    else:
        rc = lib.gdn_hybrid_decode_weighted(*ptrs, B, H, Hkv, dk, dv, n_sink, window, dt,
                                            _UPDATES[update], flags, float(weights[0]),
                                            float(weights[1]), _stream(q))
        _lib.check("gdn_hybrid_decode_weighted", rc)
    return o


def cache_from_prefill(k, v, a, b, H: int, n_sink: int, window: int, update: str = "gdn"):
    """Decode cache after a prefill of k/v [B,T,Hkv,d] with gates a, b.

    Returns (k_cache, v_cache, a_cache, b_cache).
    """
    B, T, Hkv, dk = k.shape
    dv = v.shape[3]
    dt = _io_dtype(k, v)
    _f32(a, b)
    N = n_sink + window
    dev = k.device
    kc = torch.empty(B, Hkv, N, dk, dtype=k.dtype, device=dev)
    vc = torch.empty(B, Hkv, N, dv, dtype=k.dtype, device=dev)
    ac = torch.empty((B, window, H, dk) if update in ("gla", "dgd") else (B, window, H),
                     dtype=torch.float32, device=dev)
    bc = torch.empty(B, window, H, dtype=torch.float32, device=dev)
    lib = _lib.load()
    rc = lib.gdn_hybrid_cache_from_prefill(_p(k), _p(v), _p(a), _p(b), _p(kc), _p(vc), _p(ac),
                                           _p(bc), B, T, H, Hkv, dk, dv, n_sink, window, dt,
                                           _UPDATES[update], _stream(k))
    _lib.check("gdn_hybrid_cache_from_prefill", rc)
    return kc, vc, ac, bc


def shortconv_qkv(q, k, v, wq, wk, wv, rope_theta: float = 1e6, pos0: int = 0,
                  flags: int = ROPE | L2NORM, out=None):
    """RoPE -> causal depthwise conv -> L2 norm on q, k (conv only on v).

    q [B,T,H,d], k/v [B,T,Hkv,d]; wq [H*d,ks], wk/wv [Hkv*d,ks] fp32.
    Returns (q_out, k_out, v_out).
    """
    B, T, H, d = q.shape
    Hkv = k.shape[2]
    ks = wq.shape[1]
    dt = _io_dtype(q, k, v)
    _f32(wq, wk, wv)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    qo, ko, vo = out
    lib = _lib.load()
    rc = lib.shortconv_qkv(_p(q), _p(k), _p(v), _p(wq), _p(wk), _p(wv), _p(qo), _p(ko), _p(vo),
                           B, T, H, Hkv, d, ks, float(rope_theta), pos0, flags, dt, _stream(q))
    _lib.check("shortconv_qkv", rc)
    return qo, ko, vo


def shortconv_history_from_prefill(q, k, v, ksize: int, rope_theta: float = 1e6, pos0: int = 0,
                                   flags: int = ROPE | L2NORM):
    """History of the short conv after a prefill of the raw q [B,T,H,d],
    k/v [B,T,Hkv,d]: fp32 [B, ksize-1, heads*d] for q, k, v (rotated inputs of
    the last ksize-1 tokens at ring index i mod (ksize-1))."""
    B, T, H, d = q.shape
    Hkv = k.shape[2]
    dt = _io_dtype(q, k, v)
    m = max(ksize - 1, 0)
    hist = (torch.empty(B, m, H * d, dtype=torch.float32, device=q.device),
            torch.empty(B, m, Hkv * d, dtype=torch.float32, device=q.device),
            torch.empty(B, m, Hkv * d, dtype=torch.float32, device=q.device))
    lib = _lib.load()
    rc = lib.shortconv_history_from_prefill(_p(q), _p(k), _p(v), _p(hist[0]), _p(hist[1]), _p(hist[2]),
                                            B, T, H, Hkv, d, ksize, float(rope_theta), pos0, flags, dt,
                                            _stream(q))
    _lib.check("shortconv_history_from_prefill", rc)
    return hist


def shortconv_decode(q, k, v, wq, wk, wv, hist_q, hist_k, hist_v, pos, rope_theta: float = 1e6,
                     pos0: int = 0, flags: int = ROPE | L2NORM, out=None):
    """One short-conv decode step: q [B,H,d], k/v [B,Hkv,d] raw projections of
    the new tokens at sequence indices pos [B] (int32, read only); updates the
    histories in place; returns (q_out, k_out, v_out)."""
    B, H, d = q.shape
    Hkv = k.shape[1]
    ks = wq.shape[1]
    dt = _io_dtype(q, k, v)
    _f32(wq, wk, wv, hist_q, hist_k, hist_v)
    if pos.dtype != torch.int32 or not pos.is_contiguous():
        raise TypeError("pos must be a contiguous int32 tensor")
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    qo, ko, vo = out
    lib = _lib.load()
    rc = lib.shortconv_qkv_decode(_p(q), _p(k), _p(v), _p(wq), _p(wk), _p(wv), _p(hist_q), _p(hist_k),
                                  _p(hist_v), _p(pos), _p(qo), _p(ko), _p(vo), B, H, Hkv, d, ks,
                                  float(rope_theta), pos0, flags, dt, _stream(q))
    _lib.check("shortconv_qkv_decode", rc)
    return qo, ko, vo

