"""Seeded synthetic workloads for the hybrid GDN + sink/SWA layer.

This module only draws random inputs and puts them in the shapes and value
distributions the layer is run on.  It holds none of the layer's arithmetic,
and both sides of every comparison (the HIP library and the CPU oracle)
consume the tensors it returns.

The pages measure on trained models (LLaMA3.1-8B, Qwen3 up to 32B) and public
evaluation suites; none of those are available, so these draws stand in for
them.  They keep the models' attention shapes (32 query / 8 KV heads at head
dim 128 for the 8B model, 64 / 8 for the 32B model), the pages' cache budgets
(64 and 128 = 8 sinks + window; 896 for long context) and the key structure
the first-order analysis assumes: unit-norm keys concentrated around one
direction per KV head.

Draw order (one generator, seed 0, fp32): q, per-KV-head mean direction mu,
key noise, v, b-logits, a-logits, then (as needed) GLA per-channel a-logits,
short-conv weights, and for decode: state, cached K, cached V, cached a,
cached b, then the per-step q, k, v, a, b.
"""

from __future__ import annotations

import dataclasses
import math

import torch

__all__ = ["Workload", "WORKLOADS", "make_prefill_inputs", "make_decode_inputs"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    d: int
    n_sink: int
    window: int
    T: int = 0                 # prefill length (0 for decode-only workloads)
    sigma: float = 0.5         # key noise scale around the head direction
    dtype: str = "bf16"        # q/k/v/o/cache element type: "f32" or "bf16"
    update: str = "gdn"        # "gdn", "gla" or "dgd" (delta rule, per-channel gate)
    write_state: bool = False
    shortconv: bool = False    # raw q/k/v go through RoPE -> conv -> L2 norm
    conv_ks: int = 8
    rope_theta: float = 1e6
    state_var: float = 0.02    # decode: variance of the random initial state
    pos0: int = 0              # decode: position of the first new token
    steps: int = 0             # decode: number of consecutive steps
    gate_mean: float = -4.0    # mean of the forget-gate logit: a = exp(-softplus(N(gate_mean, 1)))

    @property
    def budget(self) -> int:
        return self.n_sink + self.window

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    # fp32 tiny layer: B=1, H=2, T=256, d=64, budget 64 = 8 + 56.
    "tiny_fp32": Workload("tiny_fp32", B=1, H=2, Hkv=2, d=64, n_sink=8, window=56,
                          T=256, sigma=0.5, dtype="f32", write_state=True),
    # LLaMA3.1-8B attention shape, T=4096, budget 64 = 8 + 56.
    "llama8b_t4096": Workload("llama8b_t4096", B=1, H=32, Hkv=8, d=128, n_sink=8,
                              window=56, T=4096, sigma=0.5),
    # Long-context prefill, T=32768, budget 128 = 8 + 120, final states out.
    "longctx_b8_t32768": Workload("longctx_b8_t32768", B=8, H=32, Hkv=8, d=128,
                                  n_sink=8, window=120, T=32768, sigma=1.0,
                                  write_state=True),
    # The delta rule with a diagonal (per-channel) gate at the long-context
    # head shape: 8 sequences of 8192 tokens, budget 8 + 120, final state out.
    "dgd_b8_t8192": Workload("dgd_b8_t8192", B=8, H=32, Hkv=8, d=128, n_sink=8, window=120,
                             T=8192, sigma=1.0, write_state=True, update="dgd"),
    # Decode: 256 sequences, 32 query / 8 KV heads, cache 8 + 56, t = 4096+.
    "decode_b256": Workload("decode_b256", B=256, H=32, Hkv=8, d=128, n_sink=8,
                            window=56, sigma=0.5, pos0=4096, steps=1000),
    # Qwen3-32B attention shape with the full structural stack, budget 896.
    "qwen32b_t8192_gdn": Workload("qwen32b_t8192_gdn", B=2, H=64, Hkv=8, d=128,
                                  n_sink=8, window=888, T=8192, sigma=0.5,
                                  shortconv=True, update="gdn"),
    "qwen32b_t8192_gla": Workload("qwen32b_t8192_gla", B=2, H=64, Hkv=8, d=128,
                                  n_sink=8, window=888, T=8192, sigma=0.5,
                                  shortconv=True, update="gla"),
    # Serving the Qwen-shaped stack: decode steps after the T=8192 prefill
    # (short-conv decode feeding the layer's decode step), budget 896.
    "qwen32b_decode": Workload("qwen32b_decode", B=2, H=64, Hkv=8, d=128, n_sink=8,
                               window=888, sigma=0.5, shortconv=True, pos0=8192, steps=200),
}


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_prefill_inputs(w: Workload, device="cpu", seed: int = 0, T: int | None = None,
                        B: int | None = None):
    """Inputs of a prefill workload (optionally with a different T or B).

    Returns a dict with q [B,T,H,d], k/v [B,T,Hkv,d] in ``w.torch_dtype``,
    a [B,T,H] (GLA: [B,T,H,d]) and b [B,T,H] in fp32 and, for the short-conv
    stack, raw q/k/v plus conv weights wq [H*d,ks], wk/wv [Hkv*d,ks] in fp32.
    """
    T = w.T if T is None else T
    B = w.B if B is None else B
    g = _gen(device, seed)
    f32 = dict(device=device, dtype=torch.float32, generator=g)
    d = w.d
    q = torch.randn(B, T, w.H, d, **f32)
    mu = _unit(torch.randn(w.Hkv, d, **f32))
    knoise = torch.randn(B, T, w.Hkv, d, **f32)
    v = torch.randn(B, T, w.Hkv, d, **f32)
    b_logit = torch.randn(B, T, w.H, **f32)
    a_logit = torch.randn(B, T, w.H, **f32) + w.gate_mean
    k = mu[None, None] + w.sigma * knoise
    out = {}
    if w.update in ("gla", "dgd"):
        a_logit = torch.randn(B, T, w.H, d, **f32) + w.gate_mean
    if w.shortconv:
        ks = w.conv_ks
        std = 1.0 / math.sqrt(ks)
        out["wq"] = torch.randn(w.H * d, ks, **f32) * std
        out["wk"] = torch.randn(w.Hkv * d, ks, **f32) * std
        out["wv"] = torch.randn(w.Hkv * d, ks, **f32) * std
    else:
        q = _unit(q)
        k = _unit(k)
    dt = w.torch_dtype
    out.update(
        q=q.to(dt).contiguous(),
        k=k.to(dt).contiguous(),
        v=v.to(dt).contiguous(),
        a=torch.exp(-torch.nn.functional.softplus(a_logit)).contiguous(),
        b=torch.sigmoid(b_logit).contiguous(),
    )
    return out


def make_decode_inputs(w: Workload, device="cpu", seed: int = 0, steps: int | None = None,
                       B: int | None = None):
    """Random decode state + cache at position ``w.pos0`` and per-step inputs.

    Returns state [B,H,d,d] fp32 ~ N(0, state_var); k_cache/v_cache
    [B,Hkv,N,d]; a_cache/b_cache [B,W,H] (GLA a: [B,W,H,d]); pos [B] int32;
    and per-step q [S,B,H,d], k/v [S,B,Hkv,d], a [S,B,H] (GLA [S,B,H,d]),
    b [S,B,H].  For the short-conv stack the per-step q, k are the raw
    (un-normalised) projections, and conv weights wq [H*d,ks], wk/wv
    [Hkv*d,ks] ~ N(0, 1/ks) and fp32 histories hist_q [B,ks-1,H*d],
    hist_k/hist_v [B,ks-1,Hkv*d] ~ N(0, 1) are added (drawn last).
    """
    steps = w.steps if steps is None else steps
    B = w.B if B is None else B
    g = _gen(device, seed)
    f32 = dict(device=device, dtype=torch.float32, generator=g)
    d, H, Hkv, N, W = w.d, w.H, w.Hkv, w.budget, w.window
    dt = w.torch_dtype
    mu = _unit(torch.randn(Hkv, d, **f32))

    def keys(*lead):
        x = mu.view(*([1] * len(lead[:-1])), Hkv, d) + w.sigma * torch.randn(*lead, d, **f32)
        return x if raw else _unit(x)

    def gate_a(*shape):
        return torch.exp(-torch.nn.functional.softplus(torch.randn(*shape, **f32) + w.gate_mean))

    raw = False
    state = torch.randn(B, H, d, d, **f32) * math.sqrt(w.state_var)
    k_cache = keys(B, N, Hkv).permute(0, 2, 1, 3).to(dt).contiguous()
    raw = w.shortconv          # the cache holds prepared keys; new tokens arrive raw
    v_cache = torch.randn(B, Hkv, N, d, **f32).to(dt).contiguous()
    a_shape = (B, W, H, d) if w.update in ("gla", "dgd") else (B, W, H)
    a_cache = gate_a(*a_shape).contiguous()
    b_cache = torch.sigmoid(torch.randn(B, W, H, **f32)).contiguous()
    pos = torch.full((B,), w.pos0, dtype=torch.int32, device=device)
    q = torch.randn(steps, B, H, d, **f32)
    q = (q if raw else _unit(q)).to(dt).contiguous()
    k = keys(steps, B, Hkv).to(dt).contiguous()
    v = torch.randn(steps, B, Hkv, d, **f32).to(dt).contiguous()
    a_step_shape = (steps, B, H, d) if w.update in ("gla", "dgd") else (steps, B, H)
    a = gate_a(*a_step_shape).contiguous()
    b = torch.sigmoid(torch.randn(steps, B, H, **f32)).contiguous()
    out = dict(state=state, k_cache=k_cache, v_cache=v_cache, a_cache=a_cache,
               b_cache=b_cache, pos=pos, q=q, k=k, v=v, a=a, b=b)
    if w.shortconv:
        ks = w.conv_ks
        std = 1.0 / math.sqrt(ks)
        out["wq"] = torch.randn(H * d, ks, **f32) * std
        out["wk"] = torch.randn(Hkv * d, ks, **f32) * std
        out["wv"] = torch.randn(Hkv * d, ks, **f32) * std
        out["hist_q"] = torch.randn(B, ks - 1, H * d, **f32)
        out["hist_k"] = torch.randn(B, ks - 1, Hkv * d, **f32)
        out["hist_v"] = torch.randn(B, ks - 1, Hkv * d, **f32)
    return out
