"""Plain fp64 CPU oracle of the hybrid GDN + sink/sliding-window attention layer.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use this module.  The product (the HIP
library under ``swa_chunked_gated_amd``) never imports it and shares no code
with it.  Everything here is written from the method's definition, slow and
literal: loops over tokens, explicit index sets, NumPy float64.

Sources (the pages, cited by page title and section):

* P1 = "The Key to Going Linear: Analysis-Driven Transformer Linearization"
  (Chinese summary page of arXiv 2607.07706v1).
  - section 线性注意力替换机制 (linear-attention replacement): the GLA update
    S_t = G_t S_{t-1} + k_t v_t^T with a diagonal input-dependent forget gate,
    and the GDN update S_t = (I - b_t k_t k_t^T) G_t S_{t-1} + b_t k_t v_t^T
    with a per-token scalar b_t ("beta").
  - section 从 softmax 到 delta 规则的一阶近似 (first-order approximation):
    the softmax logits are q^T k / sqrt(d) (Lemma 1), and the effective
    attention weight of token i is q^T prod_j (I - b_j k_j k_j^T) k_i.
  - section 填补近似缺口的实用设计 (practical designs): a fixed attention
    budget of 64 = 8 sink tokens that always get full attention + 56
    sliding-window tokens; the linear path handles every other token.
  - section 实践建议 item 2 (fixed cache budget split into sinks and window)
    and item 3 (kernel-8 short convolution on Q/K/V after RoPE, before the L2
    normalisation).
* P2 = "線性化 Transformer 但不掉品質" (news page), section 方法到底怎麼做:
  sink tokens, short convolutions and fixed-budget cache routing are the three
  structural additions.
* P3 = "Untangling Component Imbalance in Hybrid Linear Attention Conversion
  Methods", sections 核心思路 / 关键设计: a hybrid layer combines a linear
  branch with sliding-window softmax.

Readings where the pages are silent (the full list with reasons is kept with
the design notes of the repository):

* Column vectors; S is d_k x d_v; the linear output is S^T q.
* GDN gate is one scalar a_t per (token, query head); a_t (I - b k k^T) S is
  the same as (I - b k k^T) a_t S for a scalar gate.  The diagonal-gate
  variant ("dgd") keeps the page's order for a per-channel gate: the gate
  first, then the delta projection, (I - b k k^T) Diag(alpha) S.
* Softmax set of query t:  A(t) = { i <= t : i < n_sink or i > t - window }
  (window includes the current token; sinks are absolute positions 0..n_sink-1;
  the union counts each key once).
* Linear set of query t:   L(t) = { i : n_sink <= i <= t - window }, i.e. the
  recurrence runs over evicted non-sink tokens and is queried with lag
  ``window``: o_lin,t = S^(t-window)^T q_t, and 0 while t - window < n_sink.
* Layer output: o = o_lin + o_swa (plain sum); with branch weights
  (inference-time hybridisation, P3 关键设计 (1)) o = w_lin o_lin + w_swa o_swa.
* Grouped-query attention: query head h uses KV head h // (H // Hkv); gates
  and the state are per query head.
* Short conv: causal, depthwise, zero history, no bias, no activation; tap
  w[c, ks-1] multiplies the current token.  RoPE: rotate-half pairs
  (j, j + d/2), inv_freq_j = theta^(-2j/d), position pos0 + t, on q and k only.
  L2 norm: x / sqrt(sum x^2 + 1e-6), on q and k only.

Pins (in ``tests/test_oracle_pins.py``): brute-force partition of the index
sets; the materialised effective-attention product form on tiny inputs;
exact retrieval with orthonormal keys; equality with full causal softmax
(torch SDPA, fp64) when T <= budget; an fp64 chunked (WY/UT) form for several
chunk sizes; the GLA diagonal-product form; for the diagonal-gate delta
rule: a channel-uniform gate == the scalar-gate rule, the per-channel
closed form with one-hot keys, and an fp64 chunked form with per-channel
decays; prefill + decode == longer
prefill; GQA == explicitly repeated K/V; torch conv1d for the short conv;
RoPE closed forms and invariants; short-conv decode steps from a prefill's
history == the longer prefill's rows.  No function here is "parity unpinned"
against the mathematics; none is pinned by printed values, since the pages
print no worked example.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "in_softmax_set",
    "in_linear_set",
    "softmax_index_set",
    "linear_index_set",
    "gdn_linear_branch",
    "gla_linear_branch",
    "dgd_linear_branch",
    "swa_branch",
    "hybrid_prefill",
    "cache_from_prefill",
    "decode_step",
    "rope",
    "causal_depthwise_conv",
    "l2norm",
    "shortconv_qkv",
    "shortconv_history_from_prefill",
    "shortconv_decode_step",
]

BRANCH_LINEAR = 1
BRANCH_SOFTMAX = 2
WRITE_STATE = 4


# --------------------------------------------------------------------------
# Fixed-budget cache routing (P1, 填补近似缺口的实用设计; P2, 方法到底怎麼做)
# --------------------------------------------------------------------------

def in_softmax_set(t: int, i: int, n_sink: int, window: int) -> bool:
    """True iff key i is attended by softmax at query t (sinks + window)."""
    return i <= t and (i < n_sink or i > t - window)


def in_linear_set(t: int, i: int, n_sink: int, window: int) -> bool:
    """True iff key i has been folded into the linear state read by query t."""
    return n_sink <= i <= t - window


def softmax_index_set(t: int, n_sink: int, window: int) -> np.ndarray:
    """Explicit A(t) as a sorted int array, built from the predicate."""
    i = np.arange(t + 1)
    keep = (i < n_sink) | (i > t - window)
    return i[keep]


def linear_index_set(t: int, n_sink: int, window: int) -> np.ndarray:
    """Explicit L(t) as a sorted int array."""
    return np.arange(n_sink, max(n_sink, t - window + 1))


def _expand_kv(x: np.ndarray, H: int) -> np.ndarray:
    """[B,T,Hkv,d] -> [B,T,H,d]: query head h reads KV head h // (H // Hkv)."""
    Hkv = x.shape[2]
    assert H % Hkv == 0
    return np.repeat(x, H // Hkv, axis=2)


# --------------------------------------------------------------------------
# Linear branch (P1, 线性注意力替换机制: GDN and GLA updates)
# --------------------------------------------------------------------------

def gdn_linear_branch(q, k, v, a, b, n_sink: int, window: int):
    """Lagged gated delta rule.

    For i = n_sink .. T-1-window (the tokens that have left the window):
        S <- a_i (I - b_i k_i k_i^T) S + b_i k_i v_i^T
        o_lin[i + window] = S^T q[i + window]
    Rows t < n_sink + window get 0.  Returns (o_lin [B,T,H,dv], S [B,H,dk,dv]),
    S being the state after the last folded token (zero if none).
    """
    q = np.asarray(q, np.float64)
    B, T, H, dk = q.shape
    kh = _expand_kv(np.asarray(k, np.float64), H)
    vh = _expand_kv(np.asarray(v, np.float64), H)
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    dv = vh.shape[-1]
    S = np.zeros((B, H, dk, dv))
    o = np.zeros((B, T, H, dv))
    for i in range(n_sink, T - window):
        ki = kh[:, i]                                   # [B,H,dk]
        vi = vh[:, i]                                   # [B,H,dv]
        ai = a[:, i][:, :, None, None]                  # [B,H,1,1]
        bi = b[:, i][:, :, None, None]
        # (I - b k k^T) S evaluated as S - b k (k^T S)
        kS = np.einsum("bhk,bhkv->bhv", ki, S)          # k^T S  [B,H,dv]
        proj_S = S - bi * (ki[:, :, :, None] * kS[:, :, None, :])
        S = ai * proj_S + bi * (ki[:, :, :, None] * vi[:, :, None, :])
        t = i + window
        o[:, t] = np.einsum("bhkv,bhk->bhv", S, q[:, t])
    return o, S


def gla_linear_branch(q, k, v, alpha, n_sink: int, window: int):
    """Lagged gated linear attention with a diagonal gate on the d_k rows.

    For i = n_sink .. T-1-window:
        S <- Diag(alpha_i) S + k_i v_i^T
        o_lin[i + window] = S^T q[i + window]
    ``alpha`` is [B,T,H,dk].  Returns (o_lin, S_final).
    """
    q = np.asarray(q, np.float64)
    B, T, H, dk = q.shape
    kh = _expand_kv(np.asarray(k, np.float64), H)
    vh = _expand_kv(np.asarray(v, np.float64), H)
    alpha = np.asarray(alpha, np.float64)
    dv = vh.shape[-1]
    S = np.zeros((B, H, dk, dv))
    o = np.zeros((B, T, H, dv))
    for i in range(n_sink, T - window):
        S = alpha[:, i][:, :, :, None] * S \
            + kh[:, i][:, :, :, None] * vh[:, i][:, :, None, :]
        t = i + window
        o[:, t] = np.einsum("bhkv,bhk->bhv", S, q[:, t])
    return o, S


def dgd_linear_branch(q, k, v, alpha, b, n_sink: int, window: int):
    """Lagged delta rule with a diagonal gate (P1, 线性注意力替换机制: the GDN
    update with G_t = Diag(alpha_t), one forget value per d_k channel).

    For i = n_sink .. T-1-window:
        S <- (I - b_i k_i k_i^T) Diag(alpha_i) S + b_i k_i v_i^T
        o_lin[i + window] = S^T q[i + window]
    ``alpha`` is [B,T,H,dk], ``b`` [B,T,H].  Returns (o_lin, S_final).
    """
    q = np.asarray(q, np.float64)
    B, T, H, dk = q.shape
    kh = _expand_kv(np.asarray(k, np.float64), H)
    vh = _expand_kv(np.asarray(v, np.float64), H)
    alpha = np.asarray(alpha, np.float64)
    b = np.asarray(b, np.float64)
    dv = vh.shape[-1]
    S = np.zeros((B, H, dk, dv))
    o = np.zeros((B, T, H, dv))
    for i in range(n_sink, T - window):
        ki = kh[:, i]                                   # [B,H,dk]
        vi = vh[:, i]
        bi = b[:, i][:, :, None, None]
        GS = alpha[:, i][:, :, :, None] * S             # Diag(alpha_i) S
        kGS = np.einsum("bhk,bhkv->bhv", ki, GS)        # k^T Diag(alpha) S
        S = GS - bi * (ki[:, :, :, None] * kGS[:, :, None, :]) \
            + bi * (ki[:, :, :, None] * vi[:, :, None, :])
        t = i + window
        o[:, t] = np.einsum("bhkv,bhk->bhv", S, q[:, t])
    return o, S


# --------------------------------------------------------------------------
# Softmax branch over sinks + sliding window (P1, 填补近似缺口的实用设计;
# scale 1/sqrt(d_k) from the first-order-approximation section)
# --------------------------------------------------------------------------

def swa_branch(q, k, v, n_sink: int, window: int, rows=None):
    """o_swa[t] = sum_{i in A(t)} softmax_i(q_t . k_i / sqrt(d_k)) v_i.

    ``rows`` optionally restricts the query rows computed (others stay 0).
    """
    q = np.asarray(q, np.float64)
    B, T, H, dk = q.shape
    kh = _expand_kv(np.asarray(k, np.float64), H)
    vh = _expand_kv(np.asarray(v, np.float64), H)
    dv = vh.shape[-1]
    o = np.zeros((B, T, H, dv))
    scale = 1.0 / np.sqrt(dk)
    for t in (range(T) if rows is None else rows):
        idx = softmax_index_set(int(t), n_sink, window)
        logits = np.einsum("bhd,bnhd->bhn", q[:, t], kh[:, idx]) * scale
        logits = logits - logits.max(axis=-1, keepdims=True)
        p = np.exp(logits)
        p = p / p.sum(axis=-1, keepdims=True)
        o[:, t] = np.einsum("bhn,bnhd->bhd", p, vh[:, idx])
    return o


# --------------------------------------------------------------------------
# The layer: prefill
# --------------------------------------------------------------------------

def hybrid_prefill(q, k, v, a, b, n_sink: int, window: int, update: str = "gdn",
                   flags: int = BRANCH_LINEAR | BRANCH_SOFTMAX | WRITE_STATE,
                   w_lin: float = 1.0, w_swa: float = 1.0):
    """o = w_lin o_lin + w_swa o_swa for a whole sequence starting at
    position 0; the weights (P3, 关键设计 (1): inference-time hybridisation
    sets the branches' contributions by weights) default to the plain sum.

    ``update`` is "gdn" (a, b: [B,T,H]), "gla" (a: [B,T,H,dk], b unused) or
    "dgd" (the delta rule with a diagonal gate: a [B,T,H,dk], b [B,T,H]).
    Returns (o [B,T,H,dv], final state [B,H,dk,dv] or None).
    """
    q = np.asarray(q, np.float64)
    B, T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    o = np.zeros((B, T, H, dv))
    S = None
    if flags & (BRANCH_LINEAR | WRITE_STATE):
        if update == "gdn":
            o_lin, S = gdn_linear_branch(q, k, v, a, b, n_sink, window)
        elif update == "gla":
            o_lin, S = gla_linear_branch(q, k, v, a, n_sink, window)
        elif update == "dgd":
            o_lin, S = dgd_linear_branch(q, k, v, a, b, n_sink, window)
        else:
            raise ValueError(update)
        if flags & BRANCH_LINEAR:
            o = o + w_lin * o_lin
    if flags & BRANCH_SOFTMAX:
        o = o + w_swa * swa_branch(q, k, v, n_sink, window)
    return o, (S if flags & WRITE_STATE else None)


# --------------------------------------------------------------------------
# Decode: fixed-budget cache with n_sink sink slots + a window-slot ring
# --------------------------------------------------------------------------

def cache_slot(i: int, n_sink: int, window: int) -> int:
    """Cache slot of absolute token i: sinks stay put, the rest go round a ring."""
    return i if i < n_sink else n_sink + (i - n_sink) % window


def cache_from_prefill(k, v, a, b, n_sink: int, window: int, update: str = "gdn"):
    """Cache contents right after a prefill of T tokens (decode resumes at T).

    Holds sinks 0..min(n_sink,T)-1 and window tokens max(n_sink, T-window)..T-1
    (the oldest of those is the one the next decode step folds into the state),
    each in its slot; the gates of the window tokens go to ring index
    (i - n_sink) mod window.  Unwritten slots are zero.
    Returns (k_cache [B,Hkv,N,dk], v_cache, a_cache [B,W,H(,dk)], b_cache [B,W,H]).
    """
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    a = np.asarray(a, np.float64)
    B, T, Hkv, dk = k.shape
    dv = v.shape[-1]
    H = a.shape[2]
    N = n_sink + window
    kc = np.zeros((B, Hkv, N, dk))
    vc = np.zeros((B, Hkv, N, dv))
    ac = np.zeros((B, window, H) + ((dk,) if update in ("gla", "dgd") else ()))
    bc = np.zeros((B, window, H))
    toks = list(range(min(n_sink, T))) + list(range(max(n_sink, T - window), T))
    for i in toks:
        s = cache_slot(i, n_sink, window)
        kc[:, :, s] = k[:, i]
        vc[:, :, s] = v[:, i]
        if i >= n_sink:
            r = (i - n_sink) % window
            ac[:, r] = a[:, i]
            if b is not None:
                bc[:, r] = np.asarray(b, np.float64)[:, i]
    return kc, vc, ac, bc


def decode_step(q, k, v, a, b, state, k_cache, v_cache, a_cache, b_cache, pos,
                n_sink: int, window: int, update: str = "gdn",
                flags: int = BRANCH_LINEAR | BRANCH_SOFTMAX, w_lin: float = 1.0,
                w_swa: float = 1.0):
    """One decode step for every sequence; returns new copies of everything.
    The output is w_lin o_lin + w_swa o_swa (weights as in hybrid_prefill).

    q [B,H,dk]; k [B,Hkv,dk]; v [B,Hkv,dv]; a [B,H] (GLA, DGD: [B,H,dk]); b [B,H];
    state [B,H,dk,dv]; caches as in ``cache_from_prefill``; pos [B] = index t
    of the new token.  Per sequence:
      1. e = t - window; if e >= n_sink, fold token e (read from its slot,
         gates from ring index (e - n_sink) mod window) into the state.
      2. o_lin = S^T q.
      3. o_swa = softmax over A(t): cached keys for i in A(t), i < t, and the
         new k for i = t.
      4. Store the new token in slot(t) (and its gates when t >= n_sink).
      5. pos += 1.
    Returns (o [B,H,dv], state, k_cache, v_cache, a_cache, b_cache, pos).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    a = np.asarray(a, np.float64)
    b = None if b is None else np.asarray(b, np.float64)
    S = np.array(state, np.float64, copy=True)
    kc = np.array(k_cache, np.float64, copy=True)
    vc = np.array(v_cache, np.float64, copy=True)
    ac = np.array(a_cache, np.float64, copy=True)
    bc = np.array(b_cache, np.float64, copy=True)
    pos = np.array(pos, np.int64, copy=True)
    B, H, dk = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    dv = v.shape[-1]
    o = np.zeros((B, H, dv))
    scale = 1.0 / np.sqrt(dk)
    heads = np.arange(H)
    kvh = heads // G
    for bi in range(B):
        t = int(pos[bi])
        # 1. eviction into the linear state
        e = t - window
        if e >= n_sink:
            s_e = cache_slot(e, n_sink, window)
            r_e = (e - n_sink) % window
            ke = kc[bi, kvh, s_e]                       # [H,dk]
            ve = vc[bi, kvh, s_e]                       # [H,dv]
            if update == "gdn":
                ae = ac[bi, r_e][:, None, None]         # [H,1,1]
                be = bc[bi, r_e][:, None, None]
                kS = np.einsum("hk,hkv->hv", ke, S[bi])  # k_e^T S
                proj_S = S[bi] - be * (ke[:, :, None] * kS[:, None, :])
                S[bi] = ae * proj_S + be * (ke[:, :, None] * ve[:, None, :])
            elif update == "dgd":
                be = bc[bi, r_e][:, None, None]
                GS = ac[bi, r_e][:, :, None] * S[bi]    # Diag(alpha_e) S
                kGS = np.einsum("hk,hkv->hv", ke, GS)
                S[bi] = GS - be * (ke[:, :, None] * kGS[:, None, :]) \
                    + be * (ke[:, :, None] * ve[:, None, :])
            else:
                S[bi] = ac[bi, r_e][:, :, None] * S[bi] \
                    + ke[:, :, None] * ve[:, None, :]
        # 2. linear read-out
        o_lin = np.einsum("hkv,hk->hv", S[bi], q[bi])
        # 3. softmax over sinks + window, new token included
        idx = softmax_index_set(t, n_sink, window)
        keys = np.zeros((len(idx), H, dk))
        vals = np.zeros((len(idx), H, dv))
        for n, i in enumerate(idx):
            if i == t:
                keys[n] = k[bi, kvh]
                vals[n] = v[bi, kvh]
            else:
                s = cache_slot(int(i), n_sink, window)
                keys[n] = kc[bi, kvh, s]
                vals[n] = vc[bi, kvh, s]
        logits = np.einsum("hd,nhd->hn", q[bi], keys) * scale
        logits = logits - logits.max(axis=-1, keepdims=True)
        p = np.exp(logits)
        p = p / p.sum(axis=-1, keepdims=True)
        o_swa = np.einsum("hn,nhd->hd", p, vals)
        out = np.zeros((H, dv))
        if flags & BRANCH_LINEAR:
            out = out + w_lin * o_lin
        if flags & BRANCH_SOFTMAX:
            out = out + w_swa * o_swa
        o[bi] = out
        # 4. store the new token
        s_t = cache_slot(t, n_sink, window)
        kc[bi, :, s_t] = k[bi]
        vc[bi, :, s_t] = v[bi]
        if t >= n_sink:
            r_t = (t - n_sink) % window
            ac[bi, r_t] = a[bi]
            if b is not None:
                bc[bi, r_t] = b[bi]
        # 5. advance
        pos[bi] = t + 1
    return o, S, kc, vc, ac, bc, pos


# --------------------------------------------------------------------------
# Q/K/V structural preparation (P1, 实践建议 item 3: RoPE -> kernel-8 causal
# short conv -> L2 norm)
# --------------------------------------------------------------------------

def rope(x, theta: float, pos0: int = 0):
    """Rotate-half RoPE on [B,T,H,d] at absolute positions pos0 + t."""
    x = np.asarray(x, np.float64)
    B, T, H, d = x.shape
    half = d // 2
    inv_freq = theta ** (-2.0 * np.arange(half) / d)            # [half]
    ang = (pos0 + np.arange(T))[:, None] * inv_freq[None, :]     # [T,half]
    c = np.cos(ang)[None, :, None, :]
    s = np.sin(ang)[None, :, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def causal_depthwise_conv(x, w):
    """y[t, c] = sum_{j=0}^{ks-1} w[c, ks-1-j] * x[t-j, c], zero history.

    x is [B,T,H,d] with channel c = h*d + i; w is [H*d, ks].
    """
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    B, T, H, d = x.shape
    ks = w.shape[1]
    xc = x.reshape(B, T, H * d)
    y = np.zeros_like(xc)
    for j in range(ks):
        if j >= T:
            break
        y[:, j:, :] += w[None, None, :, ks - 1 - j] * xc[:, : T - j, :]
    return y.reshape(B, T, H, d)


def l2norm(x, eps: float = 1e-6):
    """x / sqrt(sum_i x_i^2 + eps) over the last axis."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt((x * x).sum(axis=-1, keepdims=True) + eps)


def shortconv_qkv(q, k, v, wq, wk, wv, rope_theta: float, pos0: int = 0,
                  flags: int = 3):
    """RoPE (flag 1, q and k) -> causal depthwise conv (q, k, v) -> L2 norm
    (flag 2, q and k).  Returns (q_out, k_out, v_out) in fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    if flags & 1:
        q = rope(q, rope_theta, pos0)
        k = rope(k, rope_theta, pos0)
    q = causal_depthwise_conv(q, wq)
    k = causal_depthwise_conv(k, wk)
    v = causal_depthwise_conv(v, wv)
    if flags & 2:
        q = l2norm(q)
        k = l2norm(k)
    return q, k, v


# --------------------------------------------------------------------------
# Q/K/V preparation in decode (the same operation as shortconv_qkv, taken one
# token at a time): each sequence keeps the inputs of its last ks - 1 tokens
# after RoPE and before the convolution; token i sits at ring index
# i mod (ks - 1).  Tokens before the sequence start count as zero.
# --------------------------------------------------------------------------

def _rope_row(x, pos: int, theta: float):
    """Rotate-half RoPE of one token's heads x [heads, d] at position pos."""
    x = np.asarray(x, np.float64)
    half = x.shape[-1] // 2
    ang = pos * theta ** (-2.0 * np.arange(half) / x.shape[-1])
    c, s = np.cos(ang), np.sin(ang)
    return np.concatenate([x[:, :half] * c - x[:, half:] * s, x[:, half:] * c + x[:, :half] * s], axis=-1)


def shortconv_history_from_prefill(q, k, v, ksize: int, rope_theta: float, pos0: int = 0,
                                 flags: int = 3):
    """History after a prefill of T tokens (positions pos0 .. pos0+T-1), so that
    decoding continues with token T: for q, k, v the inputs of tokens
    T-ks+1 .. T-1 (rotated for q and k when flags & 1), each at ring index
    i mod (ks-1).  Returns three fp64 arrays [B, ks-1, heads*d]."""
    out = []
    for x, rot in ((q, True), (k, True), (v, False)):
        x = np.asarray(x, np.float64)
        B, T, nh, d = x.shape
        hist = np.zeros((B, max(ksize - 1, 0), nh * d))
        for i in range(T - (ksize - 1), T):
            if i < 0:
                continue
            for b in range(B):
                xi = _rope_row(x[b, i], pos0 + i, rope_theta) if (rot and flags & 1) else x[b, i]
                hist[b, i % (ksize - 1)] = xi.reshape(-1)
        out.append(hist)
    return tuple(out)


def shortconv_decode_step(q, k, v, wq, wk, wv, hist_q, hist_k, hist_v, pos, rope_theta: float,
                          pos0: int = 0, flags: int = 3):
    """One new token per sequence: q [B,H,d], k, v [B,Hkv,d] (raw projections),
    pos [B] the token's index in its sequence.  RoPE at position pos0 + pos
    (flags & 1, q and k), causal depthwise conv over the token and its ks-1
    predecessors from the history (y = sum_j w[c, ks-1-j] x[t-j]), L2 norm
    (flags & 2, q and k).  The histories [B, ks-1, C] are updated in place
    (the new input replaces token t-ks+1 at ring index t mod (ks-1)).
    Returns (q_out, k_out, v_out) in fp64."""
    outs = []
    for x, w, hist, rot in ((q, wq, hist_q, True), (k, wk, hist_k, True), (v, wv, hist_v, False)):
        x = np.asarray(x, np.float64)
        w = np.asarray(w, np.float64)
        B, nh, d = x.shape
        ks = w.shape[1]
        y = np.zeros((B, nh * d))
        for b in range(B):
            t = int(pos[b])
            xt = _rope_row(x[b], pos0 + t, rope_theta) if (rot and flags & 1) else x[b]
            xt = xt.reshape(-1)
            acc = w[:, ks - 1] * xt
            for j in range(1, ks):
                if t - j >= 0:
                    acc = acc + w[:, ks - 1 - j] * hist[b, (t - j) % (ks - 1)]
            if ks > 1:
                hist[b, t % (ks - 1)] = xt
            y[b] = acc
        y = y.reshape(B, nh, d)
        if rot and flags & 2:
            y = l2norm(y)
        outs.append(y)
    return tuple(outs)
