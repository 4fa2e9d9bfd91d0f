"""Plain fp64 CPU oracle of the hybrid layer's backward pass (the gradients
of a loss through both branches), for the training path.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use this module; the product never
imports it.  Written from the forward definitions in ``oracle.hybrid`` by
reverse-mode differentiation, one token at a time, slow and literal.

Sources (pages cited by title and section):
* "The Key to Going Linear: Analysis-Driven Transformer Linearization",
  section 线性注意力替换机制: the recurrences differentiated here (gated delta
  rule, GLA, and the delta rule with the diagonal gate); section 实践建议
  item 4 speaks of training the linearised layers, which needs these
  gradients; section 填补近似缺口的实用设计: the sink + window budget and the
  lag of the linear read-out.
* Softmax logits q.k / sqrt(d) (section 从 softmax 到 delta 规则的一阶近似).

Conventions: the loss is L = sum(do * o) + sum(dS * S_final) for given
upstream gradients do [B,T,H,dv] and dS [B,H,dk,dv] (the final state's);
o = w_lin o_lin + w_swa o_swa.  GQA: gradients of k and v sum over the query
heads that share a KV head.  Pinned against central finite differences of
the forward oracle (tests/test_oracle_backward_pins.py).
"""

from __future__ import annotations

import numpy as np

from . import hybrid as F

__all__ = ["linear_branch_backward", "swa_branch_backward", "hybrid_prefill_backward"]


def _collapse_kv(x: np.ndarray, Hkv: int) -> np.ndarray:
    """[B,T,H,d] gradients of expanded K/V -> [B,T,Hkv,d] (sum over the G
    query heads of each KV head)."""
    B, T, H, d = x.shape
    return x.reshape(B, T, Hkv, H // Hkv, d).sum(axis=3)


def linear_branch_backward(q, k, v, a, b, n_sink: int, window: int, do, dS=None,
                           update: str = "gdn"):
    """Gradients of sum(do * o_lin) + sum(dS * S_final) for the lagged
    recurrence of ``update`` ("gdn": scalar a, b; "gla": per-channel a;
    "dgd": per-channel a and scalar b).  Returns (dq, dk, dv, da, db); db is
    None for GLA.

    Forward (token i = n_sink .. T-1-window, S_{i-1} the state before it):
      gdn: S_i = a_i (S_{i-1} - b_i k_i (k_i^T S_{i-1})) + b_i k_i v_i^T
      gla: S_i = Diag(a_i) S_{i-1} + k_i v_i^T
      dgd: X = Diag(a_i) S_{i-1};  S_i = X - b_i k_i (k_i^T X) + b_i k_i v_i^T
      o_lin[i + window] = S_i^T q[i + window]
    """
    q = np.asarray(q, np.float64)
    B, T, H, dk = q.shape
    Hkv = np.asarray(k).shape[2]
    kh = F._expand_kv(np.asarray(k, np.float64), H)
    vh = F._expand_kv(np.asarray(v, np.float64), H)
    a = np.asarray(a, np.float64)
    b = None if b is None else np.asarray(b, np.float64)
    do = np.asarray(do, np.float64)
    dv_ = vh.shape[-1]
    # forward, keeping every state
    steps = list(range(n_sink, T - window))
    S = np.zeros((B, H, dk, dv_))
    states = [S]
    for i in steps:
        ki, vi = kh[:, i], vh[:, i]
        if update == "gdn":
            ai = a[:, i][:, :, None, None]
            bi = b[:, i][:, :, None, None]
            kS = np.einsum("bhk,bhkv->bhv", ki, S)
            S = ai * (S - bi * ki[..., :, None] * kS[..., None, :]) + bi * ki[..., :, None] * vi[..., None, :]
        elif update == "gla":
            S = a[:, i][..., :, None] * S + ki[..., :, None] * vi[..., None, :]
        elif update == "dgd":
            bi = b[:, i][:, :, None, None]
            X = a[:, i][..., :, None] * S
            kX = np.einsum("bhk,bhkv->bhv", ki, X)
            S = X - bi * ki[..., :, None] * kX[..., None, :] + bi * ki[..., :, None] * vi[..., None, :]
        else:
            raise ValueError(update)
        states.append(S)
    # reverse sweep
    dq = np.zeros_like(q)
    dkh = np.zeros_like(kh)
    dvh = np.zeros_like(vh)
    da = np.zeros_like(a)
    db = None if update == "gla" else np.zeros_like(b)
    G = np.zeros((B, H, dk, dv_)) if dS is None else np.array(dS, np.float64, copy=True)
    for n in range(len(steps) - 1, -1, -1):
        i = steps[n]
        t = i + window
        Si, Sp = states[n + 1], states[n]
        # read-out o[t] = S_i^T q_t
        dq[:, t] += np.einsum("bhkv,bhv->bhk", Si, do[:, t])
        G = G + q[:, t][..., :, None] * do[:, t][..., None, :]
        ki, vi = kh[:, i], vh[:, i]
        if update == "gdn":
            ai = a[:, i][:, :, None, None]
            bi = b[:, i][:, :, None, None]
            kS = np.einsum("bhk,bhkv->bhv", ki, Sp)                 # k^T S_{i-1}
            proj = Sp - bi * ki[..., :, None] * kS[..., None, :]     # (I - b k k^T) S_{i-1}
            da[:, i] += np.einsum("bhkv,bhkv->bh", G, proj)
            kvT = ki[..., :, None] * vi[..., None, :]
            kkS = ki[..., :, None] * kS[..., None, :]
            db[:, i] += np.einsum("bhkv,bhkv->bh", G, kvT - ai * kkS)
            dvh[:, i] += b[:, i][..., None] * np.einsum("bhkv,bhk->bhv", G, ki)
            GS = np.einsum("bhkv,bhjv->bhkj", G, Sp)                 # G S^T
            dkh[:, i] += -(a[:, i] * b[:, i])[..., None] * (np.einsum("bhkj,bhj->bhk", GS, ki)
                                                            + np.einsum("bhjk,bhj->bhk", GS, ki)) \
                + b[:, i][..., None] * np.einsum("bhkv,bhv->bhk", G, vi)
            kG = np.einsum("bhk,bhkv->bhv", ki, G)
            G = ai * (G - bi * ki[..., :, None] * kG[..., None, :])
        elif update == "gla":
            da[:, i] += np.einsum("bhkv,bhkv->bhk", G, Sp)
            dkh[:, i] += np.einsum("bhkv,bhv->bhk", G, vi)
            dvh[:, i] += np.einsum("bhkv,bhk->bhv", G, ki)
            G = a[:, i][..., :, None] * G
        else:  # dgd
            bi = b[:, i][:, :, None, None]
            X = a[:, i][..., :, None] * Sp
            kX = np.einsum("bhk,bhkv->bhv", ki, X)
            kvT = ki[..., :, None] * vi[..., None, :]
            db[:, i] += np.einsum("bhkv,bhkv->bh", G, kvT - ki[..., :, None] * kX[..., None, :])
            dvh[:, i] += b[:, i][..., None] * np.einsum("bhkv,bhk->bhv", G, ki)
            GX = np.einsum("bhkv,bhjv->bhkj", G, X)                  # G X^T
            dkh[:, i] += -b[:, i][..., None] * (np.einsum("bhkj,bhj->bhk", GX, ki)
                                                + np.einsum("bhjk,bhj->bhk", GX, ki)) \
                + b[:, i][..., None] * np.einsum("bhkv,bhv->bhk", G, vi)
            kG = np.einsum("bhk,bhkv->bhv", ki, G)
            dX = G - bi * ki[..., :, None] * kG[..., None, :]
            da[:, i] += np.einsum("bhkv,bhkv->bhk", dX, Sp)
            G = a[:, i][..., :, None] * dX
    return dq, _collapse_kv(dkh, Hkv), _collapse_kv(dvh, Hkv), da, db


def swa_branch_backward(q, k, v, n_sink: int, window: int, do):
    """Gradients of sum(do * o_swa) (the softmax over A(t), logits
    q.k / sqrt(d)).  Returns (dq, dk, dv)."""
    q = np.asarray(q, np.float64)
    B, T, H, dk = q.shape
    Hkv = np.asarray(k).shape[2]
    kh = F._expand_kv(np.asarray(k, np.float64), H)
    vh = F._expand_kv(np.asarray(v, np.float64), H)
    do = np.asarray(do, np.float64)
    scale = 1.0 / np.sqrt(dk)
    dq = np.zeros_like(q)
    dkh = np.zeros_like(kh)
    dvh = np.zeros_like(vh)
    for t in range(T):
        idx = F.softmax_index_set(t, n_sink, window)
        z = np.einsum("bhd,bnhd->bhn", q[:, t], kh[:, idx]) * scale
        z = z - z.max(axis=-1, keepdims=True)
        p = np.exp(z)
        p = p / p.sum(axis=-1, keepdims=True)                       # [B,H,n]
        dp = np.einsum("bhv,bnhv->bhn", do[:, t], vh[:, idx])
        dz = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
        dq[:, t] += scale * np.einsum("bhn,bnhd->bhd", dz, kh[:, idx])
        dkh[:, idx] += scale * np.einsum("bhn,bhd->bnhd", dz, q[:, t])
        dvh[:, idx] += np.einsum("bhn,bhv->bnhv", p, do[:, t])
    return dq, _collapse_kv(dkh, Hkv), _collapse_kv(dvh, Hkv)


def hybrid_prefill_backward(q, k, v, a, b, n_sink: int, window: int, do, dS=None,
                            update: str = "gdn", w_lin: float = 1.0, w_swa: float = 1.0):
    """Gradients of sum(do * o) + sum(dS * S_final), o = w_lin o_lin +
    w_swa o_swa.  Returns (dq, dk, dv, da, db)."""
    do = np.asarray(do, np.float64)
    dq, dk, dv, da, db = linear_branch_backward(q, k, v, a, b, n_sink, window, w_lin * do, dS,
                                                update=update)
    sq, sk, sv = swa_branch_backward(q, k, v, n_sink, window, w_swa * do)
    return dq + sq, dk + sk, dv + sv, da, db
