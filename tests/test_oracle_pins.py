"""Pins of the CPU oracle against facts fixed outside it (no GPU needed).

Each test checks the oracle against something other than itself: brute-force
enumeration, a closed form, a library routine (torch SDPA / conv1d in fp64),
or a different algorithm for the same quantity (the materialised
effective-attention product form, an fp64 chunked WY/UT form, decode
stepping).  The pages print no worked numeric example, so no value here is
taken from them; the definitions cited are in ``oracle.hybrid``.
"""

import math

import numpy as np
import pytest
import torch

from oracle import hybrid as O

RNG = np.random.default_rng(1234)


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_layer(B, T, H, Hkv, d, rng=RNG, concentrated=0.5, gla=False):
    q = unit(rng.standard_normal((B, T, H, d)))
    mu = unit(rng.standard_normal((Hkv, d)))
    k = unit(mu[None, None] + concentrated * rng.standard_normal((B, T, Hkv, d)))
    v = rng.standard_normal((B, T, Hkv, d))
    b = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    if gla:
        a = np.exp(-np.log1p(np.exp(rng.standard_normal((B, T, H, d)) - 2.0)))
    else:
        a = np.exp(-np.log1p(np.exp(rng.standard_normal((B, T, H)) - 2.0)))
    return q, k, v, a, b


# ---------------------------------------------------------------- index sets

@pytest.mark.parametrize("n_sink,window", [(8, 56), (8, 120), (8, 888), (0, 1), (3, 5), (1, 1), (5, 2)])
def test_partition_bruteforce(n_sink, window):
    """A(t) and L(t) are disjoint, cover {0..t}, and |A(t)| = min(t+1, budget)."""
    N = n_sink + window
    for t in range(0, 4 * N + 3):
        A = set(O.softmax_index_set(t, n_sink, window).tolist())
        L = set(O.linear_index_set(t, n_sink, window).tolist())
        assert A.isdisjoint(L)
        assert A | L == set(range(t + 1))
        assert len(A) == min(t + 1, N)
        for i in range(t + 1):
            assert O.in_softmax_set(t, i, n_sink, window) == (i in A)
            assert O.in_linear_set(t, i, n_sink, window) == (i in L)
        # sinks are exactly the first n_sink tokens, always attended
        assert set(range(min(n_sink, t + 1))) <= A
        # the window is the last `window` tokens, current token included
        assert set(range(max(0, t - window + 1), t + 1)) <= A


def test_softmax_probe_recovers_index_sets():
    """q = 0 makes softmax uniform; one-hot v then reveals each A(t) exactly."""
    n_sink, window, T = 3, 5, 40
    B, H, d = 1, 1, T
    q = np.zeros((B, T, H, d))
    k = RNG.standard_normal((B, T, H, d))
    v = np.eye(T)[None, :, None, :]                 # v_i = e_i
    o = O.swa_branch(q, k, v, n_sink, window)
    for t in range(T):
        A = O.softmax_index_set(t, n_sink, window)
        got = np.nonzero(np.abs(o[0, t, 0]) > 1e-12)[0]
        assert got.tolist() == A.tolist()
        assert np.allclose(o[0, t, 0, A], 1.0 / len(A), atol=1e-15)


def test_linear_probe_recovers_index_sets():
    """With a = b = 1 and orthonormal keys that never repeat, o_lin[t] read
    with q = sum of all keys is the sum of v_i over exactly L(t)."""
    n_sink, window, T = 3, 5, 30
    d = T
    k = np.eye(T)[None, :, None, :]                 # k_i = e_i
    v = np.eye(T)[None, :, None, :]                 # v_i = e_i marks token i
    q = np.ones((1, T, 1, d))
    a = np.ones((1, T, 1))
    b = np.ones((1, T, 1))
    o, _ = O.gdn_linear_branch(q, k, v, a, b, n_sink, window)
    for t in range(T):
        L = O.linear_index_set(t, n_sink, window)
        got = np.nonzero(np.abs(o[0, t, 0]) > 1e-12)[0]
        assert got.tolist() == L.tolist()
        assert np.allclose(o[0, t, 0, L], 1.0, atol=1e-14)


# ------------------------------------------------- check 1: effective form

@pytest.mark.parametrize("n_sink,window,T,d", [(2, 3, 24, 6), (0, 1, 20, 5), (4, 4, 30, 8)])
def test_gdn_matches_materialised_effective_attention(n_sink, window, T, d):
    """o_lin[t] = sum_{i in L(t)} b_i [q_t^T A_e ... A_{i+1} k_i] v_i with
    A_j = a_j (I - b_j k_j k_j^T), e = t - window, newest factor on the left."""
    B, H = 2, 2
    q, k, v, a, b = rand_layer(B, T, H, H, d)
    o, S = O.gdn_linear_branch(q, k, v, a, b, n_sink, window)
    ref = np.zeros_like(o)
    for bi in range(B):
        for h in range(H):
            for t in range(T):
                e = t - window
                M = np.eye(d)                      # A_e ... A_{i+1}
                for i in range(e, n_sink - 1, -1):
                    coef = b[bi, i, h] * (q[bi, t, h] @ M @ k[bi, i, h])
                    ref[bi, t, h] += coef * v[bi, i, h]
                    Ai = a[bi, i, h] * (np.eye(d) - b[bi, i, h] * np.outer(k[bi, i, h], k[bi, i, h]))
                    M = M @ Ai
    np.testing.assert_allclose(o, ref, atol=1e-13, rtol=0)


def test_gla_matches_diagonal_product_form():
    """GLA: o_lin[t] = sum_{i in L(t)} [q_t^T Diag(prod_{j=i+1}^{e} alpha_j) k_i] v_i."""
    n_sink, window, T, d, B, H = 2, 3, 25, 6, 1, 2
    q, k, v, a, b = rand_layer(B, T, H, H, d, gla=True)
    o, _ = O.gla_linear_branch(q, k, v, a, n_sink, window)
    ref = np.zeros_like(o)
    for h in range(H):
        for t in range(T):
            e = t - window
            for i in range(n_sink, e + 1):
                decay = np.prod(a[0, i + 1:e + 1, h], axis=0) if e > i else np.ones(d)
                ref[0, t, h] += (q[0, t, h] * decay) @ k[0, i, h] * v[0, i, h]
    np.testing.assert_allclose(o, ref, atol=1e-13, rtol=0)


# ------------------------------------------- check 2: exact retrieval

def test_orthonormal_retrieval_a1_b1():
    """Orthonormal keys with repeats, a = b = 1: querying with e_c returns the
    latest v_i with k_i = e_c among i in L(t), or 0."""
    n_sink, window, T, d = 2, 3, 60, 4
    rng = np.random.default_rng(7)
    basis = rng.integers(0, d, size=T)
    k = np.eye(d)[basis][None, :, None, :]
    v = rng.standard_normal((1, T, 1, 5))
    qc = rng.integers(0, d, size=T)
    q = np.eye(d)[qc][None, :, None, :]
    a = np.ones((1, T, 1))
    b = np.ones((1, T, 1))
    o, _ = O.gdn_linear_branch(q, k, v, a, b, n_sink, window)
    for t in range(T):
        cand = [i for i in range(n_sink, t - window + 1) if basis[i] == qc[t]]
        want = v[0, cand[-1], 0] if cand else np.zeros(5)
        np.testing.assert_allclose(o[0, t, 0], want, atol=1e-14, rtol=0)


def test_orthonormal_retrieval_constant_decay():
    """Same with constant a < 1: the retrieved value decays as a^(e(t) - i)."""
    n_sink, window, T, d, alpha = 1, 2, 40, 3, 0.9
    rng = np.random.default_rng(8)
    basis = rng.integers(0, d, size=T)
    k = np.eye(d)[basis][None, :, None, :]
    v = rng.standard_normal((1, T, 1, 4))
    qc = rng.integers(0, d, size=T)
    q = np.eye(d)[qc][None, :, None, :]
    a = np.full((1, T, 1), alpha)
    b = np.ones((1, T, 1))
    o, _ = O.gdn_linear_branch(q, k, v, a, b, n_sink, window)
    for t in range(T):
        e = t - window
        cand = [i for i in range(n_sink, e + 1) if basis[i] == qc[t]]
        want = alpha ** (e - cand[-1]) * v[0, cand[-1], 0] if cand else np.zeros(4)
        np.testing.assert_allclose(o[0, t, 0], want, atol=1e-14, rtol=0)


def test_single_token_and_zero_beta():
    """One folded token gives b (q.k) v (state starts at zero, so a drops out);
    b = 0 everywhere gives a zero linear branch."""
    n_sink, window, d = 1, 2, 5
    T = n_sink + window + 1          # exactly one token (index n_sink) folded
    q, k, v, a, b = rand_layer(1, T, 1, 1, d)
    o, S = O.gdn_linear_branch(q, k, v, a, b, n_sink, window)
    t = T - 1
    i = n_sink
    want = b[0, i, 0] * (q[0, t, 0] @ k[0, i, 0]) * v[0, i, 0]
    np.testing.assert_allclose(o[0, t, 0], want, atol=1e-15)
    np.testing.assert_allclose(S[0, 0], b[0, i, 0] * np.outer(k[0, i, 0], v[0, i, 0]), atol=1e-15)
    q, k, v, a, b = rand_layer(1, 30, 2, 2, d)
    o, S = O.gdn_linear_branch(q, k, v, a, np.zeros_like(b), n_sink, window)
    assert np.all(o == 0) and np.all(S == 0)


# -------------------------------- check 3: equals full causal softmax

def _sdpa(q, k, v, mask=None, causal=False):
    H = q.shape[2]
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(0, 2, 1, 3)))
    tk = torch.from_numpy(np.ascontiguousarray(np.repeat(k, H // k.shape[2], axis=2).transpose(0, 2, 1, 3)))
    tv = torch.from_numpy(np.ascontiguousarray(np.repeat(v, H // v.shape[2], axis=2).transpose(0, 2, 1, 3)))
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal)
    return o.numpy().transpose(0, 2, 1, 3)


@pytest.mark.parametrize("T", [1, 7, 63, 64])
def test_hybrid_equals_full_causal_softmax_when_T_le_budget(T):
    """For T <= n_sink + window every key is in A(t): the layer is exactly
    full causal softmax attention (torch SDPA, fp64) and the linear branch is 0."""
    n_sink, window, B, H, Hkv, d = 8, 56, 2, 4, 2, 16
    q, k, v, a, b = rand_layer(B, T, H, Hkv, d)
    o, S = O.hybrid_prefill(q, k, v, a, b, n_sink, window)
    ref = _sdpa(q, k, v, causal=True)
    np.testing.assert_allclose(o, ref, atol=1e-13, rtol=0)
    assert np.all(S == 0)


def test_softmax_branch_equals_sdpa_with_budget_mask():
    """For T > budget the softmax branch equals SDPA under the boolean mask of
    A(t) (library routine vs the oracle's explicit per-row index lists)."""
    n_sink, window, T, B, H, Hkv, d = 3, 6, 50, 1, 4, 1, 8
    q, k, v, a, b = rand_layer(B, T, H, Hkv, d)
    o = O.swa_branch(q, k, v, n_sink, window)
    mask = np.zeros((T, T), bool)
    for t in range(T):
        mask[t, O.softmax_index_set(t, n_sink, window)] = True
    ref = _sdpa(q, k, v, mask=mask)
    np.testing.assert_allclose(o, ref, atol=1e-13, rtol=0)


def test_degenerate_window1_nosink():
    """n_sink = 0, window = 1: softmax sees only the current token (o_swa = v_t)
    and the linear state holds tokens 0..t-1."""
    T, d = 12, 4
    q, k, v, a, b = rand_layer(1, T, 1, 1, d)
    o = O.swa_branch(q, k, v, 0, 1)
    np.testing.assert_allclose(o, v, atol=1e-15)
    o_lin, _ = O.gdn_linear_branch(q, k, v, a, b, 0, 1)
    assert np.all(o_lin[0, 0] == 0)
    # second row: exactly token 0 folded
    want = b[0, 0, 0] * (q[0, 1, 0] @ k[0, 0, 0]) * v[0, 0, 0]
    np.testing.assert_allclose(o_lin[0, 1, 0], want, atol=1e-15)


# ------------------------------------- check 4: chunked (WY/UT) form

def chunked_gdn(q, k, v, a, b, n_sink, window, C):
    """fp64 chunked form: within a chunk with incoming state S0,
    (I + L) U = diag(b) V - diag(b gamma) K S0, L_rs = b_r gamma_r/gamma_s k_r.k_s (s < r),
    O = diag(gamma) Q S0 + (M o Q K^T) U with M_rs = gamma_r/gamma_s (s <= r),
    S_C = gamma_C S0 + (diag(gamma_C/gamma) K)^T U; Q are the lag-shifted queries."""
    B, T, H, dk = q.shape
    G = H // k.shape[2]
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    Sf = np.zeros((B, H, dk, dv))
    for bi in range(B):
        for h in range(H):
            g = h // G
            S = np.zeros((dk, dv))
            for c0 in range(n_sink, T - window, C):
                c1 = min(c0 + C, T - window)
                K = k[bi, c0:c1, g]
                V = v[bi, c0:c1, g]
                Q = q[bi, c0 + window:c1 + window, h]
                bb = b[bi, c0:c1, h]
                gam = np.exp(np.cumsum(np.log(a[bi, c0:c1, h])))
                ratio = gam[:, None] / gam[None, :]
                L = np.tril(bb[:, None] * ratio * (K @ K.T), -1)
                Tm = np.linalg.inv(np.eye(len(bb)) + L)
                Wm = Tm @ ((bb * gam)[:, None] * K)
                Ut = Tm @ (bb[:, None] * V)
                U = Ut - Wm @ S
                o[bi, c0 + window:c1 + window, h] = gam[:, None] * (Q @ S) + (np.tril(ratio) * (Q @ K.T)) @ U
                Kt = (gam[-1] / gam)[:, None] * K
                S_next = gam[-1] * S + Kt.T @ U
                # the chunk is an affine map S -> (gamma_C I - Kt^T Wm) S + Kt^T Ut
                np.testing.assert_allclose(S_next, (gam[-1] * np.eye(dk) - Kt.T @ Wm) @ S + Kt.T @ Ut,
                                           atol=1e-12)
                S = S_next
            Sf[bi, h] = S
    return o, Sf


def segmented_gdn(q, k, v, a, b, n_sink, window, C, P):
    """fp64 segmented chunk scan: the stream's chunks split into P segments.
    Phase 1 (independent per segment): run the chunk form from a zero state
    on V, giving local outputs and the segment's end state N_s, and on the
    augmented value columns [0 | I] (initial state I, V = 0), giving the
    segment's state map M_s = prod M_c and, as outputs, every row's
    q_hat = P_t^T q_t (P_t: the map from the segment's start to the row's
    state).  Phase 2: S_in(s+1) = M_s S_in(s) + N_s.  Phase 3:
    o_t = o_local_t + S_in(s)^T q_hat_t."""
    B, T, H, dk = q.shape
    G = H // k.shape[2]
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    Sf = np.zeros((B, H, dk, dv))
    starts = list(range(n_sink, T - window, C))
    per = -(-len(starts) // P) if starts else 0
    for bi in range(B):
        for h in range(H):
            g = h // G
            segs = []
            for s0 in range(0, len(starts), per):
                S = np.zeros((dk, dv))
                Pm = np.eye(dk)
                rows = []
                for c0 in starts[s0:s0 + per]:
                    c1 = min(c0 + C, T - window)
                    K = k[bi, c0:c1, g]
                    V = v[bi, c0:c1, g]
                    Q = q[bi, c0 + window:c1 + window, h]
                    bb = b[bi, c0:c1, h]
                    gam = np.exp(np.cumsum(np.log(a[bi, c0:c1, h])))
                    ratio = gam[:, None] / gam[None, :]
                    L = np.tril(bb[:, None] * ratio * (K @ K.T), -1)
                    Tm = np.linalg.inv(np.eye(len(bb)) + L)
                    Wm = Tm @ ((bb * gam)[:, None] * K)
                    Ut = Tm @ (bb[:, None] * V)
                    Aq = np.tril(ratio) * (Q @ K.T)
                    Kt = (gam[-1] / gam)[:, None] * K
                    U = Ut - Wm @ S
                    UP = -Wm @ Pm
                    rows.append((c0 + window, c1 + window,
                                 gam[:, None] * (Q @ S) + Aq @ U,        # o_local
                                 gam[:, None] * (Q @ Pm) + Aq @ UP))     # q_hat rows
                    S = gam[-1] * S + Kt.T @ U
                    Pm = gam[-1] * Pm + Kt.T @ UP
                segs.append((S, Pm, rows))
            S_in = np.zeros((dk, dv))
            for N_s, M_s, rows in segs:
                for r0, r1, o_loc, q_hat in rows:
                    o[bi, r0:r1, h] = o_loc + q_hat @ S_in
                S_in = M_s @ S_in + N_s
            Sf[bi, h] = S_in
    return o, Sf


@pytest.mark.parametrize("C,P", [(16, 1), (16, 3), (16, 8), (7, 5), (64, 2)])
def test_segmented_chunk_scan_matches_stepwise(C, P):
    """Segment composition (affine maps M_s, N_s per segment, a P-step carry
    and a per-row fix-up through q_hat) reproduces the stepwise outputs and
    final state."""
    n_sink, window, T, B, H, Hkv, d = 4, 12, 190, 1, 2, 1, 8
    q, k, v, a, b = rand_layer(B, T, H, Hkv, d)
    o, S = O.gdn_linear_branch(q, k, v, a, b, n_sink, window)
    os_, Ss = segmented_gdn(q, k, v, a, b, n_sink, window, C, P)
    np.testing.assert_allclose(os_, o, atol=1e-11, rtol=0)
    np.testing.assert_allclose(Ss, S, atol=1e-11, rtol=0)


@pytest.mark.parametrize("C", [64, 16, 7])
def test_chunked_form_matches_stepwise(C):
    n_sink, window, T, B, H, Hkv, d = 4, 12, 173, 1, 4, 2, 8
    q, k, v, a, b = rand_layer(B, T, H, Hkv, d)
    o, S = O.gdn_linear_branch(q, k, v, a, b, n_sink, window)
    oc, Sc = chunked_gdn(q, k, v, a, b, n_sink, window, C)
    np.testing.assert_allclose(oc, o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(Sc, S, atol=1e-12, rtol=0)


# ------------------------- delta rule with a diagonal (per-channel) gate

def test_dgd_channel_uniform_gate_equals_scalar_gate_gdn():
    """alpha_i = a_i in every channel: Diag(alpha_i) = a_i I, so the
    diagonal-gate delta rule is the scalar-gate one."""
    n_sink, window, T, B, H, Hkv, d = 3, 4, 41, 2, 4, 2, 8
    q, k, v, a, b = rand_layer(B, T, H, Hkv, d)
    alpha = np.repeat(a[..., None], d, axis=-1)
    o1, S1 = O.dgd_linear_branch(q, k, v, alpha, b, n_sink, window)
    o2, S2 = O.gdn_linear_branch(q, k, v, a, b, n_sink, window)
    np.testing.assert_allclose(o1, o2, atol=1e-13, rtol=0)
    np.testing.assert_allclose(S1, S2, atol=1e-13, rtol=0)


def test_dgd_one_hot_keys_closed_form():
    """k_i = e_{c_i} (channels may repeat): the projection touches row c_i
    only, so each row of S follows its own scalar recursion:
    every row decays by its channel's gate, then row c_i <- (1 - b_i) row +
    b_i v_i.  The readout is S^T q at lag ``window``."""
    n_sink, window, T, d, dv = 2, 3, 30, 6, 5
    rng = np.random.default_rng(11)
    ch = rng.integers(0, d, T)
    k = np.eye(d)[ch][None, :, None, :]
    v = rng.standard_normal((1, T, 1, dv))
    q = rng.standard_normal((1, T, 1, d))
    alpha = rng.uniform(0.3, 1.0, (1, T, 1, d))
    b = rng.uniform(0.0, 1.0, (1, T, 1))
    o, S = O.dgd_linear_branch(q, k, v, alpha, b, n_sink, window)
    R = np.zeros((d, dv))
    o_ref = np.zeros((T, dv))
    for i in range(n_sink, T - window):
        R = alpha[0, i, 0][:, None] * R
        c = ch[i]
        R[c] = (1 - b[0, i, 0]) * R[c] + b[0, i, 0] * v[0, i, 0]
        o_ref[i + window] = R.T @ q[0, i + window, 0]
    np.testing.assert_allclose(S[0, 0], R, atol=1e-14, rtol=0)
    np.testing.assert_allclose(o[0, :, 0], o_ref, atol=1e-14, rtol=0)


def chunked_dgd(q, k, v, alpha, b, n_sink, window, C):
    """fp64 chunked form with per-channel decays: in a chunk with incoming
    state S0 and Gam_r = prod_{s <= r} alpha_s (per channel),
    (I + L) U = diag(b) (V - (K o Gam) S0), L_rs = b_r (k_r o Gam_r).(k_s / Gam_s) (s < r),
    O = (Q o Gam) S0 + ([s <= r] (Q o Gam)(K / Gam)^T) U,
    S_C = Diag(Gam_C) S0 + (K o Gam_C / Gam)^T U."""
    B, T, H, dk = q.shape
    G = H // k.shape[2]
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    Sf = np.zeros((B, H, dk, dv))
    for bi in range(B):
        for h in range(H):
            g = h // G
            S = np.zeros((dk, dv))
            for c0 in range(n_sink, T - window, C):
                c1 = min(c0 + C, T - window)
                K = k[bi, c0:c1, g]
                V = v[bi, c0:c1, g]
                Q = q[bi, c0 + window:c1 + window, h]
                bb = b[bi, c0:c1, h]
                Gam = np.cumprod(alpha[bi, c0:c1, h], axis=0)       # [C, dk]
                Kg, Kd = K * Gam, K / Gam
                L = np.tril(bb[:, None] * (Kg @ Kd.T), -1)
                Tm = np.linalg.inv(np.eye(len(bb)) + L)
                Wm = Tm @ (bb[:, None] * Kg)
                Ut = Tm @ (bb[:, None] * V)
                U = Ut - Wm @ S
                Qg = Q * Gam
                o[bi, c0 + window:c1 + window, h] = Qg @ S + np.tril(Qg @ Kd.T) @ U
                S = Gam[-1][:, None] * S + (K * (Gam[-1] / Gam)).T @ U
            Sf[bi, h] = S
    return o, Sf


@pytest.mark.parametrize("C", [64, 16, 7])
def test_dgd_chunked_form_matches_stepwise(C):
    n_sink, window, T, B, H, Hkv, d = 4, 12, 173, 1, 4, 2, 8
    q, k, v, a, b = rand_layer(B, T, H, Hkv, d, gla=True)
    o, S = O.dgd_linear_branch(q, k, v, a, b, n_sink, window)
    oc, Sc = chunked_dgd(q, k, v, a, b, n_sink, window, C)
    np.testing.assert_allclose(oc, o, atol=1e-11, rtol=0)
    np.testing.assert_allclose(Sc, S, atol=1e-11, rtol=0)


def test_gla_alpha1_equals_gdn_a1_b1_on_fresh_orthonormal_keys():
    """With orthonormal keys that never repeat, the delta projection removes
    nothing, so GLA (alpha = 1) and GDN (a = b = 1) coincide."""
    n_sink, window, T, d = 2, 3, 20, 20
    rng = np.random.default_rng(3)
    perm = rng.permutation(d)
    k = np.eye(d)[perm[:T]][None, :, None, :]
    v = rng.standard_normal((1, T, 1, 6))
    q = rng.standard_normal((1, T, 1, d))
    o1, S1 = O.gla_linear_branch(q, k, v, np.ones((1, T, 1, d)), n_sink, window)
    o2, S2 = O.gdn_linear_branch(q, k, v, np.ones((1, T, 1)), np.ones((1, T, 1)), n_sink, window)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(S1, S2, atol=1e-14)


# ---------------------------------------------- invariants of the layer

def test_gqa_equals_repeated_kv():
    n_sink, window, T, B, H, Hkv, d = 2, 5, 33, 2, 6, 2, 8
    q, k, v, a, b = rand_layer(B, T, H, Hkv, d)
    o1, S1 = O.hybrid_prefill(q, k, v, a, b, n_sink, window)
    kr = torch.from_numpy(k).repeat_interleave(H // Hkv, dim=2).numpy()
    vr = torch.from_numpy(v).repeat_interleave(H // Hkv, dim=2).numpy()
    o2, S2 = O.hybrid_prefill(q, kr, vr, a, b, n_sink, window)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def test_linear_in_v():
    n_sink, window, T, B, H, d = 2, 5, 40, 1, 2, 8
    q, k, v, a, b = rand_layer(B, T, H, H, d)
    for update, aa in (("gdn", a), ("gla", rand_layer(B, T, H, H, d, gla=True)[3])):
        o1, S1 = O.hybrid_prefill(q, k, v, aa, b, n_sink, window, update=update)
        o2, S2 = O.hybrid_prefill(q, k, 4.0 * v, aa, b, n_sink, window, update=update)
        np.testing.assert_array_equal(4.0 * o1, o2)
        np.testing.assert_array_equal(4.0 * S1, S2)


# ------------------------------------------- decode: lag and ring cache

@pytest.mark.parametrize("update", ["gdn", "gla", "dgd"])
@pytest.mark.parametrize("T0", [1, 3, 7, 8, 9, 10, 29])
def test_prefill_then_decode_equals_longer_prefill(update, T0):
    """prefill(T0) + n decode steps reproduces prefill(T0 + n): outputs, final
    state and cache contents (budget 8 = 3 sinks + 5 window)."""
    n_sink, window, n, B, H, Hkv, d = 3, 5, 14, 2, 4, 2, 6
    T = T0 + n
    q, k, v, a, b = rand_layer(B, T, H, Hkv, d, gla=(update != "gdn"))
    o_full, S_full = O.hybrid_prefill(q, k, v, a, b, n_sink, window, update=update)
    _, S = O.hybrid_prefill(q[:, :T0], k[:, :T0], v[:, :T0], a[:, :T0], b[:, :T0],
                            n_sink, window, update=update)
    kc, vc, ac, bc = O.cache_from_prefill(k[:, :T0], v[:, :T0], a[:, :T0], b[:, :T0],
                                          n_sink, window, update=update)
    pos = np.full(B, T0)
    for t in range(T0, T):
        o, S, kc, vc, ac, bc, pos = O.decode_step(q[:, t], k[:, t], v[:, t], a[:, t], b[:, t], S,
                                                  kc, vc, ac, bc, pos, n_sink, window, update=update)
        np.testing.assert_allclose(o, o_full[:, t], atol=1e-13, rtol=0)
    assert np.all(pos == T)
    np.testing.assert_allclose(S, S_full, atol=1e-13, rtol=0)
    kc2, vc2, ac2, bc2 = O.cache_from_prefill(k, v, a, b, n_sink, window, update=update)
    np.testing.assert_array_equal(kc, kc2)
    np.testing.assert_array_equal(vc, vc2)
    np.testing.assert_array_equal(ac, ac2)
    np.testing.assert_array_equal(bc, bc2)


# ------------------------------------------------------------ short conv

def test_causal_conv_matches_torch_conv1d():
    B, T, H, d, ks = 2, 37, 3, 4, 8
    x = RNG.standard_normal((B, T, H, d))
    w = RNG.standard_normal((H * d, ks))
    y = O.causal_depthwise_conv(x, w)
    xt = torch.from_numpy(x.reshape(B, T, H * d)).permute(0, 2, 1)
    yt = torch.nn.functional.conv1d(xt, torch.from_numpy(w)[:, None, :], padding=ks - 1, groups=H * d)
    ref = yt[:, :, :T].permute(0, 2, 1).reshape(B, T, H, d).numpy()
    np.testing.assert_allclose(y, ref, atol=1e-13, rtol=0)


def test_conv_identity_tap():
    x = RNG.standard_normal((1, 9, 2, 4))
    w = np.zeros((8, 8))
    w[:, 7] = 1.0
    np.testing.assert_array_equal(O.causal_depthwise_conv(x, w), x)
    w = np.zeros((8, 8))
    w[:, 6] = 1.0                                    # one-token delay
    y = O.causal_depthwise_conv(x, w)
    np.testing.assert_array_equal(y[:, 1:], x[:, :-1])
    assert np.all(y[:, 0] == 0)


def test_rope_closed_form_and_invariants():
    d, theta = 8, 10000.0
    T = 20
    e0 = np.zeros((1, T, 1, d))
    e0[..., 0] = 1.0
    r = O.rope(e0, theta, pos0=3)
    p = 3 + np.arange(T)
    np.testing.assert_allclose(r[0, :, 0, 0], np.cos(p), atol=1e-15)
    np.testing.assert_allclose(r[0, :, 0, d // 2], np.sin(p), atol=1e-15)
    # the last pair rotates with inv_freq theta^(-2(d/2-1)/d)
    e = np.zeros((1, T, 1, d))
    e[..., d // 2 - 1] = 1.0
    f = theta ** (-2.0 * (d // 2 - 1) / d)
    np.testing.assert_allclose(O.rope(e, theta)[0, :, 0, d - 1], np.sin(np.arange(T) * f), atol=1e-15)
    x = RNG.standard_normal((2, T, 3, d))
    y = RNG.standard_normal((2, T, 3, d))
    rx = O.rope(x, theta)
    np.testing.assert_allclose(np.linalg.norm(rx, axis=-1), np.linalg.norm(x, axis=-1), atol=1e-13)
    # <R_m u, R_n w> depends only on m - n
    u = np.broadcast_to(x[:, :1], x.shape)
    w = np.broadcast_to(y[:, :1], y.shape)
    ru, rw = O.rope(u, theta), O.rope(w, theta)
    dots = np.einsum("bthd,bthd->bth", ru[:, 5:], rw[:, :-5])
    np.testing.assert_allclose(dots, dots[:, :1].repeat(dots.shape[1], 1), atol=1e-12)


def test_shortconv_pipeline_order_and_norm():
    B, T, H, Hkv, d = 1, 16, 2, 1, 8
    q = RNG.standard_normal((B, T, H, d))
    k = RNG.standard_normal((B, T, Hkv, d))
    v = RNG.standard_normal((B, T, Hkv, d))
    wq = RNG.standard_normal((H * d, 8))
    wk = RNG.standard_normal((Hkv * d, 8))
    wv = RNG.standard_normal((Hkv * d, 8))
    qo, ko, vo = O.shortconv_qkv(q, k, v, wq, wk, wv, 1e6, 0, flags=3)
    np.testing.assert_allclose(np.linalg.norm(qo, axis=-1), 1.0, atol=1e-6)
    np.testing.assert_allclose(np.linalg.norm(ko, axis=-1), 1.0, atol=1e-6)
    np.testing.assert_allclose(vo, O.causal_depthwise_conv(v, wv), atol=0)
    # RoPE comes before the conv: with a one-token-delay tap the output at t is
    # the input of t-1 rotated at position t-1, not at t.
    w_delay = np.zeros((H * d, 8))
    w_delay[:, 6] = 1.0
    qo, _, _ = O.shortconv_qkv(q, k, v, w_delay, wk, wv, 100.0, 0, flags=1)
    np.testing.assert_allclose(qo[:, 1:], O.rope(q, 100.0)[:, :-1], atol=1e-14)


@pytest.mark.parametrize("ks", [1, 2, 8])
@pytest.mark.parametrize("T0", [0, 1, 6, 7, 8, 13])
def test_shortconv_decode_steps_equal_prefill_rows(ks, T0):
    # Decode keeps the last ks-1 rotated inputs in a ring; stepping tokens
    # T0 .. T-1 from the history of a T0-token prefill must give the rows of
    # the T-token prefill (itself pinned to torch conv1d), including the zero
    # history before the sequence start and the RoPE position offset pos0.
    B, T, H, Hkv, d, pos0 = 2, 20, 4, 2, 8, 5
    q = RNG.standard_normal((B, T, H, d))
    k = RNG.standard_normal((B, T, Hkv, d))
    v = RNG.standard_normal((B, T, Hkv, d))
    wq = RNG.standard_normal((H * d, ks))
    wk = RNG.standard_normal((Hkv * d, ks))
    wv = RNG.standard_normal((Hkv * d, ks))
    for flags in (0, 1, 3):
        ref = O.shortconv_qkv(q, k, v, wq, wk, wv, 1e4, pos0, flags=flags)
        hq, hk, hv = O.shortconv_history_from_prefill(q[:, :T0], k[:, :T0], v[:, :T0], ks, 1e4, pos0, flags)
        assert hq.shape == (B, ks - 1, H * d) and hk.shape == (B, ks - 1, Hkv * d)
        for t in range(T0, T):
            out = O.shortconv_decode_step(q[:, t], k[:, t], v[:, t], wq, wk, wv, hq, hk, hv,
                                          np.full(B, t), 1e4, pos0, flags)
            for x, r in zip(out, ref):
                np.testing.assert_allclose(x, r[:, t], rtol=0, atol=1e-12)


def test_shortconv_history_holds_rotated_inputs_at_ring_slots():
    # The history after a prefill is the rotated (pre-conv) input of the last
    # ks-1 tokens, token i at ring index i mod (ks-1): check against RoPE of the
    # whole sequence, and that earlier tokens leave no trace.
    B, T, H, d, ks, pos0 = 1, 11, 2, 8, 8, 3
    x = RNG.standard_normal((B, T, H, d))
    hq, _, hv = O.shortconv_history_from_prefill(x, x, x, ks, 50.0, pos0, flags=1)
    rot = O.rope(x, 50.0, pos0)
    for i in range(T - ks + 1, T):
        np.testing.assert_allclose(hq[0, i % (ks - 1)], rot[0, i].reshape(-1), atol=1e-14)
        np.testing.assert_array_equal(hv[0, i % (ks - 1)], x[0, i].reshape(-1))


@pytest.mark.parametrize("update", ["gdn", "gla", "dgd"])
def test_branch_weights_reduce_to_single_branch_flags(update):
    # Weights (1, 0) and (0, 1) give the single-branch outputs (the softmax
    # branch is pinned to SDPA, the linear branch to closed forms); general
    # weights give their combination, in prefill and in decode.
    B, T, H, Hkv, d, ns, win = 1, 40, 4, 2, 8, 2, 9
    q = unit(RNG.standard_normal((B, T, H, d)))
    k = unit(RNG.standard_normal((B, T, Hkv, d)))
    v = RNG.standard_normal((B, T, Hkv, d))
    a = RNG.uniform(0.8, 1.0, (B, T, H, d) if update != "gdn" else (B, T, H))
    b = RNG.uniform(0.0, 1.0, (B, T, H))
    lin, _ = O.hybrid_prefill(q, k, v, a, b, ns, win, update, flags=O.BRANCH_LINEAR)
    sm, _ = O.hybrid_prefill(q, k, v, a, b, ns, win, update, flags=O.BRANCH_SOFTMAX)
    both = O.BRANCH_LINEAR | O.BRANCH_SOFTMAX
    np.testing.assert_array_equal(O.hybrid_prefill(q, k, v, a, b, ns, win, update, both, 1.0, 0.0)[0], lin)
    np.testing.assert_array_equal(O.hybrid_prefill(q, k, v, a, b, ns, win, update, both, 0.0, 1.0)[0], sm)
    got, _ = O.hybrid_prefill(q, k, v, a, b, ns, win, update, both, 0.25, 1.5)
    np.testing.assert_allclose(got, 0.25 * lin + 1.5 * sm, atol=1e-13)
    # decode: the next token's output with weights from the same caches
    T0 = T - 1
    pre = [x[:, :T0] for x in (q, k, v, a, b)]
    _, S = O.hybrid_prefill(*pre, ns, win, update, flags=O.WRITE_STATE)
    caches = O.cache_from_prefill(pre[1], pre[2], pre[3], pre[4], ns, win, update)
    step = [x[:, T0] for x in (q, k, v, a, b)]
    pos = np.full(B, T0)
    o_w = O.decode_step(*step, S, *caches, pos, ns, win, update, both, 0.25, 1.5)[0]
    np.testing.assert_allclose(o_w, got[:, T0], atol=1e-12)
