"""Pins of the backward oracle against central finite differences of the
forward oracle (fp64), on tiny layers: every input gradient of the loss
sum(do * o) + sum(dS * S_final), for the three recurrences, both branches,
GQA and branch weights.  No GPU."""

import numpy as np
import pytest

from oracle import backward as BW
from oracle import hybrid as O


def loss(q, k, v, a, b, do, dS, ns, win, update, w_lin=1.0, w_swa=1.0):
    o, S = O.hybrid_prefill(q, k, v, a, b, ns, win, update=update, w_lin=w_lin, w_swa=w_swa)
    return float(np.sum(do * o) + np.sum(dS * S))


def fd_grad(f, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + h
        fp = f()
        x[i] = old - h
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


def layer(update, B=1, T=11, H=2, Hkv=1, d=3, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, d)) * 0.7
    k = rng.standard_normal((B, T, Hkv, d)) * 0.7
    v = rng.standard_normal((B, T, Hkv, d))
    shape = (B, T, H, d) if update != "gdn" else (B, T, H)
    a = rng.uniform(0.5, 1.0, shape)
    b = rng.uniform(0.1, 0.9, (B, T, H))
    do = rng.standard_normal((B, T, H, d))
    dS = rng.standard_normal((B, H, d, d))
    return q, k, v, a, b, do, dS


@pytest.mark.parametrize("update", ["gdn", "gla", "dgd"])
@pytest.mark.parametrize("ns,win,H,Hkv,w", [(1, 3, 2, 1, (1.0, 1.0)), (0, 2, 4, 2, (0.7, 1.3)),
                                           (2, 1, 2, 2, (1.0, 0.0))])
def test_backward_matches_finite_differences(update, ns, win, H, Hkv, w):
    q, k, v, a, b, do, dS = layer(update, H=H, Hkv=Hkv, seed=ns + 3 * win + H)
    args = [q, k, v, a, b]
    grads = BW.hybrid_prefill_backward(q, k, v, a, b, ns, win, do, dS, update=update,
                                       w_lin=w[0], w_swa=w[1])
    names = ["q", "k", "v", "a", "b"]
    for name, x, g in zip(names, args, grads):
        if update == "gla" and name == "b":
            assert g is None
            continue
        ref = fd_grad(lambda: loss(*args, do, dS, ns, win, update, *w), x)
        np.testing.assert_allclose(g, ref, atol=2e-7, rtol=1e-6, err_msg=f"{update} d{name}")


def test_backward_gradients_of_untouched_tokens():
    """Tokens that never leave the window carry no gate gradient, and with
    the linear branch weighted 0 only the state output reaches the gates."""
    q, k, v, a, b, do, dS = layer("gdn", T=9)
    ns, win = 1, 3
    _, _, _, da, db = BW.hybrid_prefill_backward(q, k, v, a, b, ns, win, do, dS, update="gdn")
    last = 9 - win          # tokens from here on never leave the window
    assert np.all(da[:, last:] == 0) and np.all(db[:, last:] == 0)
    assert np.all(da[:, :ns] == 0) and np.all(db[:, :ns] == 0)
