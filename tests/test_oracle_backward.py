"""Pins of the oracle's backward (CPU, float64), each independent of its formulas.

The backward follows the exactref.ai "scaled_dot_product_attention.backward"
section.  What fixes it here, without trusting its own arithmetic:
  * central finite differences of the loss sum(grad * out) through the
    (separately pinned) forward oracle, element by element on tiny inputs;
  * torch's autograd through torch.nn.functional.scaled_dot_product_attention
    in float64 on the CPU (the library routine the pages compare against);
  * identities that hold exactly: key gradients sum to zero over the keys of a
    head (softmax is unchanged by a common shift of a row's logits), value
    gradients sum to the summed output gradient of the rows that keep a key, a
    single key or identical keys give a zero query gradient;
  * the special rows the section describes: a row with no kept key contributes
    0, a NaN row makes every gradient it touches NaN.
A mutated copy of the backward (a wrong sign, a dropped D term, a transposed
product, a missing scale) fails the finite-difference pin (checked at the end).
"""
import math

import numpy as np
import pytest
import torch

from oracle import sdpa_oracle as O


def _rand(shape, rng):
    return rng.standard_normal(shape)


def _loss(q, k, v, g, **kw):
    out, _ = O.sdpa(q, k, v, **kw)
    return float((out * g).sum())


def _fd_grads(q, k, v, g, h=1e-6, **kw):
    """Central differences of sum(g * out) with respect to every input element."""
    res = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        x = base[which]
        gr = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            fp = _loss(*base, g, **kw)
            x[idx] = old - h
            fm = _loss(*base, g, **kw)
            x[idx] = old
            gr[idx] = (fp - fm) / (2 * h)
        res.append(gr)
    return res


CASES = [
    dict(),
    dict(is_causal=True),
    dict(scale=0.7),
    dict(is_causal=True, scale=-1.3),
    dict(attn_mask="float"),
    dict(attn_mask="bool", is_causal=True),
    dict(enable_gqa=True),
    dict(enable_gqa=True, is_causal=True, attn_mask="float"),
]


def _inputs(case, seed):
    rng = np.random.default_rng(seed)
    hq, hk = (4, 2) if case.get("enable_gqa") else (2, 2)
    L, S, E, Ev = 3, 5, 4, 3
    q = _rand((1, hq, L, E), rng)
    k = _rand((1, hk, S, E), rng)
    v = _rand((1, hk, S, Ev), rng)
    g = _rand((1, hq, L, Ev), rng)
    kw = dict(case)
    if case.get("attn_mask") == "float":
        m = rng.standard_normal((L, S))
        m[0, 4] = -math.inf
        kw["attn_mask"] = m
    elif case.get("attn_mask") == "bool":
        m = rng.random((hq, L, S)) < 0.7
        m[:, :, 0] = True
        kw["attn_mask"] = m
    return q, k, v, g, kw


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_backward_matches_finite_differences(ci):
    q, k, v, g, kw = _inputs(CASES[ci], seed=100 + ci)
    dq, dk, dv = O.sdpa_backward(q, k, v, g, **kw)
    fq, fk, fv = _fd_grads(q, k, v, g, **kw)
    for a, b, n in ((dq, fq, "q"), (dk, fk, "k"), (dv, fv, "v")):
        assert a.shape == b.shape, n
        assert np.abs(a - b).max() < 1e-7, (n, np.abs(a - b).max())


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_backward_matches_torch_autograd(ci):
    q, k, v, g, kw = _inputs(CASES[ci], seed=200 + ci)
    dq, dk, dv = O.sdpa_backward(q, k, v, g, **kw)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    m = kw.get("attn_mask")
    causal = kw.get("is_causal", False)
    if m is not None and causal:
        # torch takes one or the other: the intersection of both kept sets as one mask
        L, S = q.shape[-2], k.shape[-2]
        tril = np.tril(np.ones((L, S), dtype=bool))
        m = (m & tril) if m.dtype == np.bool_ else m + np.where(tril, 0.0, -np.inf)
        causal = False
    tm = None if m is None else torch.tensor(m)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=tm, is_causal=causal, scale=kw.get("scale"),
        enable_gqa=kw.get("enable_gqa", False))
    out.backward(torch.tensor(g))
    for a, t, n in ((dq, tq, "q"), (dk, tk, "k"), (dv, tv, "v")):
        assert np.abs(a - t.grad.numpy()).max() < 1e-12, n


def test_backward_identities():
    rng = np.random.default_rng(7)
    q, k, v, g = (_rand(s, rng) for s in ((2, 3, 6, 5), (2, 3, 9, 5), (2, 3, 9, 4), (2, 3, 6, 4)))
    for causal in (False, True):
        dq, dk, dv = O.sdpa_backward(q, k, v, g, is_causal=causal)
        # a common shift of a row's logits changes nothing: sum_j dS_ij = 0, so key gradients sum to 0
        assert np.abs(dk.sum(axis=-2)).max() < 1e-12
        # every row keeps a key and its weights sum to 1: value gradients sum to the summed grad
        assert np.abs(dv.sum(axis=-2) - g.sum(axis=-2)).max() < 1e-12
    # one key: its weight is exactly 1, so the query and key gradients vanish and grad_value = sum of grad
    dq, dk, dv = O.sdpa_backward(q, k[:, :, :1], v[:, :, :1], g)
    assert np.abs(dq).max() == 0 and np.abs(dk).max() < 1e-15
    assert np.abs(dv[:, :, 0] - g.sum(axis=-2)).max() < 1e-12
    # identical keys: uniform weights whatever the query, so grad_query is 0
    kk = np.repeat(k[:, :, :1], 9, axis=2)
    dq, _, dv = O.sdpa_backward(q, kk, v, g)
    assert np.abs(dq).max() < 1e-13
    # with uniform weights grad_value is the mean of grad over the queries for every key
    assert np.abs(dv - g.sum(axis=-2, keepdims=True) / 9).max() < 1e-12


def test_backward_special_rows():
    rng = np.random.default_rng(8)
    q, k, v, g = (_rand(s, rng) for s in ((1, 1, 4, 3), (1, 1, 5, 3), (1, 1, 5, 2), (1, 1, 4, 2)))
    m = np.zeros((4, 5))
    m[1, :] = -math.inf                      # row 1 keeps no key: it contributes 0
    dq, dk, dv = O.sdpa_backward(q, k, v, g, attn_mask=m)
    assert (dq[0, 0, 1] == 0).all()
    g2 = g.copy()
    g2[0, 0, 1] = 1e3                        # its output gradient then changes nothing
    _, dk2, dv2 = O.sdpa_backward(q, k, v, g2, attn_mask=m)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)
    qn = q.copy()
    qn[0, 0, 2, 1] = np.nan                  # a NaN row: its gradients and every key it touches are NaN
    dq, dk, dv = O.sdpa_backward(qn, k, v, g)
    assert np.isnan(dq[0, 0, 2]).all() and np.isnan(dk).all() and np.isnan(dv).all()
    assert np.isfinite(dq[0, 0, [0, 1, 3]]).all()


def test_backward_gqa_folds_copies():
    """grad_key/grad_value of a shared head are the sums over its query heads (Backward)."""
    rng = np.random.default_rng(9)
    q, g = _rand((1, 6, 4, 3), rng), _rand((1, 6, 4, 2), rng)
    k, v = _rand((1, 2, 5, 3), rng), _rand((1, 2, 5, 2), rng)
    dq, dk, dv = O.sdpa_backward(q, k, v, g, enable_gqa=True, is_causal=True)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    eq, ek, ev = O.sdpa_backward(q, kr, vr, g, is_causal=True)
    assert np.abs(dq - eq).max() < 1e-14
    assert np.abs(dk - ek.reshape(1, 2, 3, 5, 3).sum(axis=2)).max() < 1e-13
    assert np.abs(dv - ev.reshape(1, 2, 3, 5, 2).sum(axis=2)).max() < 1e-13


def test_finite_difference_pin_catches_planted_mistakes():
    """Planted mistakes in a copy of the backward, each caught by the finite-difference pin."""
    q, k, v, g, kw = _inputs(dict(is_causal=True, scale=0.9), seed=5)
    fq, fk, fv = _fd_grads(q, k, v, g, **kw)

    def mutated(kind):
        p = O.weights(q, k, is_causal=True, scale=0.9)
        dp = g @ np.swapaxes(v, -1, -2)
        d = (p * dp).sum(-1, keepdims=True)
        ds = p * (dp + d) if kind == "sign" else (p * dp if kind == "noD" else p * (dp - d))
        gv = np.swapaxes(p, -1, -2) @ g if kind != "transpose" else p[..., :, :3].swapaxes(-1, -2) @ g
        sc = 1.0 if kind == "noscale" else 0.9
        return sc * ds @ k, sc * np.swapaxes(ds, -1, -2) @ q, gv

    for kind in ("sign", "noD", "noscale", "transpose"):
        mq, mk, mv = mutated(kind)
        err = max(np.abs(mq - fq).max(), np.abs(mk - fk).max(),
                  np.abs(mv - fv).max() if mv.shape == fv.shape else np.inf)
        assert err > 1e-3, kind
