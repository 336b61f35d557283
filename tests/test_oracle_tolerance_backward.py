"""Pins of the backward's per-element tolerance (oracle/tolerance.py, analyse_backward), CPU only.

The exactref.ai "scaled_dot_product_attention.backward" section lists the
roundings its tolerance() budgets (the forward's scores, scale, logits, shift,
exp and row sum; P rounded once; the accumulations of dP, D, grad_value, dS K
and dS^T Q; dP - D, dS and the scale product rounded; the rounding to dtype)
and the ones only named algorithms budget (P without a division by the row
sum, rounding to the input dtype in between, D from the forward output).  The
page prints no backward tolerance value, so the model is fixed here by:
  * soundness: float32 emulations of the page's program (index order, 2 and 4
    lanes; exp off by up to the budgeted steps) lie in the default range, and
    in random orders in the any-order range; a FlashAttention-style emulation
    (P = exp2 of a fused scale-and-shift against the forward's logsumexp, D
    from the forward's output, P and dS rounded to bf16/fp16 before their
    products, sums in random orders, the forward itself the blocked emulation
    the forward pins cover) lies in the BlockedBackward range, both over every
    forward output and logsumexp the forward's model allows and for the ones
    the emulated forward returned, handed over as values (as a backward kernel
    receives them); grouped heads sum over the group's query heads;
  * the exact gradients (the float64 oracle) lie in every range;
  * not vacuous: planted mistakes (D dropped, dP - D with the wrong sign, the
    scale missing from grad_key, dS used untransposed for grad_key, P rounded
    to too few bits) fall outside, the emulations use a visible part of the
    budget, and the ranges stay within stated bounds;
  * rows that keep no key contribute exactly 0, NaN rows give NaN gradients
    that must be matched.
"""
import math

import numpy as np
import pytest

from oracle import sdpa_oracle as O
from oracle import tolerance as T
from test_oracle_tolerance import (LN2, LOG2E, _bias, _inputs, _mask, _perturb, _round_bits, _sum32, _to_fmt,
                                   emulate_blocked)

NAMES = ("grad_query", "grad_key", "grad_value")


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def emulate_page_backward(q, k, v, g, bias, scale, fmt, order="index", ulps=2, seed=0, mistake=None):
    """The page's default backward program in float32 for one head (q (L, E), k (S, E),
    v (S, Ev), g (L, Ev) hold values of ``fmt``; bias (L, S)); returns (grad_query,
    grad_key, grad_value) in fmt as float64.  ``mistake`` plants an error."""
    rng = np.random.default_rng(seed)
    q32, k32, v32, g32 = (_f32(x) for x in (q, k, v, g))
    L, S = q32.shape[0], k32.shape[0]
    c = np.float32(scale)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        s = _sum32(_f32(q32[:, None, :] * k32[None]), 2, order, rng) if q32.shape[1] else np.zeros((L, S), np.float32)
        ell = _f32(s.astype(np.float64) * np.float64(c) + np.asarray(bias, np.float64))
        m = np.max(ell, axis=1)
        m = np.where(np.isneginf(m), np.float32(0), m)
        d = _f32(ell - m[:, None])
        w = _perturb(_f32(np.exp(d.astype(np.float64))), ulps, rng)
        w = _f32(np.where(np.isneginf(ell), np.float32(0), w))
        rs = _sum32(w, 1, order, rng)
        P = _f32(np.where(rs[:, None] > 0, w / np.where(rs > 0, rs, 1)[:, None], 0))
        if mistake == "p_bits":
            P = _round_bits(P, 4)
        dP = _sum32(_f32(g32[:, None, :] * v32[None]), 2, order, rng) if g32.shape[1] else np.zeros((L, S), np.float32)
        D = _sum32(_f32(P * dP), 1, order, rng)
        t = _f32(dP - D[:, None])
        if mistake == "no_d":
            t = dP
        if mistake == "sign":
            t = _f32(D[:, None] - dP)
        dS = _f32(P * t)
        gv = _sum32(_f32(P[:, :, None] * g32[:, None, :]), 0, order, rng)
        gq = _f32(c * _sum32(_f32(dS[:, :, None] * k32[None]), 1, order, rng))
        dSk = dS if mistake == "untransposed" else dS.T
        gk = _sum32(_f32(dSk[:, :, None] * q32[None]), 1, order, rng)
        gk = gk if mistake == "no_scale" else _f32(c * gk)
    return tuple(_to_fmt(x, fmt).astype(np.float64) for x in (gq, gk, gv))


def emulate_flash_backward(q, k, v, g, bias, scale, fmt, o, lse, order="random", seed=0, masked=False, mistake=None):
    """A FlashAttention-style backward in float32 for one head: P = exp2(t) with t the fused
    s * (scale * log2 e) - lse * log2 e (one rounding; with a float mask the rounded logit
    times log2 e instead), D_i = g_i . o_i from the forward's output o, dS = P (dP - D),
    P and dS rounded to ``fmt`` before their products, every sum in a random order.
    ``mistake`` plants an error."""
    rng = np.random.default_rng(seed)
    q32, k32, v32, g32, o32 = (_f32(x) for x in (q, k, v, g, o))
    L, S = q32.shape[0], k32.shape[0]
    lse = np.where(np.isneginf(lse), 0.0, lse)
    lse2 = _f32(_f32(lse) * np.float32(LOG2E))
    c2 = np.float32(scale * LOG2E)
    with np.errstate(invalid="ignore", over="ignore"):
        s = _sum32(_f32(q32[:, None, :] * k32[None]), 2, order, rng) if q32.shape[1] else np.zeros((L, S), np.float32)
        if masked:
            ell = _f32(s.astype(np.float64) * np.float64(np.float32(scale)) + np.asarray(bias, np.float64))
            t = _f32(ell.astype(np.float64) * np.float64(np.float32(LOG2E)) - lse2[:, None])
        else:
            t = _f32(s.astype(np.float64) * np.float64(c2) - lse2[:, None])
        P = _perturb(_f32(np.exp2(t.astype(np.float64))), 1, rng)
        P = _f32(np.where(np.isfinite(bias), P, 0))
        dP = _sum32(_f32(g32[:, None, :] * v32[None]), 2, order, rng)
        D = _sum32(_f32(g32 * o32), 1, order, rng)
        dS = _f32(P * _f32(dP - (0 if mistake == "no_d" else D[:, None])))
        Pi, dSi = _to_fmt(P, fmt), _to_fmt(dS, fmt)
        if mistake == "ds_bits":
            dSi = _round_bits(dS, 5)
        if mistake == "lse_off":    # the logsumexp read one row off
            return emulate_flash_backward(q, k, v, g, bias, scale, fmt, o, np.roll(lse, 1), order, seed, masked)
        gv = _sum32(_f32(Pi[:, :, None] * g32[:, None, :]), 0, order, rng)
        gq = _f32(np.float32(scale) * _sum32(_f32(dSi[:, :, None] * k32[None]), 1, order, rng))
        gk = _f32(np.float32(scale) * _sum32(_f32(dSi.T[:, :, None] * q32[None]), 1, order, rng))
    return tuple(_to_fmt(x, fmt).astype(np.float64) for x in (gq, gk, gv))


def _case(fmt, L, S, E, Ev, seed, heads=2, mask=False, causal=False, scale=None):
    q, k, v = _inputs((heads, L, E), (heads, S, E), (heads, S, Ev), fmt, seed)
    g = _inputs((heads, L, Ev), (1, 1, 1), (1, 1, 1), fmt, seed + 1000)[0]
    m = _mask(L, S, seed) if mask else None
    sc = (1 / math.sqrt(E) if E else 0.0) if scale is None else scale
    return q, k, v, g, m, _bias(L, S, causal, m), sc


def _covered(a, grads, what):
    c = a.covers(**dict(zip(NAMES, grads)))
    for n in NAMES:
        assert c[n].all(), (what, n, np.argwhere(~c[n])[:3])


def _usage(a, grads):
    u = 0.0
    for n, x in zip(NAMES, grads):
        fin = a.tolerance[n] > 0
        if fin.any():
            u = max(u, float((np.abs(x - a.rounded[n])[fin] / a.tolerance[n][fin]).max()))
    return u


PAGE_CASES = [
    dict(fmt="fp32"),
    dict(fmt="fp32", causal=True, scale=-0.4),
    dict(fmt="fp32", mask=True, scale=1.0),
    dict(fmt="bf16", causal=True),
    dict(fmt="fp16", mask=True),
]


@pytest.mark.parametrize("ci", range(len(PAGE_CASES)))
def test_page_backward_program_is_covered(ci):
    """The page's backward program in every normal order (exp off by up to 2 steps) lies in
    the default range, and uses a visible part of it."""
    case = PAGE_CASES[ci]
    fmt = case["fmt"]
    q, k, v, g, m, bias, sc = _case(fmt, 11, 29, 12, 6, 20 + ci, mask=case.get("mask", False),
                                    causal=case.get("causal", False), scale=case.get("scale"))
    a = T.analyse_backward(q, k, v, g, attn_mask=m, is_causal=case.get("causal", False), scale=case.get("scale"),
                           dtype=fmt)
    used = 0.0
    for order in ("index", "lanes2", "lanes4", "lanes4p"):
        for seed in range(2):
            grads = [np.stack(x) for x in zip(*[emulate_page_backward(q[h], k[h], v[h], g[h], bias, sc, fmt, order,
                                                                       2, seed + h) for h in range(2)])]
            _covered(a, grads, (case, order, seed))
            used = max(used, _usage(a, grads))
    _covered(a, [O.sdpa_backward(q, k, v, g, attn_mask=m, is_causal=case.get("causal", False),
                                 scale=case.get("scale"))[i] for i in range(3)], "exact")
    if fmt == "fp32":
        assert used > 0.01, used


def test_backward_any_order_encloses_random_orders_and_the_normal_range():
    for ci, case in enumerate(PAGE_CASES):
        fmt = case["fmt"]
        kw = dict(mask=case.get("mask", False), causal=case.get("causal", False), scale=case.get("scale"))
        q, k, v, g, m, bias, sc = _case(fmt, 9, 23, 10, 5, 40 + ci, **kw)
        akw = dict(attn_mask=m, is_causal=kw["causal"], scale=kw["scale"], dtype=fmt)
        n = T.analyse_backward(q, k, v, g, **akw)
        a = T.analyse_backward(q, k, v, g, standard="any_order", **akw)
        for name in NAMES:
            assert (a.low[name] <= n.low[name]).all() and (a.high[name] >= n.high[name]).all()
        for seed in range(3):
            grads = [np.stack(x) for x in zip(*[emulate_page_backward(q[h], k[h], v[h], g[h], bias, sc, fmt, "random",
                                                                       2, seed + h) for h in range(2)])]
            _covered(a, grads, (ci, seed))


def test_backward_grouped_heads_sum_over_the_group():
    """Four query heads on two key/value heads: grad_key and grad_value of a key/value head
    are one sum over its two query heads' rows (emulated in index order, head-major)."""
    fmt = "fp32"
    q = _inputs((4, 10, 8), (1, 1, 1), (1, 1, 1), fmt, 60)[0]
    _, k, v = _inputs((1, 1, 1), (2, 17, 8), (2, 17, 6), fmt, 61)
    g = _inputs((4, 10, 6), (1, 1, 1), (1, 1, 1), fmt, 62)[0]
    a = T.analyse_backward(q, k, v, g, is_causal=True, enable_gqa=True)
    bias = _bias(10, 17, True, None)
    sc = 1 / math.sqrt(8)
    gq, gk, gv = [], [], []
    for kv in range(2):
        # the two query heads of this key/value head stacked along the rows: one program
        qq = np.concatenate([q[2 * kv], q[2 * kv + 1]])
        gg = np.concatenate([g[2 * kv], g[2 * kv + 1]])
        bb = np.concatenate([bias, bias])
        x = emulate_page_backward(qq, k[kv], v[kv], gg, bb, sc, fmt, "index")
        gq += [x[0][:10], x[0][10:]]
        gk.append(x[1])
        gv.append(x[2])
    _covered(a, [np.stack(gq), np.stack(gk), np.stack(gv)], "gqa")
    ex = O.sdpa_backward(q, k, v, g, is_causal=True, enable_gqa=True)
    _covered(a, ex, "gqa exact")


LAZY = 8 * LN2
FLASH_CASES = [
    dict(fmt="bf16"),
    dict(fmt="bf16", causal=True, lazy=True),
    dict(fmt="bf16", mask=True, scale=-0.3),
    dict(fmt="fp16", causal=True, scale=1.0),
    dict(fmt="fp16", mask=True, causal=True, lazy=True),
]


def _flash(case, seed, L=33, S=90, E=32, Ev=24, given=False, mistake=None):
    """The flash emulation on a case, with the BlockedBackward analysis: over every forward
    output and logsumexp the forward's model allows, or (``given``) for the emulated
    forward's own output and logsumexp, handed over as values."""
    fmt = case["fmt"]
    q, k, v, g, m, bias, sc = _case(fmt, L, S, E, Ev, seed, mask=case.get("mask", False),
                                    causal=case.get("causal", False), scale=case.get("scale"))
    masked = m is not None
    fwd = T.Blocked(block_n=32, shift_slack=LAZY if case.get("lazy") else 0.0,
                    extra_logit_roundings=1 if masked else 0)
    alg = T.BlockedBackward(forward=fwd, extra_logit_roundings=1, extra_lse_roundings=1)
    heads, fo, fl = [], [], []
    for h in range(2):
        o, lse = emulate_blocked(q[h], k[h], v[h], bias, sc, fmt, block=32, lazy=case.get("lazy", False),
                                 seed=seed + h)
        fo.append(o)
        fl.append(lse)
        heads.append(emulate_flash_backward(q[h], k[h], v[h], g[h], bias, sc, fmt, o, lse, seed=seed + h,
                                            masked=masked, mistake=mistake))
    kw = dict(out=np.stack(fo), lse=np.stack(fl)) if given else {}
    a = T.analyse_backward(q, k, v, g, attn_mask=m, is_causal=case.get("causal", False), scale=sc, dtype=fmt,
                           standard="any_order", algorithm=alg, **kw)
    return a, [np.stack(x) for x in zip(*heads)], (q, k, v, g, m, sc)


@pytest.mark.parametrize("ci", range(len(FLASH_CASES)))
@pytest.mark.parametrize("given", [False, True])
def test_flash_backward_is_covered(ci, given):
    for seed in (1, 2):
        a, grads, (q, k, v, g, m, sc) = _flash(FLASH_CASES[ci], 70 + 10 * ci + seed, given=given)
        _covered(a, grads, (FLASH_CASES[ci], seed))
        if not given:   # (with a given forward output, the exact gradients need not be in range)
            _covered(a, O.sdpa_backward(q, k, v, g, attn_mask=m, is_causal=FLASH_CASES[ci].get("causal", False),
                                        scale=sc), "exact")


def test_backward_tolerance_is_not_vacuous():
    """fp32 under the default budget: every tolerance below 2^-14 max|gradient| + 1e-5 (the
    fixed bar the fp32 backward was held to before) and the emulations use a visible part;
    bf16 under BlockedBackward for a given forward output and logsumexp: the emulation
    uses a visible part, and the median tolerance is below half that fixed bar's bf16 form
    (2^-6 max|gradient| + 1e-3) and the largest within 1.5 times it."""
    q, k, v, g, m, bias, sc = _case("fp32", 16, 48, 16, 8, 90, causal=True)
    a = T.analyse_backward(q, k, v, g, is_causal=True)
    for n in NAMES:
        x = np.abs(a.rounded[n])
        assert (a.tolerance[n] <= 2.0 ** -14 * x.max() + 1e-5).all(), n
    grads = [np.stack(x) for x in zip(*[emulate_page_backward(q[h], k[h], v[h], g[h], bias, sc, "fp32")
                                        for h in range(2)])]
    assert _usage(a, grads) > 0.01
    a, grads, _ = _flash(dict(fmt="bf16", causal=True), 91, L=64, S=128, E=64, Ev=64, given=True)
    assert _usage(a, grads) > 0.2
    for n in NAMES:
        bar = 2.0 ** -6 * np.abs(a.rounded[n]).max() + 1e-3
        assert np.median(a.tolerance[n]) < 0.5 * bar and a.tolerance[n].max() < 1.5 * bar, n


@pytest.mark.parametrize("mistake", ["no_d", "sign", "no_scale", "untransposed", "p_bits"])
def test_backward_planted_mistakes_are_not_covered(mistake):
    q, k, v, g, m, bias, sc = _case("fp32", 24, 24, 16, 8, 95, causal=True)
    a = T.analyse_backward(q, k, v, g, is_causal=True)
    grads = [np.stack(x) for x in zip(*[emulate_page_backward(q[h], k[h], v[h], g[h], bias, sc, "fp32",
                                                               mistake=mistake) for h in range(2)])]
    c = a.covers(**dict(zip(NAMES, grads)))
    assert not all(c[n].all() for n in NAMES), mistake


def test_backward_special_rows():
    """A row that keeps no key contributes nothing (its grad_query is exactly 0, and
    grad_key/grad_value are as if it were absent); a NaN in a query makes its row's
    gradients NaN, and every key's grad_key/grad_value NaN too, all matched exactly."""
    q, k, v, g, _, _, _ = _case("bf16", 6, 9, 8, 4, 97)
    m = np.zeros((6, 9))
    m[2] = -np.inf
    a = T.analyse_backward(q, k, v, g, attn_mask=m, dtype="bf16")
    assert (a.low["grad_query"][:, 2] == 0).all() and (a.high["grad_query"][:, 2] == 0).all()
    keep = np.ones(6, bool)
    keep[2] = False
    b = T.analyse_backward(q[:, keep], k, v, g[:, keep], dtype="bf16")
    for n in ("grad_key", "grad_value"):
        assert np.array_equal(a.rounded[n], b.rounded[n])
    qn = q.copy()
    qn[0, 1, 0] = np.nan
    a = T.analyse_backward(qn, k, v, g, dtype="bf16")
    assert np.isnan(a.low["grad_query"][0, 1]).all() and np.isnan(a.low["grad_key"][0]).all()
    ex = O.sdpa_backward(qn, k, v, g)
    c = a.covers(**dict(zip(NAMES, ex)))
    assert all(c[n].all() for n in NAMES)
    bad = ex[1].copy()
    bad[0, 0, 0] = 0.0
    assert not a.covers(grad_key=bad)["grad_key"][0, 0, 0]


def test_backward_ulps_budget_is_monotone():
    q, k, v, g, _, _, _ = _case("fp32", 12, 30, 8, 8, 99)
    a2 = T.analyse_backward(q, k, v, g)
    a8 = T.analyse_backward(q, k, v, g, ulps=8)
    for n in NAMES:
        assert (a8.low[n] <= a2.low[n]).all() and (a8.high[n] >= a2.high[n]).all()
    assert max(a8.tolerance[n].max() - a2.tolerance[n].max() for n in NAMES) > 0


@pytest.mark.parametrize("mistake", ["no_d", "ds_bits", "lse_off"])
def test_flash_backward_planted_mistakes_are_not_covered(mistake):
    """Under the named algorithm, for the forward output and logsumexp it was handed: D
    dropped, dS rounded to 5 significant bits instead of bf16's 8, the logsumexp of the
    wrong row."""
    a, grads, _ = _flash(dict(fmt="bf16", causal=True), 93, L=48, S=64, given=True, mistake=mistake)
    c = a.covers(**dict(zip(NAMES, grads)))
    assert not all(c[n].all() for n in NAMES), mistake


def test_backward_zero_head_dims():
    """E = 0 (the logits are the mask alone; grad_query and grad_key are empty) and Ev = 0
    (grad and grad_value are empty; dP = 0, so every dS is 0)."""
    q, k, v, g, _, bias, _ = _case("fp32", 5, 7, 0, 3, 101, causal=True)
    a = T.analyse_backward(q, k, v, g, is_causal=True)
    assert a.low["grad_query"].shape == (2, 5, 0) and a.low["grad_key"].shape == (2, 7, 0)
    grads = [np.stack(x) for x in zip(*[emulate_page_backward(q[h], k[h], v[h], g[h], bias, 1.0, "fp32")
                                        for h in range(2)])]
    _covered(a, grads, "E=0")
    q, k, v, g, _, bias, sc = _case("bf16", 5, 7, 8, 0, 102)
    a = T.analyse_backward(q, k, v, g, dtype="bf16")
    assert (a.low["grad_query"] == 0).all() and (a.high["grad_query"] == 0).all()
    assert (a.low["grad_key"] == 0).all() and a.low["grad_value"].shape == (2, 7, 0)
    a = T.analyse(q, k, v, dtype="bf16")
    assert a.low.shape == (2, 5, 0) and np.isfinite(a.lse_low).all()
