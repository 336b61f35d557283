"""Pins of the per-element tolerance (oracle/tolerance.py), CPU only.

The tolerance claims to bound |computed - exact| for any float32 implementation
doing the rounding steps of the exactref.ai "scaled_dot_product_attention"
budget (sections "Tolerance options" and "Full specification"), FlashAttention
style.  Fixed here, without trusting its formula:
  * soundness: an independent float32 emulation of the blocked algorithm
    (online softmax over key blocks, exact or lazily raised maximum, weights
    rounded to bf16/fp16 before the value product, a reciprocal of the row sum,
    and a two-way key split merged by logsumexp) is covered at every element,
    over masks, causal, scales (negative, unit) and formats;
  * it is not vacuous: below the fixed 2e-2 bar on unit-normal inputs, and
    within a modest factor of the emulation's actual error;
  * planted mistakes are not covered: weights rounded to too few bits, one
    masked key kept, and the double scaling of the xFormers pages (query
    pre-divided by sqrt(E) and scaled again);
  * the page's examples: PyTorch's float32 output of the seeded causal
    example is covered; in the padding-mask example the element whose keys are
    all padded gets a range that holds the equal-weight answer 1.5 while the
    other element's tolerance is of the order of 1e-6; a larger exp/log ulps
    budget never shrinks the tolerance;
  * special rows (NaN, no kept key) must match exactly.
"""
import math
import random

import numpy as np
import pytest
import torch

from oracle import sdpa_oracle as O
from oracle import tolerance as T

LOG2E = 1.4426950408889634


def _round_bf16(x):
    """float32 -> nearest bfloat16 (ties to even), kept in a float32 array."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32)


def _round_bits(x, bits):
    """float32 -> nearest value with ``bits`` significant bits (planted coarse rounding)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(x == 0, 1.0, np.abs(x))))
    q = 2.0 ** (e - (bits - 1))
    return (np.round(x / q) * q).astype(np.float32)


def _round_fmt(x, fmt):
    if fmt == "bf16":
        return _round_bf16(x)
    if fmt == "fp16":
        return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)
    return np.asarray(x, dtype=np.float32)


def emulate_head(q, k, v, bias, scale, fmt, block=64, lazy=False, split=None, weight_round=None):
    """One head, float32 FlashAttention-style: q (L, E), k (S, E), v (S, Ev) hold
    format values; bias (L, S) float32 (0 / -inf / a float mask) or None.
    Returns (out rounded to fmt, lse) as float32 arrays."""
    if split is not None:   # keys [0, split) and [split, S), merged by logsumexp
        o1, l1 = emulate_head(q, k[:split], v[:split], None if bias is None else bias[:, :split],
                              scale, "fp32", block, lazy, None, weight_round)
        o2, l2 = emulate_head(q, k[split:], v[split:], None if bias is None else bias[:, split:],
                              scale, "fp32", block, lazy, None, weight_round)
        m = np.maximum(l1, l2)
        w1 = np.exp(np.float32(l1 - m)).astype(np.float32)
        w2 = np.exp(np.float32(l2 - m)).astype(np.float32)
        den = (w1 + w2).astype(np.float32)
        out = ((w1[:, None] * o1 + w2[:, None] * o2) / den[:, None]).astype(np.float32)
        lse = (m + np.log(den)).astype(np.float32)
        return _round_fmt(out, fmt), lse
    wr = weight_round or (lambda p: _round_fmt(p, fmt))
    q32, k32, v32 = (np.asarray(x, dtype=np.float32) for x in (q, k, v))
    L, S, Ev = q32.shape[0], k32.shape[0], v32.shape[1]
    sc = np.float32(abs(scale))
    if scale < 0:
        q32 = -q32
    c = np.float32(abs(scale) * LOG2E)
    m = np.full(L, -np.inf, dtype=np.float32)
    lsum = np.zeros(L, dtype=np.float32)
    acc = np.zeros((L, Ev), dtype=np.float32)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        for j0 in range(0, S, block):
            j1 = min(S, j0 + block)
            s = (q32 @ k32[j0:j1].T).astype(np.float32)
            if bias is not None:
                t = ((s * sc).astype(np.float32) + bias[:, j0:j1]).astype(np.float32)
                t = (t * np.float32(LOG2E)).astype(np.float32)
            else:
                t = (s * c).astype(np.float32)
            mx = np.max(t, axis=-1)
            if lazy:
                m_new = np.where(mx > m + 8, mx, m).astype(np.float32)
            else:
                m_new = np.maximum(m, mx)
            shift = np.where(np.isneginf(m_new), np.float32(0), m_new).astype(np.float32)
            alpha = np.where(np.isneginf(m), np.float32(0), np.exp2((m - shift).astype(np.float32))).astype(np.float32)
            p = np.exp2((t - shift[:, None]).astype(np.float32)).astype(np.float32)
            lsum = (lsum * alpha + p.sum(axis=-1, dtype=np.float32)).astype(np.float32)
            acc = (acc * alpha[:, None] + wr(p) @ v32[j0:j1]).astype(np.float32)
            m = m_new
        inv = np.where(lsum == 0, np.float32(0), (np.float32(1) / lsum)).astype(np.float32)
        out = (acc * inv[:, None]).astype(np.float32)
        shift = np.where(np.isneginf(m), np.float32(0), m)
        lse = np.where(lsum == 0, -np.inf, ((shift + np.log2(lsum)).astype(np.float32) * np.float32(math.log(2.0))))
    return _round_fmt(out, fmt), lse.astype(np.float32)


def _inputs(shape_q, shape_k, shape_v, fmt, seed):
    g = torch.Generator().manual_seed(seed)
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[fmt]
    return tuple(torch.randn(s, generator=g).to(dt).double().numpy() for s in (shape_q, shape_k, shape_v))


def _bias(L, S, causal, mask):
    b = np.zeros((L, S))
    if mask is not None:
        b = b + mask
    if causal:
        b = b + O.causal_bias(L, S)
    return b


CASES = [
    dict(fmt="bf16"),
    dict(fmt="bf16", causal=True, lazy=True),
    dict(fmt="bf16", scale=1.0, block=16),
    dict(fmt="bf16", scale=-0.3, causal=True),
    dict(fmt="bf16", mask=True, split=70),
    dict(fmt="fp16", causal=True, lazy=True, split=33),
    dict(fmt="fp16", scale=1.0),
    dict(fmt="fp32", causal=True),
    dict(fmt="fp32", scale=1.0, mask=True, lazy=True),
]


def _run_case(case, seed, E=64, Ev=48, L=37, S=150, weight_round=None, scale_mult=1.0):
    fmt = case["fmt"]
    q, k, v = _inputs((2, L, E), (2, S, E), (2, S, Ev), fmt, seed)
    rng = np.random.default_rng(seed)
    mask = None
    if case.get("mask"):
        mask = rng.standard_normal((L, S)).astype(np.float32).astype(np.float64)
        mask[rng.random((L, S)) < 0.1] = -np.inf
        mask[:, 0] = 0.0
    scale = case.get("scale")
    sc = (1 / math.sqrt(E) if scale is None else scale)
    causal = case.get("causal", False)
    exact_o, exact_l = O.sdpa(q, k, v, attn_mask=mask, is_causal=causal, scale=sc)
    tol_o, tol_l = T.tolerance(q, k, v, attn_mask=mask, is_causal=causal, scale=sc, dtype=fmt)
    bias = _bias(L, S, causal, mask).astype(np.float32)
    emu = [emulate_head(q[h], k[h], v[h], None if (mask is None and not causal) else bias, sc * scale_mult, fmt,
                        block=case.get("block", 64), lazy=case.get("lazy", False), split=case.get("split"),
                        weight_round=weight_round) for h in range(2)]
    eo = np.stack([e[0] for e in emu])
    el = np.stack([e[1] for e in emu])
    return (eo, el), (exact_o, exact_l), (tol_o, tol_l)


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_emulated_algorithm_is_covered(ci):
    for seed in (1, 2):
        (eo, el), (xo, xl), (to, tl) = _run_case(CASES[ci], seed)
        ok_o, ok_l = T.covers(eo, xo, to), T.covers(el, xl, tl)
        assert ok_o.all(), (CASES[ci], np.abs(eo - xo)[~ok_o].max(), to[~ok_o].min())
        assert ok_l.all(), (CASES[ci], np.abs(el - xl)[~ok_l].max())


def test_tolerance_is_not_vacuous():
    """bf16 unit-normal inputs: below the fixed 2e-2 output bar everywhere, and the
    worst element's error uses a visible part of its budget."""
    for case in (dict(fmt="bf16"), dict(fmt="bf16", causal=True)):
        (eo, el), (xo, xl), (to, tl) = _run_case(case, 3, L=64, S=256)
        assert to.max() < 2e-2 and tl.max() < 1e-3
        fin = to > 0
        assert (np.abs(eo - xo)[fin] / to[fin]).max() > 0.1
        assert (np.abs(el - xl) / tl).max() > 1e-3


def test_planted_mistakes_are_not_covered():
    base = dict(fmt="bf16", causal=True)
    # weights rounded to 4 significant bits instead of bf16's 8
    (eo, _), (xo, _), (to, _) = _run_case(base, 4, weight_round=lambda p: _round_bits(p, 4))
    assert not T.covers(eo, xo, to).all()
    # the query pre-divided by sqrt(E) and scaled again (xFormers pages: effective scale 1/E)
    (eo, el), (xo, xl), (to, tl) = _run_case(dict(fmt="bf16"), 5, scale_mult=1 / 8.0)
    assert not T.covers(eo, xo, to).all() and not T.covers(el, xl, tl).all()
    # one key above the diagonal kept in every row (an off-by-one causal limit)
    q, k, v = _inputs((1, 30, 64), (1, 30, 64), (1, 30, 32), "bf16", 6)
    b = O.causal_bias(30, 31)[:, 1:].astype(np.float32)          # keeps j <= i + 1
    eo, el = emulate_head(q[0], k[0], v[0], b, 1 / 8.0, "bf16")
    xo, xl = O.sdpa(q, k, v, is_causal=True)
    to, tl = T.tolerance(q, k, v, is_causal=True, dtype="bf16")
    assert not T.covers(eo[None], xo, to).all() and not T.covers(el[None], xl, tl).all()


def test_checking_pytorch_example_is_covered():
    """exactref.ai "Checking PyTorch": random.Random(0) gauss draws (1, 2, 8, 16),
    causal; PyTorch's float32 result lies within the float32 tolerance."""
    rng = random.Random(0)

    def randn(*shape):
        return torch.tensor([rng.gauss(0, 1) for _ in range(math.prod(shape))]).reshape(shape)

    tq, tk, tv = randn(1, 2, 8, 16), randn(1, 2, 8, 16), randn(1, 2, 8, 16)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    xo, _ = O.sdpa(tq, tk, tv, is_causal=True)
    to, _ = T.tolerance(tq, tk, tv, is_causal=True, dtype="fp32")
    assert T.covers(ref, xo, to).all()
    # the worst-case budget (any order, truncating accumulators) stays within a few
    # times the fixed 1e-5 float32 bar
    assert to.max() < 1e-4


def test_padding_mask_example():
    """exactref.ai "Padding masks": keys hidden by float32's lowest value.  Query 0
    has every key padded: its rounded logits lose the scores and the weights come
    out equal (PyTorch gives 1.5) although the exact value is about 1.119; the
    range of correct outputs holds 1.5.  Query 1 keeps key 0: output 1.0 with a
    tolerance of the order of 1e-6 (the page prints 1.3e-6)."""
    low = float(np.finfo(np.float32).min)
    q = torch.tensor([[[1.0], [0.5]]])
    k = torch.tensor([[[1.0], [-1.0]]])
    v = torch.tensor([[[1.0], [2.0]]])
    mask = torch.tensor([[[low, low], [0.0, low]]])
    xo, _ = O.sdpa(q, k, v, attn_mask=mask)
    # the float64 oracle also loses the scores next to float32's lowest value and
    # gives the equal-weight 1.5 (its documented reading of this case)
    assert xo[0, 0, 0] == 1.5 and xo[0, 1, 0] == 1.0
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    to, _ = T.tolerance(q, k, v, attn_mask=mask.numpy().astype(np.float64), dtype="fp32")
    assert T.covers(ref, xo, to).all()
    lo, hi = T.finite_range(xo, to)
    exact0 = (math.exp(1.0) * 1.0 + math.exp(-1.0) * 2.0) / (math.exp(1.0) + math.exp(-1.0))
    assert abs(exact0 - 1.1192029220221176) < 1e-15   # the page's exact value
    assert lo[0, 0, 0] <= exact0 <= hi[0, 0, 0] and lo[0, 0, 0] <= 1.5 <= hi[0, 0, 0]
    assert 1e-7 < to[0, 1, 0] < 1e-5


def test_ulps_budget_is_monotone():
    q, k, v = _inputs((1, 3, 20, 32), (1, 3, 50, 32), (1, 3, 50, 32), "fp32", 8)
    t2, l2 = T.tolerance(q, k, v, dtype="fp32")
    t8, l8 = T.tolerance(q, k, v, dtype="fp32", ulps=8)
    assert (t8 >= t2).all() and (l8 >= l2).all() and t8.max() > t2.max()


def test_special_rows_need_exact_matches():
    q, k, v = _inputs((1, 4, 16), (1, 6, 16), (1, 6, 8), "bf16", 9)
    q[0, 1, 3] = np.nan
    m = np.zeros((4, 6))
    m[2, :] = -np.inf                         # row 2 keeps nothing
    xo, xl = O.sdpa(q, k, v, attn_mask=m)
    to, tl = T.tolerance(q, k, v, attn_mask=m, dtype="bf16")
    assert (to[0, 1] == 0).all() and (to[0, 2] == 0).all() and tl[0, 1] == 0 and tl[0, 2] == 0
    good = xo.copy()
    assert T.covers(good, xo, to).all() and T.covers(xl, xl, tl).all()
    bad = xo.copy()
    bad[0, 2, 0] = 1e-30                      # an empty row must be exactly 0
    assert not T.covers(bad, xo, to)[0, 2, 0]
    bad = xo.copy()
    bad[0, 1, 0] = 0.0                        # a NaN row must stay NaN
    assert not T.covers(bad, xo, to)[0, 1, 0]
    ll = xl.copy()
    ll[0, 2] = -1e30                          # lse -inf must be matched exactly
    assert not T.covers(ll, xl, tl)[0, 2]
