"""Per-element tolerance of computed attention (an ExactRef-style finite range), float64 host code.

TEST INFRASTRUCTURE ONLY, like sdpa_oracle: only ``tests/``, ``__graft_entry__``
and the benchmark's cpu_baseline leg may import it; the HIP path never does.

What it computes.  The exactref.ai "scaled_dot_product_attention" page
("Tolerance options", "Padding masks", "Full specification") defines, per
output element, the range of values a correct implementation may return
(``finite_range``) and the tolerance, the largest distance from the exact value
correctly rounded to the output format (``rounded``) to either end of that
range.  A correct implementation is one that performs the page's list of
roundings in the page's order; the page names them but prints no formula.  This
module encloses that set by interval arithmetic on the float32 grid (the
compute format for float32, bfloat16 and float16 inputs):

  1. the scale factor: scale (or 1/sqrt(E)) rounded to float32;
  2. the score accumulation: each product q_e k_je rounded, then summed;
  3. one rounding of each logit: scale * s + mask, rounded once;
  4. the shift by the row maximum: l_j - max_j l_j, rounded;
  5. exp within ``ulps`` float32 steps of the correctly rounded value;
  6. the row sum of the weights;
  7. the value accumulation: each product w_j v_je rounded, then summed;
  8. the final division (value sum over row sum), rounded;
  9. the rounding to the output format (none when it is float32);
 10. logsumexp: log of the row sum within ``ulps`` steps, then one rounding of
     the row maximum plus that logarithm.

Reading of "a rounding" (the page leaves it open): the standard model, the
result is the exact result x times (1 + d) with |d| <= u = 2^-24, and the
enclosure of those values is rounded outward to the float32 grid.  A result
whose relative bound reaches past the largest finite float32 is rounded to
nearest instead (the overflow rule then decides it, as for the lowest-float
padding mask, which keeps such rows finite as the page says).  Every listed
step is a rounding even where its exact result happens to be a float32,
except the first term of an accumulation (adding it to the empty sum is
exact).  Sums ("normal accumulation": index order, or 2 or 4 SIMD-style
lanes) take the hull of the enclosures of those orders; ``standard=
"any_order"`` uses the classical bound gamma(n - 1) * sum |t_i| with the
per-step relative bound 3u of an outward-rounded step, which encloses every
order.  With these readings the page's padding-mask example comes out exactly
as printed (tolerance 0.38079822063446045 and 1.3113021850585938e-06, finite
range [1.499998927116394, 1.5000011920928955]); the worked example's largest
tolerances come out 8.1e-6 (ulps=2) and 1.24e-5 (ulps=8) against the page's
5.96e-6 and 1.45e-5 (the tests pin both and state the difference).

Named algorithms (``algorithm=Blocked(...)``): the page budgets for them the
roundings its default omits, and this option adds exactly those: the weights
rounded to the input format before the value product (optionally also in the
row sum the output is divided by), online-softmax rescaling
of the running sums (one rescale per key block after the first, each an exp
within ulps and a rounded product; the exp error cancels between value sum and
row sum in the output but not in the logsumexp), and the output formed with a
reciprocal of the row sum.  Two further allowances exist for the implementation
under test and are off unless given: ``shift_slack`` (the shift may trail the
row maximum by up to that much, natural-log units: the magnitudes the shift
and logarithm roundings see grow by it), ``extra_logit_roundings``,
``extra_shift_roundings`` and ``extra_lse_roundings`` (an exponent formed in
base 2 through a rounded log2 e rounds the logit, or the shifted logit, once or
twice more; a base-2 logarithm scaled by ln 2 rounds the logsumexp once more)
and ``split_size`` (keys cut into contiguous parts of that many whose
normalised outputs and logsumexps are merged through their logsumexps, as
split-KV decoding does).

Rows the page calls special (a NaN or +inf logit, no kept key) and elements
whose exact value is not finite must be matched exactly.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

from .sdpa_oracle import _expand_kv, _f64, _row_classes, logits, resolve_scale, sdpa

__all__ = ["Blocked", "Analysis", "analyse", "tolerance", "finite_range", "covers"]

# Formats: (significant bits p, minimum normal exponent, largest finite value)
FORMATS = {
    "fp32": (24, -126, float(np.finfo(np.float32).max)),
    "bf16": (8, -126, float.fromhex("0x1.fep127")),
    "fp16": (11, -14, 65504.0),
}
_EPS64 = 2.0 ** -51          # bound on numpy's float64 exp/log error, relative


@dataclass(frozen=True)
class Blocked:
    """A blocked online-softmax algorithm (FlashAttention style), with its extra roundings.

    block_n:     keys per block (rescales per row = key blocks - 1)
    round_weights: weights rounded to the input format before the value product
    round_row_sum: the row sum that divides the output adds those rounded weights
                 (the logsumexp still takes the unrounded ones)
    reciprocal:  output = value sum * (1 / row sum)
    Implementation allowances (0 / 1: off):
    shift_slack: the shift may trail the row maximum by this much (natural-log units)
    extra_logit_roundings: further roundings of each logit (an exponent formed in base 2
                 with a rounded log2 e rounds the logit once more)
    extra_shift_roundings: further roundings of each shifted logit
    extra_lse_roundings: further roundings of the logsumexp (a logarithm in base 2
                 scaled by ln 2 afterwards)
    split_size:  keys cut into parts of this many (the last one shorter), merged
                 through their logsumexps (0: no split)
    """
    block_n: int = 64
    round_weights: bool = True
    round_row_sum: bool = False
    reciprocal: bool = True
    shift_slack: float = 0.0
    extra_logit_roundings: int = 0
    extra_shift_roundings: int = 0
    extra_lse_roundings: int = 0
    split_size: int = 0


# ---------------------------------------------------------------- float grids

def _ulp(x, fmt):
    """Spacing of the format's grid at |x| (upward from a binade's start)."""
    p, emin, _ = FORMATS[fmt]
    _, e = np.frexp(np.abs(x))
    e = np.maximum(e - 1, emin)
    return np.ldexp(1.0, e - p + 1)


def _rd(x, fmt):
    """Largest grid value <= x (-inf below the finite range, the largest finite value above it)."""
    x = np.asarray(x, dtype=np.float64)
    _, _, fmax = FORMATS[fmt]
    pos = np.where(x >= 0, x, 0.0)
    neg = np.where(x < 0, -x, 0.0)
    with np.errstate(invalid="ignore", over="ignore"):
        up = _ulp(pos, fmt)
        r_pos = np.floor(pos / up) * up
        un = _ulp(neg, fmt)
        r_neg = -(np.ceil(neg / un) * un)
    r = np.where(x >= 0, r_pos, r_neg)
    r = np.where(r > fmax, fmax, r)
    r = np.where(r < -fmax, -np.inf, r)
    return np.where(np.isfinite(x), r, x)


def _ru(x, fmt):
    return -_rd(-np.asarray(x, dtype=np.float64), fmt)


def _rn(x, fmt):
    """Nearest grid value, ties to even; IEEE overflow past the largest value plus half an ulp."""
    x = np.asarray(x, dtype=np.float64)
    lo, hi = _rd(x, fmt), _ru(x, fmt)
    _, _, fmax = FORMATS[fmt]
    with np.errstate(invalid="ignore"):
        dl, dh = x - lo, hi - x
        even_lo = np.fmod(np.where(np.isfinite(lo), lo / _ulp(lo, fmt), 0.0), 2.0) == 0
        r = np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(even_lo, lo, hi)))
    half = float(_ulp(np.float64(fmax), fmt)) / 2
    r = np.where(x >= fmax + half, np.inf, np.where(x > fmax, fmax, r))
    r = np.where(x <= -(fmax + half), -np.inf, np.where(x < -fmax, -fmax, r))
    return np.where(np.isfinite(x), r, x)


def _steps(x, fmt, k):
    """(k grid steps below x, k grid steps above x) for x on the grid."""
    lo = np.asarray(x, dtype=np.float64)
    hi = lo
    for _ in range(k):
        lo = _rd(np.nextafter(lo, -np.inf), fmt)
        hi = _ru(np.nextafter(hi, np.inf), fmt)
    return lo, hi


# ------------------------------------------ outward float64 arithmetic (exact where it can be)

def _two_sum_err(a, b, s):
    bb = s - a
    return (a - (s - bb)) + (b - bb)


def _split(a):
    c = 134217729.0 * a
    hi = c - (c - a)
    return hi, a - hi


def _two_prod_err(a, b, p):
    ah, al = _split(a)
    bh, bl = _split(b)
    return al * bl - (((p - ah * bh) - al * bh) - ah * bl)


def _fix(s, err, side):
    """Move a float64 result one ulp outward when its exact error points outward."""
    with np.errstate(invalid="ignore"):
        if side < 0:
            return np.where(np.isfinite(s) & (err < 0), np.nextafter(s, -np.inf), s)
        return np.where(np.isfinite(s) & (err > 0), np.nextafter(s, np.inf), s)


def _add(a, b, side):
    with np.errstate(invalid="ignore", over="ignore"):
        s = a + b
        return _fix(s, _two_sum_err(a, b, s), side)


def _mul(a, b, side):
    with np.errstate(invalid="ignore", over="ignore"):
        p = a * b
        return _fix(p, _two_prod_err(a, b, p), side)


def _div(a, b, side):
    """a / b (b > 0) rounded outward in float64."""
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        q = a / b
        p = q * b
        r = (a - p) - _two_prod_err(q, b, p)   # a - q b exactly (a - p is exact: Sterbenz)
        return _fix(q, r, side)


def _iv_add(x, y):
    return _add(x[0], y[0], -1), _add(x[1], y[1], +1)


def _iv_mul(x, y):
    lo = [_mul(x[i], y[j], -1) for i in (0, 1) for j in (0, 1)]
    hi = [_mul(x[i], y[j], +1) for i in (0, 1) for j in (0, 1)]
    return (np.minimum(np.minimum(lo[0], lo[1]), np.minimum(lo[2], lo[3])),
            np.maximum(np.maximum(hi[0], hi[1]), np.maximum(hi[2], hi[3])))


def _iv_div_pos(x, y):
    """x / y for y > 0."""
    lo = [_div(x[i], y[j], -1) for i in (0, 1) for j in (0, 1)]
    hi = [_div(x[i], y[j], +1) for i in (0, 1) for j in (0, 1)]
    return (np.minimum(np.minimum(lo[0], lo[1]), np.minimum(lo[2], lo[3])),
            np.maximum(np.maximum(hi[0], hi[1]), np.maximum(hi[2], hi[3])))


def _gamma(k):
    """Relative bound of k outward-rounded float32 steps (each within 3u: u for the
    rounding, at most one more grid step, 2u, for the outward snap)."""
    t = 3 * k * 2.0 ** -24
    return t / (1 - t)


# ------------------------------------------------------------ the roundings

def _round(x, fmt="fp32", extra=0.0):
    """One rounding (standard model, outward on the grid) of any exact result in [lo, hi].
    ``extra`` adds to the magnitude the relative bound sees (an allowance)."""
    lo, hi = x
    p, _, fmax = FORMATS[fmt]
    u = 2.0 ** -p
    with np.errstate(invalid="ignore", over="ignore"):
        a = _add(lo, -_mul(_add(np.abs(lo), extra, +1), u, +1), -1)
        b = _add(hi, _mul(_add(np.abs(hi), extra, +1), u, +1), +1)
        edge = (a < -fmax) | (b > fmax)
        rlo = np.where(edge, _rn(lo, fmt), _rd(a, fmt))
        rhi = np.where(edge, _rn(hi, fmt), _ru(b, fmt))
        rlo = np.where(np.isinf(lo), lo, rlo)
        rhi = np.where(np.isinf(hi), hi, rhi)
    return rlo, rhi


def _exp_within(d, ulps):
    """exp over [dlo, dhi], each end within ulps float32 steps of its correctly rounded value."""
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        ylo = _rn(np.exp(d[0]) * (1 - _EPS64), "fp32")
        yhi = _rn(np.exp(d[1]) * (1 + _EPS64), "fp32")
    return np.maximum(_steps(ylo, "fp32", ulps)[0], 0.0), _steps(yhi, "fp32", ulps)[1]


def _log_within(x, ulps, extra=0.0):
    """log over [lo, hi] (> 0), each end within ulps float32 steps of its correctly rounded
    value; with ``extra`` the steps are those at magnitude |log| + extra (a logarithm of a
    row sum taken relative to a shift below the row maximum)."""
    with np.errstate(divide="ignore", invalid="ignore"):
        a, b = np.log(x[0]), np.log(x[1])
    ya = _rn(a - np.abs(a) * _EPS64, "fp32")
    yb = _rn(b + np.abs(b) * _EPS64, "fp32")
    if extra:
        return (_rd(ya - ulps * _ulp(np.abs(ya) + extra, "fp32"), "fp32"),
                _ru(yb + ulps * _ulp(np.abs(yb) + extra, "fp32"), "fp32"))
    return _steps(ya, "fp32", ulps)[0], _steps(yb, "fp32", ulps)[1]


def _accumulate(terms, axis, standard, n_extra=0):
    """Sum of interval terms (each already rounded) along ``axis``: the hull over the normal
    orders (index order; 2 or 4 lanes, each starting from its first term, then combined in
    order or pairwise), or, for any order, gamma(n - 1 + n_extra) * sum |t|."""
    lo = np.moveaxis(terms[0], axis, 0)
    hi = np.moveaxis(terms[1], axis, 0)
    n = lo.shape[0]
    if n == 0:
        z = np.zeros(lo.shape[1:])
        return z, z
    if standard == "any_order":
        with np.errstate(invalid="ignore"):
            mag = np.maximum(np.abs(lo), np.abs(hi)).sum(axis=0)
            g = _gamma(n - 1 + n_extra) + n * 2.0 ** -52     # + the float64 sums' own error
            return _rd(lo.sum(axis=0) - g * mag, "fp32"), _ru(hi.sum(axis=0) + g * mag, "fp32")
    if standard != "normal":
        raise ValueError("standard must be 'normal' or 'any_order'")

    def run(idx):
        acc = None
        for i in idx:
            t = (lo[i], hi[i])
            acc = t if acc is None else _round(_iv_add(acc, t))
        return acc

    def seq(parts):
        r = parts[0]
        for q in parts[1:]:
            r = _round(_iv_add(r, q))
        return r

    results = []
    for lanes in (1, 2, 4):
        parts = [run(range(j, n, lanes)) for j in range(min(lanes, n))]
        results.append(seq(parts))
        if len(parts) == 4:
            results.append(_round(_iv_add(_round(_iv_add(parts[0], parts[1])), _round(_iv_add(parts[2], parts[3])))))
    return (np.minimum.reduce([r[0] for r in results]), np.maximum.reduce([r[1] for r in results]))


def _prod_any(a_lo, a_hi, b):
    """Sum over the middle axis of interval a (rows, n) times exact b (n, cols), each product
    rounded, summed in any order: (lo, hi) (rows, cols), k = n + n_extra steps per term."""
    bp, bn = np.maximum(b, 0.0), np.minimum(b, 0.0)
    slo = a_lo @ bp + a_hi @ bn
    shi = a_hi @ bp + a_lo @ bn
    mag = np.maximum(np.abs(a_lo), np.abs(a_hi)) @ np.abs(b)
    return slo, shi, mag


# ----------------------------------------------------------------- the model

def _scale_interval(E, scale):
    """The scale factor rounded to float32; 1/sqrt(E) is enclosed exactly (a point when
    it is a float64 value, else its two float64 neighbours)."""
    if scale is None:
        if E == 0:
            return (np.float64(0.0), np.float64(0.0))
        c = 1.0 / math.sqrt(E)
        sq = Fraction(c) ** 2 * E               # compare c^2 with 1/E exactly
        if sq == 1:
            exact = (np.float64(c), np.float64(c))
        elif sq < 1:
            exact = (np.float64(c), np.nextafter(c, np.inf))
        else:
            exact = (np.nextafter(c, -np.inf), np.float64(c))
    else:
        exact = (np.float64(scale), np.float64(scale))
    return _round(exact)


def _scores(q, k, standard):
    """Enclosure of the computed scores (L, S): products rounded, accumulated over E."""
    L, E = q.shape
    S = k.shape[0]
    if E == 0:
        z = np.zeros((L, S))
        return z, z
    if standard == "any_order":
        g = _gamma(E) + E * 2.0 ** -52
        s = q @ k.T
        mag = np.abs(q) @ np.abs(k).T
        return _rd(s - g * mag, "fp32"), _ru(s + g * mag, "fp32")
    prod = q[:, None, :] * k[None, :, :]      # exact: two float32-grid values
    return _accumulate(_round((prod, prod)), 2, standard)


def _values(w, v, standard, n_extra):
    """Enclosure of sum_j w_j v_j (L, Ev) for interval weights w (L, S) >= 0."""
    S = v.shape[0]
    if standard == "any_order":
        slo, shi, mag = _prod_any(w[0], w[1], v)
        g = _gamma(S + n_extra) + S * 2.0 ** -52
        return _rd(slo - g * mag, "fp32"), _ru(shi + g * mag, "fp32")
    prod = _round(_iv_mul((w[0][:, :, None], w[1][:, :, None]), (v[None, :, :], v[None, :, :])))
    return _accumulate(prod, 1, standard, n_extra)


def _row_model(q, k, v, bias, sc, fmt, ulps, standard, alg):
    """Enclosures for a block of query rows of one (batch, head): q (L, E), k (S, E),
    v (S, Ev) exact values, bias (L, S) float64 (0, -inf or a float mask value; -inf for
    every key of a special row).  Returns (out (lo, hi) (L, Ev) before the rounding to the
    output format, lse (lo, hi) (L,), rows with a kept key (L,))."""
    L = q.shape[0]
    S = v.shape[0]
    if alg is not None and 0 < alg.split_size < S:
        return _split_model(q, k, v, bias, sc, fmt, ulps, standard, alg)
    kept = np.isfinite(bias)
    s = _scores(q, k, standard)
    if q.shape[1] == 0:
        x = (bias, bias)
    else:
        x = _iv_mul(s, sc)
        x = (_add(x[0], bias, -1), _add(x[1], bias, +1))
    ell = _round(x)
    for _ in range(alg.extra_logit_roundings if alg is not None else 0):
        ell = _round(ell)
    ell = (np.where(kept, ell[0], -np.inf), np.where(kept, ell[1], -np.inf))
    m = (np.max(ell[0], axis=1, initial=-np.inf), np.max(ell[1], axis=1, initial=-np.inf))
    has = np.isfinite(m[0]) & np.isfinite(m[1])
    m = (np.where(has, m[0], 0.0), np.where(has, m[1], 0.0))
    slack = alg.shift_slack if alg is not None else 0.0
    d = (_add(ell[0], -m[1][:, None], -1), _add(ell[1], -m[0][:, None], +1))
    d = _round(d, extra=slack)
    for _ in range(alg.extra_shift_roundings if alg is not None else 0):
        d = _round(d, extra=slack)
    w = _exp_within(d, ulps)
    w = (np.where(kept, w[0], 0.0), np.where(kept, w[1], 0.0))
    n_resc = 0 if alg is None else max(0, -(-S // alg.block_n) - 1)
    row_sum = _accumulate(w, 1, standard, n_extra=n_resc)
    wv = w
    if alg is not None and alg.round_weights and fmt != "fp32":
        wv = _round(w, fmt)
    vsum = _values(wv, v, standard, n_resc)
    ls = (np.maximum(row_sum[0], 2.0 ** -149), np.maximum(row_sum[1], 2.0 ** -149))   # for lse
    if alg is not None and alg.round_row_sum and wv is not w:
        row_sum = _accumulate(wv, 1, standard, n_extra=n_resc)
    rs = (np.maximum(row_sum[0], 2.0 ** -149), np.maximum(row_sum[1], 2.0 ** -149))
    if alg is not None and alg.reciprocal:
        inv = _round(_iv_div_pos((np.ones(L), np.ones(L)), rs))
        o = _round(_iv_mul(vsum, (inv[0][:, None], inv[1][:, None])))
    else:
        o = _round(_iv_div_pos(vsum, (rs[0][:, None], rs[1][:, None])))
    o = (np.where(has[:, None], o[0], 0.0), np.where(has[:, None], o[1], 0.0))   # no kept key: 0
    # logsumexp sees the row sum with the rescale factors' exp errors (they cancel in the output)
    if n_resc:
        f = (1 + (ulps + 0.5) * 2.0 ** -23) ** n_resc
        ls = (_rd(ls[0] / f, "fp32"), _ru(ls[1] * f, "fp32"))
    lse = _round(_iv_add(m, _log_within(ls, ulps, extra=slack)), extra=slack)
    for _ in range(alg.extra_lse_roundings if alg is not None else 0):
        lse = _round(lse)
    return o, lse, has


def _split_model(q, k, v, bias, sc, fmt, ulps, standard, alg):
    """Keys cut into contiguous parts of alg.split_size (an implementation allowance), each
    part's normalised output and logsumexp from the model, merged through the logsumexps:
    M = max lse_s, e_s = exp(lse_s - M) (difference rounded, taken into base 2: one more
    rounding), W = sum e_s, out = sum e_s o_s / W, lse = M + log W (log in base 2, then a
    rounded product with ln 2)."""
    S = k.shape[0]
    bounds = list(range(0, S, alg.split_size)) + [S]
    inner = Blocked(alg.block_n, alg.round_weights, alg.round_row_sum, alg.reciprocal, alg.shift_slack,
                    alg.extra_logit_roundings, alg.extra_shift_roundings, alg.extra_lse_roundings, 0)
    parts = [_row_model(q, k[a:b], v[a:b], bias[:, a:b], sc, fmt, ulps, standard, inner)
             for a, b in zip(bounds[:-1], bounds[1:])]
    has = np.logical_or.reduce([h for _, _, h in parts])
    M = (np.max(np.stack([np.where(h, l[0], -np.inf) for _, l, h in parts]), axis=0),
         np.max(np.stack([np.where(h, l[1], -np.inf) for _, l, h in parts]), axis=0))
    M = (np.where(has, M[0], 0.0), np.where(has, M[1], 0.0))
    es, terms = [], []
    for o, l, h in parts:
        dd = _round(_round((_add(l[0], -M[1], -1), _add(l[1], -M[0], +1))))
        e = _exp_within(dd, ulps)
        e = (np.where(h, e[0], 0.0), np.where(h, e[1], 0.0))
        es.append(e)
        terms.append(_round(_iv_mul((e[0][:, None], e[1][:, None]), o)))
    W = _accumulate((np.stack([e[0] for e in es], 1), np.stack([e[1] for e in es], 1)), 1, "any_order")
    num = _accumulate((np.stack([t[0] for t in terms], 1), np.stack([t[1] for t in terms], 1)), 1, "any_order")
    W = (np.maximum(W[0], 2.0 ** -149), np.maximum(W[1], 2.0 ** -149))
    o = _round(_iv_div_pos(num, (W[0][:, None], W[1][:, None])))
    lse = _round(_iv_add(M, _round(_log_within(W, ulps))))
    return o, lse, has


@dataclass
class Analysis:
    """Per-element results: the exact value rounded to the output format, the range a
    correct implementation may return, and the tolerance (largest distance from
    ``rounded`` to an end of the range); the same for logsumexp (float32)."""
    rounded: np.ndarray
    low: np.ndarray
    high: np.ndarray
    tolerance: np.ndarray
    lse_rounded: np.ndarray
    lse_low: np.ndarray
    lse_high: np.ndarray
    lse_tolerance: np.ndarray

    def covers(self, output=None, lse=None):
        """Elementwise: a computed output (and/or lse) lies in the finite range; NaN must be
        NaN and an exactly infinite or special value must be matched exactly."""
        res = []
        for c, lo, hi in ((output, self.low, self.high), (lse, self.lse_low, self.lse_high)):
            if c is None:
                continue
            c = _f64(c)
            with np.errstate(invalid="ignore"):
                both_nan = np.isnan(lo) & np.isnan(c)
                ok = both_nan | ((c >= lo) & (c <= hi))
            res.append(ok)
        return res[0] if len(res) == 1 else tuple(res)

    def finite_range(self):
        return self.low, self.high


def analyse(query, key, value, attn_mask=None, is_causal=False, scale=None, enable_gqa=False, *,
            dtype="fp32", ulps=2, standard="normal", algorithm=None):
    """The tolerance analysis of attention on these inputs (see the module docstring).

    ``dtype`` is the input/output format ("fp32", "bf16" or "fp16": the inputs must hold
    values of it); ``standard`` is "normal" (the page's default) or "any_order";
    ``algorithm`` is None (the page's default budget) or a Blocked(...).
    """
    if dtype not in FORMATS:
        raise ValueError("dtype must be fp32, bf16 or fp16")
    q, k, v = _f64(query), _f64(key), _f64(value)
    out, lse = sdpa(q, k, v, attn_mask=attn_mask, is_causal=is_causal, scale=scale, enable_gqa=enable_gqa)
    ell = logits(q, k, attn_mask, is_causal, scale, enable_gqa)
    kk, vv = _expand_kv(q, k, v, enable_gqa)
    E = q.shape[-1]
    L, S, Ev = ell.shape[-2], ell.shape[-1], vv.shape[-1]
    # the bias alone (masks folded), as the model needs it separately from the scores
    zero_q = np.zeros(q.shape[:-1] + (0,))
    bias = logits(zero_q, np.zeros(k.shape[:-1] + (0,)), attn_mask, is_causal, scale, enable_gqa)
    lead = np.broadcast_shapes(ell.shape[:-2], vv.shape[:-2], q.shape[:-2], out.shape[:-2])
    qb = np.broadcast_to(q, lead + (L, E)).reshape(-1, L, E)
    kb = np.broadcast_to(kk, lead + (S, E)).reshape(-1, S, E)
    vb = np.broadcast_to(vv, lead + (S, Ev)).reshape(-1, S, Ev)
    bb = np.broadcast_to(bias, lead + (L, S)).reshape(-1, L, S)
    ob = np.broadcast_to(out, lead + (L, Ev)).reshape(-1, L, Ev)
    lb = np.broadcast_to(lse, lead + (L,)).reshape(-1, L)
    eb = np.broadcast_to(ell, lead + (L, S)).reshape(-1, L, S)
    sc = _scale_interval(E, scale)

    lo = np.empty(ob.shape)
    hi = np.empty(ob.shape)
    llo = np.empty(lb.shape)
    lhi = np.empty(lb.shape)
    # rows in chunks that bound the (rows, keys, dim) temporaries of the normal orders
    width = max(E, Ev, 1) if standard == "normal" else 1
    chunk = max(1, min(L, (1 << 22) // max(1, S * width)))
    for n in range(ob.shape[0]):
        nan_row, inf_row, empty_row, normal = _row_classes(eb[n])
        bn = np.where(normal[:, None], bb[n], -np.inf)
        for r0 in range(0, L, chunk):
            r1 = min(L, r0 + chunk)
            o, l_, _ = _row_model(qb[n, r0:r1], kb[n], vb[n], bn[r0:r1], sc, dtype, ulps, standard, algorithm)
            if dtype != "fp32":
                o = _round(o, dtype)
            special = ~normal[r0:r1, None] | ~np.isfinite(ob[n, r0:r1])
            lo[n, r0:r1] = np.where(special, ob[n, r0:r1], o[0])
            hi[n, r0:r1] = np.where(special, ob[n, r0:r1], o[1])
            llo[n, r0:r1] = np.where(normal[r0:r1], l_[0], lb[n, r0:r1])
            lhi[n, r0:r1] = np.where(normal[r0:r1], l_[1], lb[n, r0:r1])
    rounded = _rn(ob, dtype)
    lrounded = _rn(lb, "fp32")
    with np.errstate(invalid="ignore"):
        tol = np.where(np.isfinite(rounded), np.maximum(hi - rounded, rounded - lo), 0.0)
        ltol = np.where(np.isfinite(lrounded), np.maximum(lhi - lrounded, lrounded - llo), 0.0)
    shape_o = lead + (L, Ev)
    shape_l = lead + (L,)
    return Analysis(rounded.reshape(shape_o), lo.reshape(shape_o), hi.reshape(shape_o),
                    np.nan_to_num(tol).reshape(shape_o), lrounded.reshape(shape_l), llo.reshape(shape_l),
                    lhi.reshape(shape_l), np.nan_to_num(ltol).reshape(shape_l))


def tolerance(query, key, value, attn_mask=None, is_causal=False, scale=None, enable_gqa=False, **kw):
    """(output tolerance, lse tolerance): the page's ``tolerance()`` per element."""
    a = analyse(query, key, value, attn_mask, is_causal, scale, enable_gqa, **kw)
    return a.tolerance, a.lse_tolerance


def finite_range(query, key, value, attn_mask=None, is_causal=False, scale=None, enable_gqa=False, **kw):
    """((out low, out high), (lse low, lse high)): the page's ``finite_range()`` per element."""
    a = analyse(query, key, value, attn_mask, is_causal, scale, enable_gqa, **kw)
    return (a.low, a.high), (a.lse_low, a.lse_high)


def covers(computed_out, computed_lse, query, key, value, attn_mask=None, is_causal=False, scale=None,
           enable_gqa=False, **kw):
    """(output covered, lse covered) elementwise for a computed result (either may be None)."""
    a = analyse(query, key, value, attn_mask, is_causal, scale, enable_gqa, **kw)
    res = []
    if computed_out is not None:
        res.append(a.covers(output=computed_out))
    if computed_lse is not None:
        res.append(a.covers(lse=computed_lse))
    return tuple(res)
