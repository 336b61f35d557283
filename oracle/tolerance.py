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

The backward (``analyse_backward``; the page's "scaled_dot_product_attention.
backward" section, its tolerance() paragraph) takes the same readings through
the gradient program the page lists: the forward's scores, scale factor,
logits, shift, exp within ``ulps`` and row sum; the weights P = w / row sum,
one rounding each; dP = grad V^T and D_i = sum_j P_ij dP_ij accumulated; dP - D
rounded; dS = P (dP - D) rounded; grad_value = P^T grad, dS K and dS^T Q
accumulated (each over the copies grouped heads or broadcasting made of its
input as well: one longer sum); the scale product rounded; the rounding to the
output format.  Its named algorithm (``BlockedBackward``) adds what the page
says such algorithms budget: P formed without a division by the row sum, as
exp(l - lse) from the forward's logsumexp (any value the forward's own model
allows), D from the forward's output (D_i = grad_i . O_i, O any output the
forward's model allows), P and dS rounded to the input format before their
products, and the base-2 exponent's extra roundings.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

from .sdpa_oracle import _expand_kv, _f64, _row_classes, logits, resolve_scale, sdpa

__all__ = ["Blocked", "Analysis", "analyse", "tolerance", "finite_range", "covers",
           "BlockedBackward", "BackwardAnalysis", "analyse_backward"]

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
    """Largest grid value <= x (-inf below the finite range, the largest finite value above it).
    float32 through numpy's own float32 conversion (nearest, then one step down where that
    lies above x); other formats by scaling to the grid spacing (``_rd_grid``)."""
    x = np.asarray(x, dtype=np.float64)
    if fmt != "fp32":
        return _rd_grid(x, fmt)
    with np.errstate(over="ignore", invalid="ignore"):
        y = x.astype(np.float32)
        y = np.where(y.astype(np.float64) > x, np.nextafter(y, np.float32(-np.inf)), y)
    return y.astype(np.float64)


def _rd_grid(x, fmt):
    """``_rd`` for any format of FORMATS, from the grid spacing."""
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
    if fmt == "fp32":
        with np.errstate(over="ignore"):
            return x.astype(np.float32).astype(np.float64)
    return _rn_grid(x, fmt)


def _rn_grid(x, fmt):
    """``_rn`` for any format of FORMATS, from ``_rd_grid``."""
    x = np.asarray(x, dtype=np.float64)
    lo, hi = _rd_grid(x, fmt), -_rd_grid(-x, fmt)
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
        rlo, rhi = _rd(a, fmt), _ru(b, fmt)
        if edge.any():
            rlo = np.where(edge, _rn(lo, fmt), rlo)
            rhi = np.where(edge, _rn(hi, fmt), rhi)
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
    chunk = max(1, (1 << 22) // max(1, S * E))
    parts = []
    for r in range(0, L, chunk):
        prod = q[r:r + chunk, None, :] * k[None, :, :]      # exact: two float32-grid values
        parts.append(_accumulate(_round((prod, prod)), 2, standard))
    return np.concatenate([p_[0] for p_ in parts]), np.concatenate([p_[1] for p_ in parts])


def _values(w, v, standard, n_extra):
    """Enclosure of sum_j w_j v_j (L, Ev) for interval w (L, S) and exact v (S, Ev)."""
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
    N = int(np.prod(lead, dtype=np.int64))
    qb = np.broadcast_to(q, lead + (L, E)).reshape(N, L, E)
    kb = np.broadcast_to(kk, lead + (S, E)).reshape(N, S, E)
    vb = np.broadcast_to(vv, lead + (S, Ev)).reshape(N, S, Ev)
    bb = np.broadcast_to(bias, lead + (L, S)).reshape(N, L, S)
    ob = np.broadcast_to(out, lead + (L, Ev)).reshape(N, L, Ev)
    lb = np.broadcast_to(lse, lead + (L,)).reshape(N, L)
    eb = np.broadcast_to(ell, lead + (L, S)).reshape(N, L, S)
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


# ------------------------------------------------------------------ the backward

@dataclass(frozen=True)
class BlockedBackward:
    """A FlashAttention-style backward, with the roundings the page's default omits.

    forward:      the forward (a Blocked, or None for the page's default budget) whose
                  output O and logsumexp the backward reads: P_ij = exp(l_ij - lse_i) with
                  lse_i any value that forward may return (the row sum enters through the
                  logsumexp instead of a division), and D_i = grad_i . O_i with O_i any
                  output it may return
    round_inputs: P (in the product for grad_value) and dS (in the products for grad_query
                  and grad_key) rounded to the input format (not for float32 inputs)
    extra_logit_roundings, extra_lse_roundings: further roundings of each logit and of
                  the logsumexp (an exponent formed in base 2 through scale * log2 e and
                  lse * log2 e, each rounded)
    """
    forward: Blocked | None = None
    round_inputs: bool = True
    extra_logit_roundings: int = 0
    extra_lse_roundings: int = 0


def _contract(a, b, standard):
    """Enclosure of a @ b for interval a (R, K) and exact b (K, C), every product rounded
    and the K terms accumulated (normal orders or any order); rows in chunks for the
    (R, K, C) temporaries of the normal orders."""
    R, K = a[0].shape
    C = b.shape[1]
    if K == 0 or R == 0 or C == 0:
        z = np.zeros((R, C))
        return z, z
    if standard == "any_order":
        return _values(a, b, standard, 0)
    chunk = max(1, (1 << 22) // max(1, K * C))
    parts = [_values((a[0][r:r + chunk], a[1][r:r + chunk]), b, standard, 0) for r in range(0, R, chunk)]
    return np.concatenate([p_[0] for p_ in parts]), np.concatenate([p_[1] for p_ in parts])


def _bwd_head(q, k, v, g, bias, sc, fmt, ulps, standard, alg, fwd_o, fwd_lse):
    """One (batch, head): enclosures of the weights P as they enter grad_value and of dS as
    it enters grad_query and grad_key, both (L, S).  q (L, E), k (S, E), v (S, Ev) and the
    output gradient g (L, Ev) are exact values; bias (L, S) as in the forward model (-inf for
    every key of a special row); fwd_o (lo, hi) (L, Ev) and fwd_lse (lo, hi) (L,) are the
    forward's enclosures (used by a BlockedBackward only)."""
    kept = np.isfinite(bias)
    has = kept.any(axis=1)
    s = _scores(q, k, standard)
    if q.shape[1] == 0:
        x = (bias, bias)
    else:
        x = _iv_mul(s, sc)
        x = (_add(x[0], bias, -1), _add(x[1], bias, +1))
    ell = _round(x)
    dP = _scores(g, v, standard)                      # grad_i . v_j
    if alg is None:
        ell = (np.where(kept, ell[0], -np.inf), np.where(kept, ell[1], -np.inf))
        m = (np.max(ell[0], axis=1, initial=-np.inf), np.max(ell[1], axis=1, initial=-np.inf))
        m = (np.where(has, m[0], 0.0), np.where(has, m[1], 0.0))
        d = _round((_add(ell[0], -m[1][:, None], -1), _add(ell[1], -m[0][:, None], +1)))
        w = _exp_within(d, ulps)
        w = (np.where(kept, w[0], 0.0), np.where(kept, w[1], 0.0))
        rs = _accumulate(w, 1, standard)
        rs = (np.maximum(rs[0], 2.0 ** -149), np.maximum(rs[1], 2.0 ** -149))
        P = _round(_iv_div_pos(w, (rs[0][:, None], rs[1][:, None])))
        D = _accumulate(_round(_iv_mul(P, dP)), 1, standard)
    else:
        for _ in range(alg.extra_logit_roundings):
            ell = _round(ell)
        lse = fwd_lse
        for _ in range(alg.extra_lse_roundings):
            lse = _round(lse)
        lse = (np.where(has, lse[0], 0.0), np.where(has, lse[1], 0.0))
        with np.errstate(invalid="ignore"):
            d = _round((_add(ell[0], -lse[1][:, None], -1), _add(ell[1], -lse[0][:, None], +1)))
        d = (np.where(kept, d[0], -np.inf), np.where(kept, d[1], -np.inf))
        P = _exp_within(d, ulps)
        P = (np.where(kept, P[0], 0.0), np.where(kept, P[1], 0.0))
        if g.shape[1] == 0:
            D = (np.zeros(q.shape[0]), np.zeros(q.shape[0]))
        else:
            D = _accumulate(_round(_iv_mul((g, g), fwd_o)), 1, standard)
    t = _round((_add(dP[0], -D[1][:, None], -1), _add(dP[1], -D[0][:, None], +1)))
    dS = _round(_iv_mul(P, t))
    dS = (np.where(kept, dS[0], 0.0), np.where(kept, dS[1], 0.0))
    if alg is not None and alg.round_inputs and fmt != "fp32":
        P, dS = _round(P, fmt), _round(dS, fmt)
    return P, dS


@dataclass
class BackwardAnalysis:
    """Per gradient ("grad_query", "grad_key", "grad_value"): the exact value rounded to the
    output format, the range a correct implementation may return and the tolerance."""
    rounded: dict
    low: dict
    high: dict
    tolerance: dict

    def covers(self, **computed):
        """Elementwise coverage of computed gradients, by name (grad_query=..., ...)."""
        res = {}
        for name, c in computed.items():
            c = _f64(c)
            lo, hi = self.low[name], self.high[name]
            with np.errstate(invalid="ignore"):
                res[name] = (np.isnan(lo) & np.isnan(c)) | ((c >= lo) & (c <= hi))
        return res


def _head_index(shape, expand, lead):
    """Flat index of the input copy each (flattened) head of ``lead`` reads: the input's
    leading dims numbered, grouped heads repeated (``expand``), broadcast to ``lead``."""
    idx = np.arange(int(np.prod(shape, dtype=np.int64))).reshape(shape)
    if expand > 1:
        idx = np.repeat(idx, expand, axis=-1)
    return np.broadcast_to(idx, lead).reshape(-1)


def analyse_backward(query, key, value, grad, attn_mask=None, is_causal=False, scale=None, enable_gqa=False, *,
                     dtype="fp32", ulps=2, standard="normal", algorithm=None, out=None, lse=None):
    """The tolerance analysis of the attention backward on these inputs (module docstring,
    "The backward").  ``algorithm`` is None (the page's default budget) or a
    BlockedBackward(...); the other arguments as for ``analyse``.  With a BlockedBackward,
    ``out`` and ``lse`` may give the forward's output and logsumexp the backward is handed
    (values, in the forward's shapes): they are then used as they are, instead of every
    value the forward's model allows."""
    from .sdpa_oracle import sdpa_backward
    if dtype not in FORMATS:
        raise ValueError("dtype must be fp32, bf16 or fp16")
    q, k, v, g = _f64(query), _f64(key), _f64(value), _f64(grad)
    exact = dict(zip(("grad_query", "grad_key", "grad_value"),
                     sdpa_backward(q, k, v, g, attn_mask=attn_mask, is_causal=is_causal, scale=scale,
                                   enable_gqa=enable_gqa)))
    ell = logits(q, k, attn_mask, is_causal, scale, enable_gqa)
    kk, vv = _expand_kv(q, k, v, enable_gqa)
    E = q.shape[-1]
    L, S, Ev = ell.shape[-2], ell.shape[-1], vv.shape[-1]
    zero_q = np.zeros(q.shape[:-1] + (0,))
    bias = logits(zero_q, np.zeros(k.shape[:-1] + (0,)), attn_mask, is_causal, scale, enable_gqa)
    lead = np.broadcast_shapes(ell.shape[:-2], vv.shape[:-2], q.shape[:-2], g.shape[:-2])
    N = int(np.prod(lead, dtype=np.int64))
    qb = np.broadcast_to(q, lead + (L, E)).reshape(N, L, E)
    kb = np.broadcast_to(kk, lead + (S, E)).reshape(N, S, E)
    vb = np.broadcast_to(vv, lead + (S, Ev)).reshape(N, S, Ev)
    gb = np.broadcast_to(g, lead + (L, Ev)).reshape(N, L, Ev)
    bb = np.broadcast_to(bias, lead + (L, S)).reshape(N, L, S)
    eb = np.broadcast_to(ell, lead + (L, S)).reshape(N, L, S)
    sc = _scale_interval(E, scale)
    if algorithm is not None:
        if out is None or lse is None:
            fa = analyse(q, k, v, attn_mask, is_causal, scale, enable_gqa, dtype=dtype, ulps=ulps,
                         standard=standard, algorithm=algorithm.forward)
        o_lo, o_hi = (fa.low, fa.high) if out is None else (_f64(out), _f64(out))
        l_lo, l_hi = (fa.lse_low, fa.lse_high) if lse is None else (_f64(lse), _f64(lse))
        fo = (np.broadcast_to(o_lo, lead + (L, Ev)).reshape(N, L, Ev),
              np.broadcast_to(o_hi, lead + (L, Ev)).reshape(N, L, Ev))
        fl = (np.broadcast_to(l_lo, lead + (L,)).reshape(N, L),
              np.broadcast_to(l_hi, lead + (L,)).reshape(N, L))
    heads = []
    for n in range(N):
        normal = _row_classes(eb[n])[3]
        bn = np.where(normal[:, None], bb[n], -np.inf)
        fwd = (None, None) if algorithm is None else ((fo[0][n], fo[1][n]), (fl[0][n], fl[1][n]))
        heads.append(_bwd_head(qb[n], kb[n], vb[n], gb[n], bn, sc, dtype, ulps, standard, algorithm, *fwd))
    # which input copy each head reads (grouped heads repeat key/value heads along the head axis)
    rep = q.shape[-3] // k.shape[-3] if (enable_gqa and q.ndim >= 3 and k.ndim >= 3 and k.shape[-3] > 0
                                        and q.shape[-3] != k.shape[-3]) else 1
    qi = _head_index(q.shape[:-2], 1, lead)
    ki = _head_index(k.shape[:-2], rep, lead)
    vi = _head_index(v.shape[:-2], rep, lead)

    def gather(index, count, rows, cols, term):
        """For each input copy c: the enclosure of sum over the heads n reading c of
        term(n) = (interval a (rows, K_n), exact b (K_n, cols)), one accumulation."""
        out_lo = np.zeros((count, rows, cols))
        out_hi = np.zeros((count, rows, cols))
        for c in range(count):
            ns = np.flatnonzero(index == c)
            if ns.size == 0:
                continue
            ts = [term(n) for n in ns]
            a = (np.concatenate([t[0][0] for t in ts], axis=1), np.concatenate([t[0][1] for t in ts], axis=1))
            b = np.concatenate([t[1] for t in ts], axis=0)
            out_lo[c], out_hi[c] = _contract(a, b, standard)
        return out_lo, out_hi

    nq = int(np.prod(q.shape[:-2], dtype=np.int64))
    nk = int(np.prod(k.shape[:-2], dtype=np.int64))
    nv = int(np.prod(v.shape[:-2], dtype=np.int64))
    sums = {
        "grad_query": gather(qi, nq, L, E, lambda n: (heads[n][1], kb[n])),
        "grad_key": gather(ki, nk, S, E, lambda n: ((heads[n][1][0].T, heads[n][1][1].T), qb[n])),
        "grad_value": gather(vi, nv, S, Ev, lambda n: ((heads[n][0][0].T, heads[n][0][1].T), gb[n])),
    }
    shapes = {"grad_query": q.shape, "grad_key": k.shape, "grad_value": v.shape}
    rounded, low, high, tol = {}, {}, {}, {}
    for name, r in sums.items():
        if name != "grad_value":
            r = _round(_iv_mul(r, (sc[0], sc[1])))      # the scale product
        if dtype != "fp32":
            r = _round(r, dtype)
        x = exact[name]
        special = ~np.isfinite(x)
        lo = np.where(special, x, r[0].reshape(shapes[name]))
        hi = np.where(special, x, r[1].reshape(shapes[name]))
        rd = _rn(x, dtype)
        with np.errstate(invalid="ignore"):
            tl = np.where(np.isfinite(rd), np.maximum(hi - rd, rd - lo), 0.0)
        rounded[name], low[name], high[name], tol[name] = rd, lo, hi, np.nan_to_num(tl)
    return BackwardAnalysis(rounded, low, high, tol)
