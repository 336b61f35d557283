"""Per-element error budget for computed attention (an ExactRef-style tolerance), float64.

TEST INFRASTRUCTURE ONLY, like sdpa_oracle: only ``tests/``, ``__graft_entry__``
and the benchmark's cpu_baseline leg may import it; the HIP path never does.

The exactref.ai "scaled_dot_product_attention" page (sections "Tolerance
options" and "Full specification") describes a tolerance: for each output
element, how far a correct implementation may land from the exact value, given
the rounding steps it is allowed.  The page lists those steps but does not give
its formula, so this module derives its own bound for the same list:

  budgeted everywhere  the score accumulation (any order), the scale factor,
                       one rounding of each logit, the shift by the row maximum,
                       exp within ``ulps`` units in the last place, the row sum,
                       the value accumulation, the final division and the
                       rounding to the output format; for logsumexp, log within
                       ``ulps`` and one rounding of shift plus logarithm;
  named-algorithm      the weights rounded to the input format before the value
  steps (FlashAttention product, online-softmax rescaling (a rescale at most per
  style)               32 keys), a reciprocal of the row sum, and a split over
                       keys merged through the partial logsumexps.

All arithmetic is float32 (unit roundoff u = 2^-24 for one rounding); sums may
run in any order and on accumulators that truncate, so an n-term accumulation
is bounded with gamma(n) = n*ua / (1 - n*ua), ua = 2^-23, times the sum of the
magnitudes of its terms (the classical bound for dot products, products
included).

Derivation, per query row with kept keys j (exact logits l_j, exact weights P_j,
exact output O):
  * The computed unnormalised weight of key j is exp(l_j - shift) times
    (1 + eta_j), where eta_j collects, in natural-log units, the error of the
    computed logit and of exp:
        eta_j = |scale| (1 + 2u) gamma(E) A_j + 2u (|scale s_j| + |l_j| + |b_j|)
                + u (|l_j| + Msh) + 2 ulps u
    with s_j the exact score, A_j = sum_e |q_e k_je|, b_j the mask bias and
    Msh = |max_j l_j| + 8 ln 2 a bound on the magnitude of the shift (a lazily
    raised maximum may trail the true one by up to 2^8 in the weights).  The
    shift itself cancels between the value sum and the row sum.
  * A common relative perturbation of the weights moves the normalised output
    by sum_j P_j eta_j |v_j - O| (first order: O = sum w v / sum w).
  * Weights rounded to the input format before the value product: relative
    u_w per weight (2^-8 bf16, 2^-11 fp16, 0 when they stay float32), plus an
    absolute a_w per weight for formats whose small weights lose precision
    (fp16 subnormals: 2^-25; float32 flush to zero: 2^-126), with row sums of
    at least 1 because the largest weight is exp(0) or more:
        u_w sum_j P_j |v_j| + a_w sum_j |v_j|.
  * Value and row-sum accumulations: gamma(n) (sum_j P_j |v_j| + |O|).
  * Rescales (at most R = ceil(n / 32) + 1), reciprocal, products: (2R + 4) u |O|.
  * A split over keys merged by logsumexp weights each partial output by
    exp(lse_s - lse); an error in those weights moves O by at most
    (lse_tol + 2 ulps u + 4u) sum_j P_j |v_j - O|.
  * Rounding to the output format adds half an ulp of the computed value:
    u_out (|O| + B) plus fp16's subnormal half-ulp 2^-25.
  * lse: sum_j P_j eta_j + gamma(n) + R (2 ulps u + 2u)
         + (2 ulps + 4) u (|lse| + Msh + log(n + 1)), then one float32 rounding.
The first-order bound B is multiplied by (1 + 2^-10) to cover the neglected
products of small terms.  Rows the page calls special (NaN, +inf, no kept key)
get tolerance 0: their computed values must match exactly.

Pins live in tests/test_oracle_tolerance.py: an independent float32 emulation
of the blocked algorithm is always covered; planted mistakes (weights rounded
too coarsely, a dropped mask entry, the double scaling the xFormers pages
describe) are not; the page's padding-mask and PyTorch examples come out as the
page reports.
"""
import math

import numpy as np

from .sdpa_oracle import _expand_kv, _f64, logits, resolve_scale, sdpa

__all__ = ["tolerance", "covers", "finite_range", "UNIT_ROUNDOFF"]

U32 = 2.0 ** -24          # one float32 rounding (nearest)
UA = 2.0 ** -23           # accumulations: any order, truncating accumulators allowed
UNIT_ROUNDOFF = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11, "fp32": 2.0 ** -24}
WEIGHT_ABS = {"bf16": 2.0 ** -126, "fp16": 2.0 ** -25, "fp32": 2.0 ** -126}
OUT_ABS = {"bf16": 0.0, "fp16": 2.0 ** -25, "fp32": 0.0}


def _gamma(n):
    n = np.asarray(n, dtype=np.float64)
    return n * UA / (1.0 - n * UA)


def tolerance(query, key, value, attn_mask=None, is_causal=False, scale=None, enable_gqa=False,
              dtype="bf16", ulps=2, round_weights=None, rows_per_chunk=16):
    """Bounds (out_tol (..., L, Ev), lse_tol (..., L)) on |computed - exact|.

    ``dtype`` is the input/output format ("bf16", "fp16" or "fp32");
    ``round_weights`` (default: True for bf16/fp16) budgets the weights rounded
    to that format before the value product.  Arguments otherwise as sdpa().
    """
    if dtype not in UNIT_ROUNDOFF:
        raise ValueError("dtype must be bf16, fp16 or fp32")
    if round_weights is None:
        round_weights = dtype != "fp32"
    u_w = UNIT_ROUNDOFF[dtype] if round_weights else 0.0
    a_w = WEIGHT_ABS[dtype] if round_weights else WEIGHT_ABS["fp32"]
    u_out = UNIT_ROUNDOFF[dtype]
    e_exp = 2.0 * ulps * U32

    q, k, v = _f64(query), _f64(key), _f64(value)
    out, lse = sdpa(q, k, v, attn_mask=attn_mask, is_causal=is_causal, scale=scale, enable_gqa=enable_gqa)
    ell = logits(q, k, attn_mask, is_causal, scale, enable_gqa)
    kk, vv = _expand_kv(q, k, v, enable_gqa)
    E = q.shape[-1]
    sc = resolve_scale(E, scale) if E > 0 else 0.0
    with np.errstate(invalid="ignore", over="ignore"):
        s = np.matmul(q, np.swapaxes(kk, -1, -2)) if E > 0 else np.zeros(ell.shape)
        A = np.matmul(np.abs(q), np.swapaxes(np.abs(kk), -1, -2)) if E > 0 else np.zeros(ell.shape)
    L, S, Ev = ell.shape[-2], ell.shape[-1], vv.shape[-1]
    lead = np.broadcast_shapes(ell.shape[:-2], vv.shape[:-2], out.shape[:-2])
    ell = np.broadcast_to(ell, lead + (L, S)).reshape(-1, L, S)
    s = np.broadcast_to(s, lead + (L, S)).reshape(-1, L, S)
    A = np.broadcast_to(A, lead + (L, S)).reshape(-1, L, S)
    vv = np.broadcast_to(vv, lead + (S, Ev)).reshape(-1, S, Ev)
    O = np.broadcast_to(out, lead + (L, Ev)).reshape(-1, L, Ev)
    LS = np.broadcast_to(lse, lead + (L,)).reshape(-1, L)

    out_tol = np.zeros(O.shape)
    lse_tol = np.zeros(LS.shape)
    absv = np.abs(vv)
    for n_ in range(ell.shape[0]):
        for r0 in range(0, L, rows_per_chunk):
            r1 = min(L, r0 + rows_per_chunk)
            l_ = ell[n_, r0:r1]                                   # (R, S)
            kept = np.isfinite(l_)
            normal = np.isfinite(LS[n_, r0:r1])
            if not normal.any():
                continue
            with np.errstate(invalid="ignore", over="ignore"):
                m = np.max(np.where(kept, l_, -np.inf), axis=-1)  # exact row max (finite for normal rows)
                m = np.where(normal, m, 0.0)
                P = np.where(kept, np.exp(np.where(kept, l_ - m[:, None], -np.inf)), 0.0)
                P = P / np.where(normal, P.sum(axis=-1), 1.0)[:, None]
                lk = np.where(kept, l_, 0.0)
                sk = np.where(kept, s[n_, r0:r1], 0.0)
                bk = np.where(kept, l_ - sc * s[n_, r0:r1], 0.0) if E > 0 else lk
            nk = kept.sum(axis=-1).astype(np.float64)              # kept keys per row
            msh = np.abs(m) + 8.0 * math.log(2.0)
            eta = (abs(sc) * (1 + 2 * U32) * _gamma(E) * np.where(kept, A[n_, r0:r1], 0.0)
                   + 2 * U32 * (np.abs(sc * sk) + np.abs(lk) + np.abs(bk))
                   + U32 * (np.abs(lk) + msh[:, None]) + e_exp)
            eta = np.where(kept, eta, 0.0)
            Oc = O[n_, r0:r1]                                      # (R, Ev)
            dev = np.abs(vv[n_][None, :, :] - Oc[:, None, :])     # (R, S, Ev)
            pe = np.einsum("rj,rjd->rd", P * eta, dev)
            pdev = np.einsum("rj,rjd->rd", P, dev)
            pv = P @ absv[n_]
            sv = kept.astype(np.float64) @ absv[n_]
            nrs = np.ceil(nk / 32.0) + 1.0
            lse_c = np.where(normal, LS[n_, r0:r1], 0.0)          # finite stand-in on special rows
            lt = ((P * eta).sum(axis=-1) + _gamma(nk) + nrs * (e_exp + 2 * U32)
                  + (2 * ulps + 4) * U32 * (np.abs(lse_c) + msh + np.log(nk + 1.0)))
            b = (pe + u_w * pv + a_w * sv + _gamma(nk)[:, None] * (pv + np.abs(Oc))
                 + ((2 * nrs + 4) * U32)[:, None] * np.abs(Oc)
                 + (lt + e_exp + 4 * U32)[:, None] * pdev)
            b = b * (1.0 + 2.0 ** -10)
            b = b + u_out * (np.abs(Oc) + b) + OUT_ABS[dtype]
            lt = lt * (1.0 + 2.0 ** -10) + U32 * np.abs(lse_c)
            out_tol[n_, r0:r1] = np.where(normal[:, None], b, 0.0)
            lse_tol[n_, r0:r1] = np.where(normal, lt, 0.0)
    return out_tol.reshape(lead + (L, Ev)), lse_tol.reshape(lead + (L,))


def covers(computed, exact, tol):
    """Elementwise: the computed value is within tol of the exact one.  NaN must
    be NaN and an infinite exact value must be matched exactly."""
    c, e, t = _f64(computed), _f64(exact), np.asarray(tol, dtype=np.float64)
    nan_e = np.isnan(e)
    inf_e = np.isinf(e)
    fin = ~nan_e & ~inf_e
    ok = np.zeros(np.broadcast_shapes(c.shape, e.shape), dtype=bool)
    ok = np.where(nan_e, np.isnan(c), ok)
    ok = np.where(inf_e, c == e, ok)
    with np.errstate(invalid="ignore"):
        ok = np.where(fin, np.isfinite(c) & (np.abs(c - e) <= t), ok)
    return ok


def finite_range(exact, tol):
    """The lowest and highest value a correct implementation may return, per element."""
    e = _f64(exact)
    t = np.asarray(tol, dtype=np.float64)
    return e - t, e + t
