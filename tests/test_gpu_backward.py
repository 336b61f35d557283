"""Parity of the backward kernels (through the C interface) with the float64 oracle.

The forward runs on the GPU (sdpa_fwd) to give out and lse; the backward
(sdpa_bwd) then gives grad_query, grad_key, grad_value, compared element by
element with oracle.sdpa_backward on the same input values, two ways:

  * per element: every gradient element lies in the finite range of the
    exactref.ai "scaled_dot_product_attention.backward" tolerance budget
    (oracle.tolerance.analyse_backward, summed in any order) for the named
    algorithm each kernel runs, given the forward output and logsumexp the
    backward was handed: P = exp(l - lse) in base 2 (the scale and lse taken
    into base 2 through rounded products: one more rounding of each), D from
    the forward output, and on the matrix-core kernel P and dS rounded to the
    input format before their products; elements whose exact value is 0 for
    want of any contribution (keys no kept query reaches) must be 0;
  * per tensor, as a second bar: max |GPU - oracle| <= 2^-6 max|oracle| + 1e-3
    (bf16/fp16), 2^-14 max|oracle| + 1e-5 (fp32).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import sdpa_oracle as O
from oracle import tolerance as T
from transformer_attention_04_amd import inputs
from transformer_attention_04_amd import sdpa as S

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAMES = ("grad_query", "grad_key", "grad_value")
# the kernels' named algorithms (the forward's output and logsumexp are given)
MATRIX_BWD = T.BlockedBackward(round_inputs=True, extra_logit_roundings=1, extra_lse_roundings=1)
VECTOR_BWD = T.BlockedBackward(round_inputs=False)


def bwd_alg(dtype, E, Ev):
    """The matrix-core backward runs bf16/fp16 with E == Ev in {64, 96, 128}; the
    vector-ALU backward (fp32 throughout, natural-log exponent) every other call."""
    return MATRIX_BWD if dtype != "fp32" and E == Ev and E in (64, 96, 128) else VECTOR_BWD


def check_bwd_covered(gpu, ctx, what):
    """Every gradient element in the per-element finite range (see the module docstring)."""
    q, k, v, g = ctx["qkvg"]
    a = T.analyse_backward(q, k, v, g, dtype=ctx["dtype"], standard="any_order",
                           algorithm=bwd_alg(ctx["dtype"], q.shape[-1], v.shape[-1]), out=ctx["out"],
                           lse=ctx["lse"], **ctx["kw"])
    worst = []
    for n, x in zip(NAMES, gpu):
        x = _np(x)
        c = a.covers(**{n: x})[n]
        fin = a.tolerance[n] > 0
        worst.append(float((np.abs(x - a.rounded[n])[fin] / a.tolerance[n][fin]).max(initial=0.0)))
        assert c.all(), f"{what}: {int((~c).sum())} {n} elements outside the finite range, e.g. at " \
                        f"{tuple(np.argwhere(~c)[0])}: {x[tuple(np.argwhere(~c)[0])]:.6g} not in " \
                        f"[{a.low[n][tuple(np.argwhere(~c)[0])]:.6g}, {a.high[n][tuple(np.argwhere(~c)[0])]:.6g}]"
    print(f"{what}: worst distance from the rounded exact value / tolerance " +
          " ".join(f"{n} {w:.3f}" for n, w in zip(("dq", "dk", "dv"), worst)))


def _np(t):
    return t.detach().cpu().double().numpy()


def bwd_bar(ref, dtype="bf16"):
    """bf16/fp16: 2^-6 max|ref| + 1e-3 (the derivation above).  fp32 (the vector-ALU
    backward: every step in fp32, P from exp of the rounded logit minus lse, sums over
    at most a few hundred terms, each within a few float32 ulps): 2^-14 max|ref| + 1e-5."""
    if dtype == "fp32":
        return 2.0 ** -14 * float(np.abs(ref).max(initial=0.0)) + 1e-5
    return 2.0 ** -6 * float(np.abs(ref).max(initial=0.0)) + 1e-3


def run_bwd(q, k, v, g, dtype, **kw):
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    m = kw.get("attn_mask")
    md = None if m is None else m.to(DEV)
    out, lse = S.sdpa_fwd(qd, kd, vd, attn_mask=md, is_causal=kw.get("is_causal", False), scale=kw.get("scale"),
                          enable_gqa=kw.get("enable_gqa", False))
    dq, dk, dv = S.sdpa_bwd(qd, kd, vd, out, lse, gd, attn_mask=md, is_causal=kw.get("is_causal", False),
                            scale=kw.get("scale"), enable_gqa=kw.get("enable_gqa", False))
    torch.cuda.synchronize()
    if m is not None:
        kw = dict(kw, attn_mask=m.numpy() if m.dtype == torch.bool else m.double().numpy())
    ctx = dict(qkvg=(q, k, v, g), kw=kw, dtype=dtype, out=_np(out), lse=_np(lse).reshape(out.shape[:-1]))
    return (dq, dk, dv), O.sdpa_backward(q, k, v, g, **kw), ctx


def assert_bwd(gpu, ref, what, dtype="bf16", ctx=None):
    errs = []
    for a, r, n in zip(gpu, ref, ("dq", "dk", "dv")):
        a = _np(a)
        assert a.shape == r.shape, (what, n, a.shape, r.shape)
        assert np.isfinite(a).all(), f"{what}: non-finite {n}"
        e = float(np.abs(a - r).max(initial=0.0))
        bar = bwd_bar(r, dtype)
        errs.append((e, e / bar))
        assert e <= bar, f"{what}: max |{n} error| {e:.3e} > {bar:.3e} (max|ref| {np.abs(r).max(initial=0):.3e})"
    print(f"{what}: max error (fraction of the bar) " +
          " ".join(f"{n} {e:.2e} ({f:.2f})" for n, (e, f) in zip(("dq", "dk", "dv"), errs)))
    if ctx is not None:
        check_bwd_covered(gpu, ctx, what)
    return errs


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("E", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_ragged(dtype, E, causal):
    """Several query and key tiles with ragged tails (L, S not multiples of 64 or 128)."""
    L, Sk = (300, 300) if causal else (200, 333)
    q, k, v = inputs.randn_qkv((2, 3, L, E), (2, 3, Sk, E), (2, 3, Sk, E), dtype, seed=E + L)
    g = inputs.randn_qkv((2, 3, L, E), (1, 1, 1, E), (1, 1, 1, E), dtype, seed=E + L + 1)[0]
    gpu, ref, ctx = run_bwd(q, k, v, g, dtype, is_causal=causal)
    assert_bwd(gpu, ref, f"{dtype} E={E} causal={causal}", ctx=ctx)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_backward_gqa_and_scales(dtype):
    """Grouped-query heads (grad_key/grad_value summed over the group), negative and unit scales."""
    q, k, v = inputs.randn_qkv((1, 6, 257, 128), (1, 2, 257, 128), (1, 2, 257, 128), dtype, seed=11)
    g = inputs.randn_qkv((1, 6, 257, 128), (1, 1, 1, 128), (1, 1, 1, 128), dtype, seed=12)[0]
    for causal in (False, True):
        gpu, ref, ctx = run_bwd(q, k, v, g, dtype, is_causal=causal, enable_gqa=True)
        assert_bwd(gpu, ref, f"gqa causal={causal}", ctx=ctx)
    for scale in (-0.09, 1.0):
        gpu, ref, ctx = run_bwd(q[:, :2], k, v, g[:, :2], dtype, scale=scale, is_causal=True)
        assert_bwd(gpu, ref, f"scale={scale}", ctx=ctx)


def test_backward_small_and_degenerate():
    """One key (grad_query and grad_key 0), one query, more queries than keys under causal."""
    q, k, v = inputs.randn_qkv((1, 2, 40, 64), (1, 2, 1, 64), (1, 2, 1, 64), "bf16", seed=3)
    g = inputs.randn_qkv((1, 2, 40, 64), (1, 1, 1, 64), (1, 1, 1, 64), "bf16", seed=4)[0]
    gpu, ref, ctx = run_bwd(q, k, v, g, "bf16")
    assert_bwd(gpu, ref, "S=1", ctx=ctx)
    assert float(gpu[0].abs().max()) <= 1e-3
    q, k, v = inputs.randn_qkv((1, 2, 1, 64), (1, 2, 90, 64), (1, 2, 90, 64), "bf16", seed=13)
    g = inputs.randn_qkv((1, 2, 1, 64), (1, 1, 1, 64), (1, 1, 1, 64), "bf16", seed=14)[0]
    gpu, ref, ctx = run_bwd(q, k, v, g, "bf16")
    assert_bwd(gpu, ref, "L=1", ctx=ctx)
    q, k, v = inputs.randn_qkv((1, 1, 150, 96), (1, 1, 70, 96), (1, 1, 70, 96), "bf16", seed=5)
    g = inputs.randn_qkv((1, 1, 150, 96), (1, 1, 1, 96), (1, 1, 1, 96), "bf16", seed=6)[0]
    gpu, ref, ctx = run_bwd(q, k, v, g, "bf16", is_causal=True)
    assert_bwd(gpu, ref, "L>S causal", ctx=ctx)
    q, k, v = inputs.randn_qkv((1, 1, 70, 96), (1, 1, 150, 96), (1, 1, 150, 96), "bf16", seed=7)
    g = inputs.randn_qkv((1, 1, 70, 96), (1, 1, 1, 96), (1, 1, 1, 96), "bf16", seed=8)[0]
    gpu, ref, ctx = run_bwd(q, k, v, g, "bf16", is_causal=True)
    assert_bwd(gpu, ref, "L<S causal (keys past the last query get 0)", ctx=ctx)


def test_backward_headline_shape_full():
    """The bf16 causal B=4 H=16 L=S=2048 E=128 shape, in the launch configuration the
    benchmark times: gradients written into NaN-filled buffers, every (batch, head)
    against the oracle's backward (per-tensor bar, the oracle's heads in a thread
    pool), and two of them element by element against the per-element range."""
    q, k, v = inputs.workload_inputs("bf16_causal_e128")
    g = inputs.randn_qkv(tuple(q.shape), (1, 1, 1, 128), (1, 1, 1, 128), "bf16", seed=99)[0]
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    out, lse = S.sdpa_fwd(qd, kd, vd, is_causal=True)
    grads = tuple(torch.full(t.shape, float("nan"), dtype=t.dtype, device=DEV) for t in (qd, kd, vd))
    dq, dk, dv = S.sdpa_bwd(qd, kd, vd, out, lse, gd, is_causal=True, grads=grads)
    torch.cuda.synchronize()
    assert all(a.data_ptr() == b.data_ptr() for a, b in zip((dq, dk, dv), grads))
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    oc, lc = _np(out), _np(lse).reshape(out.shape[:-1])
    B, H = q.shape[0], q.shape[1]

    def one(bh):
        b, h = divmod(bh, H)
        return bh, O.sdpa_backward(q[b, h], k[b, h], v[b, h], g[b, h], is_causal=True)

    with ThreadPoolExecutor(8) as ex:
        for bh, ref in ex.map(one, range(B * H)):
            b, h = divmod(bh, H)
            assert_bwd((dq[b, h], dk[b, h], dv[b, h]), ref, f"headline b={b} h={h}")

    # per element on two heads (the model takes ~15 s a head on the host), in parallel
    def per_element(bh):
        b, h = bh
        ctx = dict(qkvg=(q[b, h], k[b, h], v[b, h], g[b, h]), kw=dict(is_causal=True), dtype="bf16",
                   out=oc[b, h], lse=lc[b, h])
        check_bwd_covered((dq[b, h], dk[b, h], dv[b, h]), ctx, f"headline b={b} h={h}")

    with ThreadPoolExecutor(2) as ex:
        list(ex.map(per_element, [(0, 0), (3, 15)]))


@pytest.mark.parametrize("dtype,E", [("fp16", 64), ("bf16", 96), ("bf16", 128)])
def test_backward_schedules_agree(dtype, E):
    """The schedule that stores dS^T (dQ from it in one product) and the one whose
    dQ kernel recomputes S and dP give bit-identical gradients: both form the same
    P, dP, D and dS, and add dQ's products in the same order (the stored schedule
    only adds exact zeros past a slice's causal limit).  Ragged lengths (not
    multiples of 64 or 128), causal or not, grouped heads, float and bool masks."""
    cases = [(2, 4, 2, 200, 333, False, None), (1, 4, 4, 300, 300, True, None), (1, 2, 1, 65, 129, True, None),
             (2, 2, 2, 150, 150, True, "float"), (1, 2, 2, 257, 190, False, "bool")]
    for ci, (B, Hq, Hkv, L, Sk, causal, mk) in enumerate(cases):
        q, k, v = inputs.randn_qkv((B, Hq, L, E), (B, Hkv, Sk, E), (B, Hkv, Sk, E), dtype, seed=ci + E)
        g = inputs.randn_qkv((B, Hq, L, E), (1, 1, 1, E), (1, 1, 1, E), dtype, seed=ci + E + 50)[0]
        m = None
        if mk is not None:
            m = _masks((B, Hq, L, Sk), seed=ci)[0 if mk == "float" else 1]
        qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
        md = None if m is None else m.to(DEV)
        out, lse = S.sdpa_fwd(qd, kd, vd, attn_mask=md, is_causal=causal, enable_gqa=True)
        a = S.sdpa_bwd(qd, kd, vd, out, lse, gd, attn_mask=md, is_causal=causal, enable_gqa=True, store_ds=True)
        b = S.sdpa_bwd(qd, kd, vd, out, lse, gd, attn_mask=md, is_causal=causal, enable_gqa=True, store_ds=False)
        torch.cuda.synchronize()
        for n, x, y in zip(("dq", "dk", "dv"), a, b):
            assert torch.equal(x, y), (f"case {ci} {n}: schedules differ, max "
                                       f"{float((x.float() - y.float()).abs().max()):.3e}")


def _masks(shape, seed):
    g = torch.Generator().manual_seed(seed)
    fm = torch.randn(shape, generator=g)
    fm[torch.rand(shape, generator=g) < 0.15] = float("-inf")
    bm = torch.rand(shape, generator=g) < 0.8
    return fm, bm


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("E", [64, 96, 128])
def test_backward_masks(dtype, E):
    """Float (bias with -inf) and bool masks, full and broadcast shapes, with and
    without causal; rows with no kept key contribute nothing; key counts that
    are and are not whole vectors of the mask's loads."""
    for (L, Sk, mshape, causal) in ((200, 256, "full", False), (150, 333, "row", True), (130, 130, "head", True)):
        q, k, v = inputs.randn_qkv((2, 2, L, E), (2, 2, Sk, E), (2, 2, Sk, E), dtype, seed=E + L)
        g = inputs.randn_qkv((2, 2, L, E), (1, 1, 1, E), (1, 1, 1, E), dtype, seed=E + L + 1)[0]
        shape = {"full": (2, 2, L, Sk), "row": (1, 1, L, Sk), "head": (1, 2, L, Sk)}[mshape]
        fm, bm = _masks(shape, E + Sk)
        fm[..., 5, :] = float("-inf")          # a row with no kept key
        bm[..., 7, :] = False
        for m, what in ((fm, "float"), (bm, "bool")):
            gpu, ref, ctx = run_bwd(q, k, v, g, dtype, attn_mask=m, is_causal=causal)
            assert_bwd(gpu, ref, f"{dtype} E={E} {what} {mshape} causal={causal}", ctx=ctx)
            assert float(gpu[0][..., 5 if what == "float" else 7, :].abs().max()) == 0.0


def test_backward_mask_gqa_and_scale():
    q, k, v = inputs.randn_qkv((1, 4, 190, 128), (1, 2, 190, 128), (1, 2, 190, 128), "bf16", seed=41)
    g = inputs.randn_qkv((1, 4, 190, 128), (1, 1, 1, 128), (1, 1, 1, 128), "bf16", seed=42)[0]
    fm, bm = _masks((1, 4, 190, 190), 43)
    for m in (fm, bm):
        for scale in (None, -0.3):
            gpu, ref, ctx = run_bwd(q, k, v, g, "bf16", attn_mask=m, is_causal=True, enable_gqa=True, scale=scale)
            assert_bwd(gpu, ref, f"gqa {m.dtype} scale={scale}", ctx=ctx)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("E", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_varlen(dtype, E, causal):
    """Packed segments (lengths 1, 37, 128, 129, 300), grouped heads: each
    segment's gradients against the oracle's backward of that segment alone
    (the block-diagonal mask)."""
    lengths = [1, 37, 128, 129, 300]
    q, k, v, cu = inputs.varlen_inputs(lengths, 4, 2, E, dtype, seed=E + 60)
    g = inputs.varlen_inputs(lengths, 4, 2, E, dtype, seed=E + 61)[0]
    qd, kd, vd, gd, cud = (t.to(DEV) for t in (q, k, v, g, cu))
    mx = max(lengths)
    out, lse = S.sdpa_fwd_varlen(qd, kd, vd, cud, max_seqlen_q=mx, max_seqlen_k=mx, is_causal=causal,
                                 enable_gqa=True)
    dq, dk, dv = S.sdpa_bwd_varlen(qd, kd, vd, out, lse, gd, cud, max_seqlen_q=mx, max_seqlen_k=mx,
                                   is_causal=causal, enable_gqa=True)
    torch.cuda.synchronize()
    c = cu.tolist()
    for i in range(len(lengths)):
        a, b = c[i], c[i + 1]
        seg = [t[0, a:b].permute(1, 0, 2)[None] for t in (q, k, v, g)]
        ref = O.sdpa_backward(*seg, is_causal=causal, enable_gqa=True)
        gpu = [t[0, a:b].permute(1, 0, 2)[None] for t in (dq, dk, dv)]
        ctx = dict(qkvg=seg, kw=dict(is_causal=causal, enable_gqa=True), dtype=dtype,
                   out=_np(out[0, a:b].permute(1, 0, 2)[None]), lse=_np(lse.reshape(-1, lse.shape[-1])[:, a:b])[None])
        assert_bwd(gpu, ref, f"{dtype} E={E} causal={causal} segment {i} (length {b - a})", ctx=ctx)


def _draw_bwd(rng):
    hkv = rng.choice([1, 2])
    return dict(dtype=rng.choice(["bf16", "fp16"]), B=rng.choice([1, 2]), Hkv=hkv, Hq=hkv * rng.choice([1, 2, 3]),
                L=rng.choice([1, 33, 128, 150, 257]), S=rng.choice([1, 40, 128, 200, 256, 333]),
                E=rng.choice([64, 96, 128]), causal=rng.random() < 0.5,
                mask=rng.choice([None, None, "float", "bool"]), mshape=rng.choice(["full", "row", "head", "batch"]),
                scale=rng.choice([None, None, 1.0, -0.3]))


BWD_CASES = [_draw_bwd(__import__("random").Random(500 + i)) for i in range(32)]


@pytest.mark.parametrize("ci", range(len(BWD_CASES)))
def test_backward_random_configuration(ci):
    """Seeded random shapes, heads, masks, causal and scales against the oracle's backward."""
    c = BWD_CASES[ci]
    q, k, v = inputs.randn_qkv((c["B"], c["Hq"], c["L"], c["E"]), (c["B"], c["Hkv"], c["S"], c["E"]),
                               (c["B"], c["Hkv"], c["S"], c["E"]), c["dtype"], seed=700 + ci)
    g = inputs.randn_qkv((c["B"], c["Hq"], c["L"], c["E"]), (1, 1, 1, c["E"]), (1, 1, 1, c["E"]), c["dtype"],
                         seed=800 + ci)[0]
    kw = dict(is_causal=c["causal"], scale=c["scale"], enable_gqa=c["Hq"] != c["Hkv"])
    if c["mask"] is not None:
        shape = {"full": (c["B"], c["Hq"], c["L"], c["S"]), "row": (1, 1, c["L"], c["S"]),
                 "head": (1, c["Hq"], c["L"], c["S"]), "batch": (c["B"], 1, 1, c["S"])}[c["mshape"]]
        fm, bm = _masks(shape, 900 + ci)
        kw["attn_mask"] = fm if c["mask"] == "float" else bm
    gpu, ref, ctx = run_bwd(q, k, v, g, c["dtype"], **kw)
    assert_bwd(gpu, ref, f"case {ci}: {c}", ctx=ctx)


VEC_DIMS = [(64, 128), (128, 64), (40, 40), (0, 32), (96, 24), (64, 64), (128, 128)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("E,Ev", VEC_DIMS)
def test_backward_vector_alu(dtype, E, Ev):
    """fp32 inputs, value rows of another width (Ev != E) and other head dims (E = 0
    included) run on the vector-ALU backward: masks (float with -inf entries and an
    empty row, bool), causal, grouped heads, signed and unit scales, ragged tiles."""
    if dtype != "fp32" and E == Ev and E in (64, 128):
        pytest.skip("bf16/fp16 with E == Ev in {64, 96, 128} run the matrix-core backward (tests above)")
    B, Hq, Hkv, L, Sk = 2, 4, 2, 150, 170
    q, k, v = inputs.randn_qkv((B, Hq, L, E), (B, Hkv, Sk, E), (B, Hkv, Sk, Ev), dtype, seed=E * 3 + Ev)
    g = inputs.randn_qkv((B, Hq, L, Ev), (1, 1, 1, 8), (1, 1, 1, 8), dtype, seed=E * 3 + Ev + 1)[0]
    gen = torch.Generator().manual_seed(E + Ev)
    fm = torch.randn((1, Hq, L, Sk), generator=gen)
    fm[torch.rand((1, Hq, L, Sk), generator=gen) < 0.1] = float("-inf")
    fm[..., 7, :] = float("-inf")
    bm = torch.rand((B, 1, L, Sk), generator=gen) < 0.8
    for m, causal, scale in ((None, False, None), (None, True, -0.3), (fm, True, None), (bm, False, 1.0)):
        gpu, ref, ctx = run_bwd(q, k, v, g, dtype, attn_mask=m, is_causal=causal, scale=scale, enable_gqa=True)
        assert_bwd(gpu, ref, f"{dtype} E={E} Ev={Ev} mask={None if m is None else m.dtype} causal={causal} "
                             f"scale={scale}", dtype, ctx=ctx)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("E,Ev", [(64, 64), (40, 72)])
def test_backward_vector_alu_packed(dtype, E, Ev):
    """Packed segments on the vector-ALU backward, causal and not, grouped heads."""
    lengths = [1, 37, 128, 129, 300]
    cu = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int32)
    tot = sum(lengths)
    q, k, v = inputs.randn_qkv((1, tot, 4, E), (1, tot, 2, E), (1, tot, 2, Ev), dtype, seed=E + Ev + 90)
    g = inputs.randn_qkv((1, tot, 4, Ev), (1, 1, 1, 8), (1, 1, 1, 8), dtype, seed=E + Ev + 91)[0]
    qd, kd, vd, gd, cud = (t.to(DEV) for t in (q, k, v, g, cu))
    for causal in (False, True):
        out, lse = S.sdpa_fwd_varlen(qd, kd, vd, cud, max_seqlen_q=300, max_seqlen_k=300, is_causal=causal,
                                     enable_gqa=True)
        dq, dk, dv = S.sdpa_bwd_varlen(qd, kd, vd, out, lse, gd, cud, max_seqlen_q=300, max_seqlen_k=300,
                                       is_causal=causal, enable_gqa=True)
        torch.cuda.synchronize()
        c = cu.tolist()
        for i in range(len(lengths)):
            a, b = c[i], c[i + 1]
            seg = [t[0, a:b].permute(1, 0, 2)[None] for t in (q, k, v, g)]
            ref = O.sdpa_backward(*seg, is_causal=causal, enable_gqa=True)
            gpu = [t[0, a:b].permute(1, 0, 2)[None] for t in (dq, dk, dv)]
            ctx = dict(qkvg=seg, kw=dict(is_causal=causal, enable_gqa=True), dtype=dtype,
                       out=_np(out[0, a:b].permute(1, 0, 2)[None]),
                       lse=_np(lse.reshape(-1, lse.shape[-1])[:, a:b])[None])
            assert_bwd(gpu, ref, f"{dtype} E={E} Ev={Ev} causal={causal} segment {i}", dtype, ctx=ctx)
