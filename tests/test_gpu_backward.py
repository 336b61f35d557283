"""Parity of the backward kernels (through the C interface) with the float64 oracle.

The forward runs on the GPU (sdpa_fwd) to give out and lse; the backward
(sdpa_bwd) then gives grad_query, grad_key, grad_value, compared element by
element with oracle.sdpa_backward on the same bf16/fp16 input values.

Bar (derived in the backward section of the design notes): for every output
tensor, max |GPU - oracle| <= 2^-6 * max|oracle| + 1e-3.  The GPU rounds P and
dS to the input format before their products (relative 2^-9 per term for
bf16), forms D from the rounded forward output, and rounds each gradient once.
"""
import numpy as np
import pytest
import torch

from oracle import sdpa_oracle as O
from transformer_attention_04_amd import inputs
from transformer_attention_04_amd import sdpa as S

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.detach().cpu().double().numpy()


def bwd_bar(ref):
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
    return (dq, dk, dv), O.sdpa_backward(q, k, v, g, **kw)


def assert_bwd(gpu, ref, what):
    errs = []
    for a, r, n in zip(gpu, ref, ("dq", "dk", "dv")):
        a = _np(a)
        assert a.shape == r.shape, (what, n, a.shape, r.shape)
        assert np.isfinite(a).all(), f"{what}: non-finite {n}"
        e = float(np.abs(a - r).max(initial=0.0))
        errs.append((e, e / bwd_bar(r)))
        assert e <= bwd_bar(r), f"{what}: max |{n} error| {e:.3e} > {bwd_bar(r):.3e} (max|ref| {np.abs(r).max():.3e})"
    print(f"{what}: max error (fraction of the bar) " +
          " ".join(f"{n} {e:.2e} ({f:.2f})" for n, (e, f) in zip(("dq", "dk", "dv"), errs)))
    return errs


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("E", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_ragged(dtype, E, causal):
    """Several query and key tiles with ragged tails (L, S not multiples of 64 or 128)."""
    L, Sk = (300, 300) if causal else (200, 333)
    q, k, v = inputs.randn_qkv((2, 3, L, E), (2, 3, Sk, E), (2, 3, Sk, E), dtype, seed=E + L)
    g = inputs.randn_qkv((2, 3, L, E), (1, 1, 1, E), (1, 1, 1, E), dtype, seed=E + L + 1)[0]
    gpu, ref = run_bwd(q, k, v, g, dtype, is_causal=causal)
    assert_bwd(gpu, ref, f"{dtype} E={E} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_backward_gqa_and_scales(dtype):
    """Grouped-query heads (grad_key/grad_value summed over the group), negative and unit scales."""
    q, k, v = inputs.randn_qkv((1, 6, 257, 128), (1, 2, 257, 128), (1, 2, 257, 128), dtype, seed=11)
    g = inputs.randn_qkv((1, 6, 257, 128), (1, 1, 1, 128), (1, 1, 1, 128), dtype, seed=12)[0]
    for causal in (False, True):
        gpu, ref = run_bwd(q, k, v, g, dtype, is_causal=causal, enable_gqa=True)
        assert_bwd(gpu, ref, f"gqa causal={causal}")
    for scale in (-0.09, 1.0):
        gpu, ref = run_bwd(q[:, :2], k, v, g[:, :2], dtype, scale=scale, is_causal=True)
        assert_bwd(gpu, ref, f"scale={scale}")


def test_backward_small_and_degenerate():
    """One key (grad_query and grad_key 0), one query, more queries than keys under causal."""
    q, k, v = inputs.randn_qkv((1, 2, 40, 64), (1, 2, 1, 64), (1, 2, 1, 64), "bf16", seed=3)
    g = inputs.randn_qkv((1, 2, 40, 64), (1, 1, 1, 64), (1, 1, 1, 64), "bf16", seed=4)[0]
    gpu, ref = run_bwd(q, k, v, g, "bf16")
    assert_bwd(gpu, ref, "S=1")
    assert float(gpu[0].abs().max()) <= 1e-3
    q, k, v = inputs.randn_qkv((1, 2, 1, 64), (1, 2, 90, 64), (1, 2, 90, 64), "bf16", seed=13)
    g = inputs.randn_qkv((1, 2, 1, 64), (1, 1, 1, 64), (1, 1, 1, 64), "bf16", seed=14)[0]
    gpu, ref = run_bwd(q, k, v, g, "bf16")
    assert_bwd(gpu, ref, "L=1")
    q, k, v = inputs.randn_qkv((1, 1, 150, 96), (1, 1, 70, 96), (1, 1, 70, 96), "bf16", seed=5)
    g = inputs.randn_qkv((1, 1, 150, 96), (1, 1, 1, 96), (1, 1, 1, 96), "bf16", seed=6)[0]
    gpu, ref = run_bwd(q, k, v, g, "bf16", is_causal=True)
    assert_bwd(gpu, ref, "L>S causal")
    q, k, v = inputs.randn_qkv((1, 1, 70, 96), (1, 1, 150, 96), (1, 1, 150, 96), "bf16", seed=7)
    g = inputs.randn_qkv((1, 1, 70, 96), (1, 1, 1, 96), (1, 1, 1, 96), "bf16", seed=8)[0]
    gpu, ref = run_bwd(q, k, v, g, "bf16", is_causal=True)
    assert_bwd(gpu, ref, "L<S causal (keys past the last query get 0)")


def test_backward_headline_shape_sampled():
    """The bf16 causal B=4 H=16 L=S=2048 E=128 shape, in the launch configuration the
    benchmark times; five (batch, head) slices checked against the oracle."""
    q, k, v = inputs.workload_inputs("bf16_causal_e128")
    g = inputs.randn_qkv(tuple(q.shape), (1, 1, 1, 128), (1, 1, 1, 128), "bf16", seed=99)[0]
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    out, lse = S.sdpa_fwd(qd, kd, vd, is_causal=True)
    dq, dk, dv = S.sdpa_bwd(qd, kd, vd, out, lse, gd, is_causal=True)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (1, 7), (2, 15), (3, 3), (3, 15)]:
        ref = O.sdpa_backward(q[b, h], k[b, h], v[b, h], g[b, h], is_causal=True)
        assert_bwd((dq[b, h], dk[b, h], dv[b, h]), ref, f"headline b={b} h={h}")


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
            gpu, ref = run_bwd(q, k, v, g, dtype, attn_mask=m, is_causal=causal)
            assert_bwd(gpu, ref, f"{dtype} E={E} {what} {mshape} causal={causal}")
            assert float(gpu[0][..., 5 if what == "float" else 7, :].abs().max()) == 0.0


def test_backward_mask_gqa_and_scale():
    q, k, v = inputs.randn_qkv((1, 4, 190, 128), (1, 2, 190, 128), (1, 2, 190, 128), "bf16", seed=41)
    g = inputs.randn_qkv((1, 4, 190, 128), (1, 1, 1, 128), (1, 1, 1, 128), "bf16", seed=42)[0]
    fm, bm = _masks((1, 4, 190, 190), 43)
    for m in (fm, bm):
        for scale in (None, -0.3):
            gpu, ref = run_bwd(q, k, v, g, "bf16", attn_mask=m, is_causal=True, enable_gqa=True, scale=scale)
            assert_bwd(gpu, ref, f"gqa {m.dtype} scale={scale}")


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
        assert_bwd(gpu, ref, f"{dtype} E={E} causal={causal} segment {i} (length {b - a})")


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
    gpu, ref = run_bwd(q, k, v, g, c["dtype"], **kw)
    assert_bwd(gpu, ref, f"case {ci}: {c}")
