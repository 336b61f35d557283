"""Parity of attention against a paged key/value cache (sdpa_fwd_paged, through
the C interface) with the float64 oracle (oracle.sdpa_paged) on the same
bf16/fp16 values: decode steps (split-KV kernel) and chunks of many new rows
(chunked prefill, single-pass kernel).

Bars as for the forward: max |GPU - oracle| <= 2e-2 on the output and 1e-3 on
lse for bf16 / fp16.  Inputs: a shuffled page pool, ragged cached lengths
(0, 1, page, tile and split boundaries, fewer cached keys than new rows), GQA,
bottom-right causal, and table entries outside the pool.
"""
import numpy as np
import pytest
import torch

from oracle import sdpa_oracle as O
from transformer_attention_04_amd import inputs
from transformer_attention_04_amd import sdpa as S

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {"bf16": (2e-2, 1e-3), "fp16": (2e-2, 1e-3)}


def make_cache(B, Hq, Hkv, L, E, ps, lens, dtype, seed, extra_pages=7, extra_blocks=0):
    """Query rows, a shuffled page pool holding every sequence's blocks, the
    table (with ``extra_blocks`` spare columns past the longest sequence)."""
    maxb = max(1, max((n + ps - 1) // ps for n in lens)) + extra_blocks
    n_pages = B * maxb + extra_pages
    q, kc, vc = inputs.randn_qkv((B, Hq, L, E), (n_pages, Hkv, ps, E), (n_pages, Hkv, ps, E), dtype, seed)
    g = torch.Generator().manual_seed(seed + 1)
    perm = torch.randperm(n_pages, generator=g)[:B * maxb]
    bt = perm.reshape(B, maxb).to(torch.int32)
    return q, kc, vc, bt, torch.tensor(lens, dtype=torch.int32)


def run(q, kc, vc, bt, lens, dtype, **kw):
    out, lse = S.sdpa_fwd_paged(q.to(DEV), kc.to(DEV), vc.to(DEV), bt.to(DEV), lens.to(DEV),
                                max_seq_len=int(lens.max()) if lens.numel() else 0, **kw)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), lse.cpu().double().numpy()


def check(gpu, ref, dtype, what):
    (out, lse), (ro, rl) = gpu, ref
    tol_o, tol_l = TOL[dtype]
    empty = np.isneginf(rl)
    assert np.isneginf(lse[empty]).all() and (out[empty] == 0).all(), f"{what}: empty rows"
    fin = np.isfinite(rl)
    eo = np.abs(out[fin] - ro[fin]).max(initial=0.0)
    el = np.abs(lse[fin] - rl[fin]).max(initial=0.0)
    assert eo <= tol_o and el <= tol_l, f"{what}: out err {eo:.3e}, lse err {el:.3e}"


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("E", [64, 96, 128])
@pytest.mark.parametrize("ps", [16, 64])
def test_paged_ragged_lengths(dtype, E, ps):
    lens = [0, 1, 15, 16, 17, 64, 129, 700, 1000]
    B = len(lens)
    q, kc, vc, bt, ln = make_cache(B, 8, 2, 1, E, ps, lens, dtype, seed=E + ps)
    ref = O.sdpa_paged(q, kc, vc, bt, ln, enable_gqa=True)
    check(run(q, kc, vc, bt, ln, dtype, enable_gqa=True), ref, dtype, f"E={E} ps={ps}")
    # several splits per sequence
    check(run(q, kc, vc, bt, ln, dtype, enable_gqa=True, num_splits=5), ref, dtype, f"E={E} ps={ps} 5 splits")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_paged_bottom_right_causal(dtype):
    lens = [2, 33, 300, 513]
    q, kc, vc, bt, ln = make_cache(len(lens), 4, 2, 2, 128, 32, lens, dtype, seed=21)
    for causal in (False, True):
        ref = O.sdpa_paged(q, kc, vc, bt, ln, is_causal=causal, enable_gqa=True)
        check(run(q, kc, vc, bt, ln, dtype, is_causal=causal, enable_gqa=True, num_splits=3), ref, dtype,
              f"L=2 causal={causal}")
    # one new row with causal: every cached key is kept
    ref = O.sdpa_paged(q[:, :, :1], kc, vc, bt, ln, is_causal=True, enable_gqa=True)
    check(run(q[:, :, :1].contiguous(), kc, vc, bt, ln, dtype, is_causal=True, enable_gqa=True), ref, dtype,
          "L=1 causal")


def test_paged_bad_table_entry_gives_nan_rows():
    lens = [100, 100]   # blocks 0..6 of 16 keys; the table has 2 spare columns
    q, kc, vc, bt, ln = make_cache(2, 2, 2, 1, 64, 16, lens, "bf16", seed=31, extra_blocks=2)
    bt = bt.clone()
    bt[1, 3] = kc.shape[0] + 5     # outside the pool, inside sequence 1's kept range
    out, lse = run(q, kc, vc, bt, ln, "bf16")
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    ref = O.sdpa_paged(q[:1], kc, vc, bt[:1], ln[:1])
    check((out[:1], lse[:1]), ref, "bf16", "good sequence beside a bad one")
    # entries past the cached length are never read
    bt2 = bt.clone()
    bt2[1, 3] = bt[0, 3]
    bt2[1, 7] = -1
    bt2[1, 8] = 1 << 30
    out, lse = run(q, kc, vc, bt2, ln, "bf16")
    assert np.isfinite(out).all()
    check((out, lse), O.sdpa_paged(q, kc, vc, bt2[:, :7], ln), "bf16", "spare table columns")


def test_paged_full_decode_shape_sampled():
    """B=64, Hq=32, Hkv=8, 32768 cached keys each, E=128, 64-key pages in a
    shuffled pool; four sequences checked against the oracle."""
    B, Hq, Hkv, E, ps, S = 64, 32, 8, 128, 64, 32768
    q, kc, vc, bt, ln = make_cache(B, Hq, Hkv, 1, E, ps, [S] * B, "bf16", seed=0, extra_pages=0)
    out, lse = run(q, kc, vc, bt, ln, "bf16", enable_gqa=True)
    for b in (0, 9, 31, 63):
        ref = O.sdpa_paged(q[b:b + 1], kc, vc, bt[b:b + 1], ln[b:b + 1], enable_gqa=True)
        check((out[b:b + 1], lse[b:b + 1]), ref, "bf16", f"sequence {b}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("E", [64, 96, 128])
@pytest.mark.parametrize("ps", [16, 64, 256])
def test_paged_chunked_prefill(dtype, E, ps):
    """200 new rows per sequence (two query tiles, the second ragged) against
    ragged cached lengths, some shorter than the chunk (causal rows before the
    cache's first key keep nothing)."""
    lens = [0, 100, 200, 201, 333, 700, 1000]
    q, kc, vc, bt, ln = make_cache(len(lens), 8, 2, 200, E, ps, lens, dtype, seed=E + ps + 1)
    for causal in (False, True):
        ref = O.sdpa_paged(q, kc, vc, bt, ln, is_causal=causal, enable_gqa=True)
        check(run(q, kc, vc, bt, ln, dtype, is_causal=causal, enable_gqa=True), ref, dtype,
              f"E={E} ps={ps} causal={causal}")


def test_paged_chunked_prefill_no_gqa_and_scale():
    lens = [37, 64, 65, 300]
    q, kc, vc, bt, ln = make_cache(len(lens), 2, 2, 40, 128, 32, lens, "bf16", seed=77)
    for scale in (-0.3, 1.0):
        ref = O.sdpa_paged(q, kc, vc, bt, ln, is_causal=True, scale=scale)
        check(run(q, kc, vc, bt, ln, "bf16", is_causal=True, scale=scale), ref, "bf16", f"scale={scale}")


@pytest.mark.parametrize("E,ps,dtype", [(64, 16, "fp16"), (128, 16, "bf16"), (96, 64, "fp16"), (128, 32, "bf16")])
def test_paged_chunked_prefill_bad_table_entry(E, ps, dtype):
    """A page outside the pool holding keys 240.. of sequence 1 (the page of
    key 240): causal rows that keep one of its keys are NaN, earlier rows and
    sequence 0 are unaffected (eight-wave kernel: the K rows of such a page come
    from its block of NaN rows, the whole block at E = 128)."""
    lens = [300, 300]
    q, kc, vc, bt, ln = make_cache(2, 4, 2, 100, E, ps, lens, dtype, seed=91 + E + ps)
    bad = bt.clone()
    blk = 240 // ps
    bad[1, blk] = kc.shape[0] + 3
    # row i keeps keys <= 200 + i: rows from the page's first key - 200 on keep it
    r0 = max(0, blk * ps - 200)
    out, lse = run(q, kc, vc, bad, ln, dtype, is_causal=True, enable_gqa=True)
    assert np.isnan(out[1, :, r0:]).all() and np.isnan(lse[1, :, r0:]).all()
    ref = O.sdpa_paged(q, kc, vc, bt, ln, is_causal=True, enable_gqa=True)
    check((out[:1], lse[:1]), (ref[0][:1], ref[1][:1]), dtype, "good sequence")
    if r0 > 0:
        check((out[1:, :, :r0], lse[1:, :, :r0]), (ref[0][1:, :, :r0], ref[1][1:, :, :r0]), dtype,
              "rows before the bad page")


@pytest.mark.parametrize("case", ["padded_rows", "257_pages", "256_pages", "zero_scale"])
def test_paged_chunked_prefill_kernel_choice(case):
    """Chunked prefill takes the eight-wave kernel when pool rows are
    contiguous, a sequence spans at most 256 pages and the scale is not 0, and
    the four-wave kernel otherwise: both sides of each condition against the
    oracle (a pool whose rows are padded to E + 8, 257 and 256 pages of 16 keys
    in one sequence, a zero scale)."""
    E, ps = 64, 16
    lens = {"257_pages": [4100, 900], "256_pages": [4096, 900]}.get(case, [700, 333])
    q, kc, vc, bt, ln = make_cache(len(lens), 4, 2, 40, E, ps, lens, "bf16", seed=len(case) + 3)
    kw = dict(is_causal=True, enable_gqa=True)
    if case == "zero_scale":
        kw["scale"] = 0.0
    kd, vd = kc, vc
    if case == "padded_rows":
        kd = torch.zeros(kc.shape[:3] + (E + 8,), dtype=kc.dtype)
        vd = torch.zeros(vc.shape[:3] + (E + 8,), dtype=vc.dtype)
        kd[..., :E], vd[..., :E] = kc, vc
        kd, vd = kd.to(DEV)[..., :E], vd.to(DEV)[..., :E]
        assert kd.stride(2) == E + 8
    ref = O.sdpa_paged(q, kc, vc, bt, ln, **kw)
    check(run(q, kd, vd, bt, ln, "bf16", **kw), ref, "bf16", case)


def test_paged_chunked_prefill_full_shape_sampled():
    """B=8 sequences of 4096 cached keys whose last 512 are the new chunk,
    Hq=32, Hkv=8, E=128, 64-key pages in a shuffled pool, causal; query heads
    of the first and last cache head of three sequences checked."""
    B, Hq, Hkv, E, ps, S, L = 8, 32, 8, 128, 64, 4096, 512
    q, kc, vc, bt, ln = make_cache(B, Hq, Hkv, L, E, ps, [S] * B, "bf16", seed=5, extra_pages=0)
    out, lse = run(q, kc, vc, bt, ln, "bf16", is_causal=True, enable_gqa=True)
    for b in (0, 3, 7):
        for g in (0, Hkv - 1):
            hs = slice(4 * g, 4 * g + 4)
            ref = O.sdpa_paged(q[b:b + 1, hs], kc[:, g:g + 1], vc[:, g:g + 1], bt[b:b + 1], ln[b:b + 1],
                               is_causal=True, enable_gqa=True)
            check((out[b:b + 1, hs], lse[b:b + 1, hs]), ref, "bf16", f"sequence {b} cache head {g}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("E", [64, 128])
@pytest.mark.parametrize("ps", [16, 64])
def test_paged_packed_rows(dtype, E, ps):
    """Packed new rows, a different count per sequence (0, 1, a partial tile,
    several tiles, more rows than cached keys), against a shuffled page pool,
    grouped heads, causal and not: parity with oracle.sdpa_paged_varlen."""
    lens = [5, 300, 64, 1000, 130]
    counts = [1, 0, 64, 300, 200]
    q4, kc, vc, bt, ln = make_cache(len(lens), 8, 2, 1, E, ps, lens, dtype, seed=E + ps + 3)
    cu = torch.tensor([0] + list(np.cumsum(counts)), dtype=torch.int32)
    q = inputs.randn_qkv((int(cu[-1]), 8, E), (1, 1, E), (1, 1, E), dtype, seed=E + ps + 4)[0]
    for causal in (False, True):
        out, lse = S.sdpa_fwd_paged_varlen(q.to(DEV), cu.to(DEV), kc.to(DEV), vc.to(DEV), bt.to(DEV), ln.to(DEV),
                                           is_causal=causal, enable_gqa=True)
        torch.cuda.synchronize()
        ro, rl = O.sdpa_paged_varlen(q, cu, kc, vc, bt, ln, is_causal=causal, enable_gqa=True)
        # lse (Hq, total) -> (total, Hq), the leading dims of out
        check((out.cpu().double().numpy(), lse.cpu().double().numpy().T), (ro, rl.T), dtype,
              f"E={E} ps={ps} causal={causal}")


@pytest.mark.parametrize("dtype,E,ps", [("bf16", 64, 16), ("fp16", 96, 64), ("bf16", 128, 32), ("fp16", 128, 256)])
def test_paged_packed_rows_even_counts(dtype, E, ps):
    """Packed new rows of about equal counts per sequence (at least 3/4 of
    n_seqs x the largest count: the eight-wave kernel): counts 300, 280, 290,
    240, 300, 0 (the second 256-row tile of the 240-row sequence is empty, and
    both tiles of the last one) against cached lengths 1000, 250 (fewer keys
    than new rows), 700, 2000, 300, 64, grouped heads, causal and not; then a
    page outside the pool in sequence 3."""
    lens = [1000, 250, 700, 2000, 300, 64]
    counts = [300, 280, 290, 240, 300, 0]
    q4, kc, vc, bt, ln = make_cache(len(lens), 8, 2, 1, E, ps, lens, dtype, seed=E + ps + 13)
    cu = torch.tensor([0] + list(np.cumsum(counts)), dtype=torch.int32)
    q = inputs.randn_qkv((int(cu[-1]), 8, E), (1, 1, E), (1, 1, E), dtype, seed=E + ps + 14)[0]
    assert 4 * sum(counts) >= 3 * len(counts) * max(counts)

    def run_packed(table, causal):
        out, lse = S.sdpa_fwd_paged_varlen(q.to(DEV), cu.to(DEV), kc.to(DEV), vc.to(DEV), table.to(DEV),
                                           ln.to(DEV), is_causal=causal, enable_gqa=True)
        torch.cuda.synchronize()
        return out.cpu().double().numpy(), lse.cpu().double().numpy().T

    for causal in (False, True):
        ro, rl = O.sdpa_paged_varlen(q, cu, kc, vc, bt, ln, is_causal=causal, enable_gqa=True)
        check(run_packed(bt, causal), (ro, rl.T), dtype, f"E={E} ps={ps} causal={causal}")
    # a page outside the pool at key 1200 of sequence 3 (2000 keys, 240 new rows at
    # positions 1760..): every causal row of that sequence keeps it, the others do not read it
    bad = bt.clone()
    bad[3, 1200 // ps] = kc.shape[0] + 5
    out, lse = run_packed(bad, True)
    a, e = int(cu[3]), int(cu[4])
    assert np.isnan(out[a:e]).all() and np.isnan(lse[a:e]).all()
    ro, rl = O.sdpa_paged_varlen(q, cu, kc, vc, bt, ln, is_causal=True, enable_gqa=True)
    keep = np.r_[0:a, e:int(cu[-1])]
    check((out[keep], lse[keep]), (ro[keep], rl.T[keep]), dtype, "sequences without the bad page")


def test_paged_packed_rows_full_shape_sampled():
    """The chunked-prefill shape as packed rows (sdpa_fwd_paged_varlen, the
    eight-wave kernel with its pairs numbered by XCD): 8 sequences of 512 new
    rows on 4096 cached keys, Hq=32, Hkv=8, E=128, 64-key pages, causal; the
    query heads of the first and last cache head of three sequences checked."""
    B, Hq, Hkv, E, ps, Sk, L = 8, 32, 8, 128, 64, 4096, 512
    q, kc, vc, bt, ln = make_cache(B, Hq, Hkv, L, E, ps, [Sk] * B, "bf16", seed=6, extra_pages=0)
    qp = q.permute(0, 2, 1, 3).reshape(B * L, Hq, E).contiguous()
    cu = torch.arange(0, B + 1, dtype=torch.int32) * L
    out, lse = S.sdpa_fwd_paged_varlen(qp.to(DEV), cu.to(DEV), kc.to(DEV), vc.to(DEV), bt.to(DEV), ln.to(DEV),
                                       is_causal=True, enable_gqa=True)
    torch.cuda.synchronize()
    out = out.cpu().double().numpy()           # (B * L, Hq, E)
    lse = lse.cpu().double().numpy()           # (Hq, B * L)
    for b in (0, 4, 7):
        for g in (0, Hkv - 1):
            hs = slice(4 * g, 4 * g + 4)
            ro, rl = O.sdpa_paged(q[b:b + 1, hs], kc[:, g:g + 1], vc[:, g:g + 1], bt[b:b + 1], ln[b:b + 1],
                                  is_causal=True, enable_gqa=True)
            go = out[b * L:(b + 1) * L, hs].transpose(1, 0, 2)[None]
            gl = lse[hs, b * L:(b + 1) * L][None]
            check((go, gl), (ro, rl), "bf16", f"packed sequence {b} cache head {g}")
