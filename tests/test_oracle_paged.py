"""Pins of the oracle's paged-cache attention (CPU, float64).

oracle.sdpa_paged gathers each sequence's keys and values page by page and
runs the (separately pinned) dense attention.  What fixes it:
  * an in-order block table over a contiguous cache = the dense oracle on
    that cache, and a shuffled page pool = the dense oracle on the keys
    gathered independently with numpy fancy indexing;
  * ragged cached lengths = dense attention on each sequence's prefix;
  * bottom-right causal alignment: with L equal to the cached length it is
    the ordinary (top-left) causal mask; a brute-force loop fixes the general
    case; L = 1 is the same as no mask;
  * table entries outside the page pool are refused.
"""
import math

import numpy as np
import pytest

from oracle import sdpa_oracle as O


def _pool(rng, n_pages, hkv, ps, e):
    return rng.standard_normal((n_pages, hkv, ps, e)), rng.standard_normal((n_pages, hkv, ps, e))


def test_in_order_table_is_the_dense_cache():
    rng = np.random.default_rng(1)
    B, Hq, Hkv, L, E, ps, nblk = 2, 4, 2, 1, 8, 16, 5
    kc, vc = _pool(rng, B * nblk, Hkv, ps, E)
    q = rng.standard_normal((B, Hq, L, E))
    bt = np.arange(B * nblk).reshape(B, nblk)
    S = nblk * ps
    out, lse = O.sdpa_paged(q, kc, vc, bt, [S, S], enable_gqa=True)
    kd = kc.reshape(B, nblk, Hkv, ps, E).transpose(0, 2, 1, 3, 4).reshape(B, Hkv, S, E)
    vd = vc.reshape(B, nblk, Hkv, ps, E).transpose(0, 2, 1, 3, 4).reshape(B, Hkv, S, E)
    ro, rl = O.sdpa(q, kd, vd, enable_gqa=True)
    assert np.abs(out - ro).max() < 1e-13 and np.abs(lse - rl).max() < 1e-13


def test_shuffled_pool_and_ragged_lengths():
    rng = np.random.default_rng(2)
    B, Hq, Hkv, L, E, ps, maxb = 3, 2, 2, 2, 8, 16, 6
    n_pages = 40
    kc, vc = _pool(rng, n_pages, Hkv, ps, E)
    q = rng.standard_normal((B, Hq, L, E))
    bt = rng.permutation(n_pages)[:B * maxb].reshape(B, maxb)
    lens = [1, 37, 96]
    out, lse = O.sdpa_paged(q, kc, vc, bt, lens)
    for b, n in enumerate(lens):
        rows = np.arange(n)
        kb = kc[bt[b, rows // ps], :, rows % ps, :].transpose(1, 0, 2)   # (Hkv, n, E), gathered directly
        vb = vc[bt[b, rows // ps], :, rows % ps, :].transpose(1, 0, 2)
        ro, rl = O.sdpa(q[b], kb, vb)
        assert np.abs(out[b] - ro).max() < 1e-13 and np.abs(lse[b] - rl).max() < 1e-13


def test_bottom_right_causal():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, E, ps = 2, 2, 1, 4, 16
    kc, vc = _pool(rng, 8, Hkv, ps, E)
    bt = np.array([[3, 1, 6, 0], [2, 5, 7, 4]])
    # L equal to the cached length: the ordinary causal mask
    n = 21
    q = rng.standard_normal((B, Hq, n, E))
    out, lse = O.sdpa_paged(q, kc, vc, bt, [n, n], is_causal=True, enable_gqa=True)
    for b in range(B):
        rows = np.arange(n)
        kb = kc[bt[b, rows // ps], :, rows % ps, :].transpose(1, 0, 2)
        vb = vc[bt[b, rows // ps], :, rows % ps, :].transpose(1, 0, 2)
        ro, rl = O.sdpa(q[b], kb, vb, is_causal=True, enable_gqa=True)
        assert np.abs(out[b] - ro).max() < 1e-13
    # general case against a pure-Python loop
    L, lens = 3, [40, 9]
    q = rng.standard_normal((B, Hq, L, E))
    out, lse = O.sdpa_paged(q, kc, vc, bt, lens, is_causal=True, enable_gqa=True)
    for b, n in enumerate(lens):
        for h in range(Hq):
            for i in range(L):
                keep = [j for j in range(n) if j <= n - L + i]
                sc = [sum(q[b, h, i, e] * kc[bt[b, j // ps], 0, j % ps, e] for e in range(E)) / math.sqrt(E)
                      for j in keep]
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                tot = sum(w)
                for e in range(E):
                    ref = sum(wj * vc[bt[b, j // ps], 0, j % ps, e] for wj, j in zip(w, keep)) / tot
                    assert abs(out[b, h, i, e] - ref) < 1e-12
                assert abs(lse[b, h, i] - (m + math.log(tot))) < 1e-12
    # one new row: causal keeps every cached key
    q1 = q[:, :, :1]
    a = O.sdpa_paged(q1, kc, vc, bt, lens, is_causal=True, enable_gqa=True)
    c = O.sdpa_paged(q1, kc, vc, bt, lens, is_causal=False, enable_gqa=True)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


def test_out_of_range_pages_refused():
    rng = np.random.default_rng(4)
    kc, vc = _pool(rng, 4, 1, 16, 4)
    q = rng.standard_normal((1, 1, 1, 4))
    with pytest.raises(ValueError):
        O.sdpa_paged(q, kc, vc, np.array([[0, 4]]), [20])
    with pytest.raises(ValueError):
        O.sdpa_paged(q, kc, vc, np.array([[0, 1]]), [40])   # more keys than the table covers
    # entries past the needed blocks are never looked at
    out, _ = O.sdpa_paged(q, kc, vc, np.array([[2, 99]]), [16])
    assert np.isfinite(out).all()


def test_no_cached_keys_is_an_empty_row():
    """Full specification: a row with no kept key has weight 0 on every key, so
    its output is 0 and its lse is log(0) = -inf (here: nothing cached)."""
    rng = np.random.default_rng(5)
    kc, vc = _pool(rng, 3, 1, 16, 4)
    q = rng.standard_normal((2, 1, 1, 4))
    out, lse = O.sdpa_paged(q, kc, vc, np.array([[0], [1]]), [0, 5])
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all()
    assert np.isfinite(out[1]).all()
    o, l_ = O.sdpa(q[0], np.zeros((1, 0, 4)), np.zeros((1, 0, 4)))
    assert o.shape == (1, 1, 4) and (o == 0).all() and np.isneginf(l_).all()


def test_packed_rows_per_sequence():
    """sdpa_paged_varlen: packed new rows of different counts per sequence.
    Fixed against dense attention over all packed rows and all sequences'
    gathered keys at once, with one explicit bias: a key of another sequence
    is -inf, and (causal) row r of sequence b keeps its own key j iff
    j <= n_b - L_b + r; and, when every sequence has the same count, against
    the batched sdpa_paged."""
    rng = np.random.default_rng(11)
    Hq, Hkv, E, Ev, ps = 4, 2, 8, 6, 16
    lens = [5, 40, 17, 33]
    counts = [3, 0, 17, 40]                   # new rows per sequence (more than cached for the last)
    nblk = [(n + ps - 1) // ps for n in lens]
    n_pages = sum(nblk) + 3
    kc = rng.standard_normal((n_pages, Hkv, ps, E))
    vc = rng.standard_normal((n_pages, Hkv, ps, Ev))
    perm = rng.permutation(n_pages)
    bt = np.zeros((len(lens), max(nblk)), dtype=np.int64)
    pos = 0
    for b, nb in enumerate(nblk):
        bt[b, :nb] = perm[pos:pos + nb]
        pos += nb
    cu = np.concatenate([[0], np.cumsum(counts)])
    q = rng.standard_normal((int(cu[-1]), Hq, E))
    for causal in (False, True):
        out, lse = O.sdpa_paged_varlen(q, cu, kc, vc, bt, lens, is_causal=causal, enable_gqa=True)
        # dense reference: every sequence's keys gathered by hand, one packed bias
        keys = [np.concatenate([kc[bt[b, j]] for j in range(nblk[b])], axis=1)[:, :lens[b]] for b in range(4)]
        vals = [np.concatenate([vc[bt[b, j]] for j in range(nblk[b])], axis=1)[:, :lens[b]] for b in range(4)]
        K, V = np.concatenate(keys, axis=1)[None], np.concatenate(vals, axis=1)[None]
        koff = np.concatenate([[0], np.cumsum(lens)])
        bias = np.full((int(cu[-1]), int(koff[-1])), -np.inf)
        for b in range(4):
            for r in range(counts[b]):
                for j in range(lens[b]):
                    if not causal or j <= lens[b] - counts[b] + r:
                        bias[cu[b] + r, koff[b] + j] = 0.0
        ro, rl = O.sdpa(np.transpose(q, (1, 0, 2))[None], K, V, attn_mask=bias, enable_gqa=True)
        fin = np.isfinite(rl[0])
        assert np.array_equal(np.isneginf(lse), np.isneginf(rl[0]))
        assert np.abs(lse[fin] - rl[0][fin]).max() < 1e-12
        assert np.abs(out - np.transpose(ro[0], (1, 0, 2))).max() < 1e-12
    # equal counts: the batched function on the same rows
    cnt = 7
    cu2 = np.arange(5) * cnt
    q2 = rng.standard_normal((4 * cnt, Hq, E))
    o2, l2 = O.sdpa_paged_varlen(q2, cu2, kc, vc, bt, lens, is_causal=True, enable_gqa=True)
    ob, lb = O.sdpa_paged(np.transpose(q2.reshape(4, cnt, Hq, E), (0, 2, 1, 3)), kc, vc, bt, lens,
                          is_causal=True, enable_gqa=True)
    assert np.abs(o2 - np.transpose(ob, (0, 2, 1, 3)).reshape(4 * cnt, Hq, Ev)).max() < 1e-13
    fin = np.isfinite(lb)
    assert np.abs(np.transpose(l2.reshape(Hq, 4, cnt), (1, 0, 2))[fin] - lb[fin]).max() < 1e-13
