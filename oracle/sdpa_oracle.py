"""CPU oracle for exact scaled dot-product attention (forward and backward), in float64.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The HIP
product path never does, and shares no code with it.

What it computes (exactref.ai, ``scaled_dot_product_attention``, sections
"Arguments" and "Full specification"): for query (..., L, E), key (..., S, E),
value (..., S, Ev)

    logits = scale * (Q K^T) + bias        (the mask is added after scaling)
    P      = softmax(logits) over the key axis
    out    = P V
    lse    = log(sum_j exp(logits_j))      per query row

The steps follow the "standard attention" the khchao.com NN Lab page describes
in "The Memory Hierarchy Bottleneck in Standard Attention": the full score
matrix S, then the full weight matrix A, then A V, all materialised (here in
host RAM, float64).  Inputs are upcast exactly from whatever dtype they hold;
nothing is rounded back to a narrow format.  numpy's matmul serves as the one
library step (the dot products).

Readings where the pages leave a step open:
  * scale=None means 1/sqrt(E) with E the query's last dimension, computed in
    double; with E = 0 the scores are empty sums equal to 0 and the logits are
    the bias alone, whatever the scale.
  * is_causal keeps key j for query i iff j <= i, with i and j counted from the
    top-left corner (also when L != S).
  * enable_gqa maps query head h to key/value head h // (Hq / Hkv): query heads
    are grouped contiguously, as in the xFormers 5-D (B, M, G, Hq, K) layout on
    the insureai360 xFormers tutorial, section 5.
  * attn_mask and is_causal may be given together: the kept set is the
    intersection of both.
  * Row special values (Full specification): any NaN logit makes the row's
    output and lse NaN; otherwise any +inf logit makes the output NaN and the
    lse +inf; otherwise a row with no finite logit has weight 0 on every key,
    output 0 (0 * v) and lse -inf.
  * Packed variable-length input with a block-diagonal mask (insureai360
    tutorial, section 4): keys of another segment are removed; is_causal then
    applies within a segment with local indices.  Computing each segment on its
    own is the same thing, since removed keys get weight exactly 0; a test pins
    the two forms against each other.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "resolve_scale", "bias_from_mask", "causal_bias", "logits", "weights",
    "sdpa", "sdpa_backward", "block_diagonal_bias", "sdpa_varlen", "sdpa_paged", "sdpa_paged_varlen",
    "entropy",
]


def _f64(x):
    """Exact float64 copy of an array-like (torch tensors included, any float dtype)."""
    if hasattr(x, "detach"):  # a torch tensor: upcast exactly on the host
        x = x.detach().cpu()
        if x.dtype.is_floating_point:
            x = x.double()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def resolve_scale(E, scale):
    """The factor on the scores: ``scale`` if given, else 1/sqrt(E) (Arguments table)."""
    if scale is not None:
        return float(scale)
    if E == 0:
        return math.inf  # never used: with E = 0 the scores are 0 and the logits are the mask
    return 1.0 / math.sqrt(E)


def bias_from_mask(attn_mask):
    """A bool mask keeps keys where True (bias 0, else -inf); a float mask is the bias itself."""
    if attn_mask is None:
        return None
    if hasattr(attn_mask, "detach"):
        attn_mask = attn_mask.detach().cpu()
        if attn_mask.dtype.is_floating_point:
            attn_mask = attn_mask.double()
        attn_mask = attn_mask.numpy()
    m = np.asarray(attn_mask)
    if m.dtype == np.bool_:
        return np.where(m, 0.0, -np.inf)
    return m.astype(np.float64)


def causal_bias(L, S):
    """(L, S) bias: 0 where key j <= query i, -inf above the diagonal (top-left aligned)."""
    i = np.arange(L)[:, None]
    j = np.arange(S)[None, :]
    return np.where(j <= i, 0.0, -np.inf)


def _expand_kv(query, key, value, enable_gqa):
    """Repeat key/value heads for grouped-query attention (contiguous groups)."""
    if key.ndim < 3 or query.ndim < 3:
        return key, value
    hq, hk = query.shape[-3], key.shape[-3]
    if enable_gqa and hq != hk:
        if hk == 0 or hq % hk != 0:
            raise ValueError(f"query heads ({hq}) must be a multiple of key/value heads ({hk})")
        rep = hq // hk
        key = np.repeat(key, rep, axis=-3)
        value = np.repeat(value, rep, axis=-3)
    return key, value


def _logit_parts(query, key, attn_mask=None, is_causal=False, scale=None, enable_gqa=False):
    """The (..., L, S) float64 scaled scores scale * q.k and the bias (every mask folded),
    kept apart so that a bias common to a row's keys cancels exactly in the softmax."""
    q = _f64(query)
    k = _f64(key)
    k, _ = _expand_kv(q, k, k, enable_gqa)
    E = q.shape[-1]
    L, S = q.shape[-2], k.shape[-2]
    bias = np.zeros((L, S))
    mb = bias_from_mask(attn_mask)
    if mb is not None:
        bias = bias + mb
    if is_causal:
        bias = bias + causal_bias(L, S)
    with np.errstate(invalid="ignore", over="ignore"):
        if E == 0:
            cs = np.zeros(np.broadcast_shapes(q.shape[:-2], k.shape[:-2]) + (L, S))
        else:
            cs = resolve_scale(E, scale) * np.matmul(q, np.swapaxes(k, -1, -2))
    shape = np.broadcast_shapes(cs.shape, bias.shape)
    return np.broadcast_to(cs, shape), np.broadcast_to(bias, shape)


def logits(query, key, attn_mask=None, is_causal=False, scale=None, enable_gqa=False):
    """The (..., L, S) float64 logits scale * q.k + bias, with every mask folded into the bias."""
    cs, bias = _logit_parts(query, key, attn_mask, is_causal, scale, enable_gqa)
    with np.errstate(invalid="ignore", over="ignore"):
        return cs + bias


def _row_classes(ell):
    """Boolean row classes of the Full specification: NaN rows, +inf rows, empty rows, normal rows."""
    nan_row = np.isnan(ell).any(axis=-1)
    inf_row = np.isposinf(ell).any(axis=-1) & ~nan_row
    has_finite = np.isfinite(ell).any(axis=-1)
    empty_row = ~nan_row & ~inf_row & ~has_finite
    normal = ~nan_row & ~inf_row & has_finite
    return nan_row, inf_row, empty_row, normal


def _softmax_parts(cs, bias):
    """Row max m, unnormalised weights w = exp(l - m), row sum, and row classes.

    The shifted logit l_j - m is formed as (b_j - b_k) + (cs_j - cs_k) with k the
    key of the largest logit: a bias shared by the row's keys (a padding mask's
    lowest float added to every key) then cancels exactly, as the exactref.ai
    "Padding masks" section says it does in exact arithmetic, instead of
    swallowing the scores when the two are added in float64."""
    with np.errstate(invalid="ignore", over="ignore"):
        ell = cs + bias
    nan_row, inf_row, empty_row, normal = _row_classes(ell)
    with np.errstate(invalid="ignore", over="ignore"):
        if ell.shape[-1] == 0:   # no keys: every row is empty
            m = np.zeros(ell.shape[:-1])
            w = np.zeros(ell.shape)
        else:
            fin = np.where(np.isfinite(ell), ell, -np.inf)
            kmax = np.argmax(fin, axis=-1)[..., None]
            m = np.where(normal, np.take_along_axis(ell, kmax, axis=-1)[..., 0], 0.0)
            bk = np.take_along_axis(bias, kmax, axis=-1)
            ck = np.take_along_axis(cs, kmax, axis=-1)
            d = (bias - bk) + (cs - ck)
            d = np.where(np.isfinite(ell), d, ell - m[..., None])
            w = np.exp(d)
    w = np.where(normal[..., None], w, 0.0)
    rowsum = w.sum(axis=-1)
    return m, w, rowsum, (nan_row, inf_row, empty_row, normal)


def weights(query, key, attn_mask=None, is_causal=False, scale=None, enable_gqa=False):
    """The materialised (..., L, S) attention weights P (NaN rows for NaN/+inf logits, 0 rows when empty)."""
    _, w, rowsum, (nan_row, inf_row, _, normal) = _softmax_parts(
        *_logit_parts(query, key, attn_mask, is_causal, scale, enable_gqa))
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(normal[..., None], w / np.where(normal, rowsum, 1.0)[..., None], 0.0)
    p = np.where((nan_row | inf_row)[..., None], np.nan, p)
    return p


def sdpa(query, key, value, attn_mask=None, dropout_p=0.0, is_causal=False, scale=None,
         enable_gqa=False):
    """Exact attention: returns (out (..., L, Ev), lse (..., L)) in float64.

    exactref.ai ``scaled_dot_product_attention``, Full specification: out is
    softmax(Q K^T * scale + mask) V and lse is log(sum_j exp(logit_j)).
    """
    if dropout_p != 0:
        raise ValueError("dropout_p must be 0: a random dropout has no exact reference")
    q, k, v = _f64(query), _f64(key), _f64(value)
    if k.shape[-1] != q.shape[-1]:
        raise ValueError("query and key must share the last dimension E")
    if k.shape[-2] != v.shape[-2]:
        raise ValueError("key and value must share the sequence length S")
    if not enable_gqa and q.ndim >= 3 and k.ndim >= 3 and q.shape[-3] != k.shape[-3] \
            and k.shape[-3] != 1 and q.shape[-3] != 1:
        raise ValueError("query and key heads differ: pass enable_gqa=True")
    _, vv = _expand_kv(q, k, v, enable_gqa)
    m, w, rowsum, (nan_row, inf_row, empty_row, normal) = _softmax_parts(
        *_logit_parts(q, k, attn_mask, is_causal, scale, enable_gqa))
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(normal[..., None], w / np.where(normal, rowsum, 1.0)[..., None], 0.0)
        p = np.where((nan_row | inf_row)[..., None], np.nan, p)
        out = np.matmul(p, vv)
        lse = np.where(normal, m + np.log(np.where(normal, rowsum, 1.0)), 0.0)
    lse = np.where(empty_row, -np.inf, lse)
    lse = np.where(inf_row, np.inf, lse)
    lse = np.where(nan_row, np.nan, lse)
    return out, lse


def _fold_copies(g, shape, enable_gqa):
    """Sum a gradient over the copies that grouped-query expansion and broadcasting
    made of an input of ``shape`` (Backward: "each summed over the copies")."""
    if enable_gqa and g.ndim >= 3 and len(shape) >= 3 and g.shape[-3] != shape[-3] and shape[-3] > 0:
        rep = g.shape[-3] // shape[-3]
        g = g.reshape(g.shape[:-3] + (shape[-3], rep) + g.shape[-2:]).sum(axis=-3)
    while g.ndim > len(shape):
        g = g.sum(axis=0)
    for ax, (n, m) in enumerate(zip(g.shape, shape)):
        if m == 1 and n != 1:
            g = g.sum(axis=ax, keepdims=True)
    return g


def sdpa_backward(query, key, value, grad, attn_mask=None, dropout_p=0.0, is_causal=False,
                  scale=None, enable_gqa=False):
    """Gradients (grad_query, grad_key, grad_value) of exact attention, float64.

    exactref.ai ``scaled_dot_product_attention.backward``: with P the attention
    weights (materialised as in the forward), dP = grad V^T, D_i = sum_j P_ij dP_ij,
    dS = P * (dP - D); grad_value = P^T grad, grad_query = scale * dS K,
    grad_key = scale * dS^T Q, each summed over the copies that grouped-query
    expansion made of its input.  Non-finite values propagate as IEEE arithmetic
    does: a NaN row of the forward makes every gradient it touches NaN, and a row
    with no kept key has P = 0 and contributes 0.  A float mask gets no gradient.
    """
    if dropout_p != 0:
        raise ValueError("dropout_p must be 0: a random dropout has no exact reference")
    q, k, v, g = _f64(query), _f64(key), _f64(value), _f64(grad)
    if k.shape[-1] != q.shape[-1]:
        raise ValueError("query and key must share the last dimension E")
    if k.shape[-2] != v.shape[-2]:
        raise ValueError("key and value must share the sequence length S")
    if not enable_gqa and q.ndim >= 3 and k.ndim >= 3 and q.shape[-3] != k.shape[-3] \
            and k.shape[-3] != 1 and q.shape[-3] != 1:
        raise ValueError("query and key heads differ: pass enable_gqa=True")
    p = weights(q, k, attn_mask, is_causal, scale, enable_gqa)
    kk, vv = _expand_kv(q, k, v, enable_gqa)
    E = q.shape[-1]
    sc = resolve_scale(E, scale) if E > 0 else 0.0  # with E = 0, grad_query and grad_key are empty
    with np.errstate(invalid="ignore", over="ignore"):
        dp = np.matmul(g, np.swapaxes(vv, -1, -2))
        d = (p * dp).sum(axis=-1, keepdims=True)
        ds = p * (dp - d)
        gv = np.matmul(np.swapaxes(p, -1, -2), g)
        gq = sc * np.matmul(ds, kk)
        gk = sc * np.matmul(np.swapaxes(ds, -1, -2), q)
    gq = _fold_copies(gq, q.shape, False)
    gk = _fold_copies(gk, k.shape, enable_gqa)
    gv = _fold_copies(gv, v.shape, enable_gqa)
    return gq, gk, gv


def block_diagonal_bias(lengths_q, lengths_k=None, causal=False):
    """(total_q, total_k) bias of a block-diagonal mask over packed segments.

    insureai360 tutorial, section 4 (``BlockDiagonalMask`` / ``BlockDiagonalCausalMask``):
    a query sees only keys of its own segment; the causal form also removes keys
    whose local index exceeds the query's local index.
    """
    if lengths_k is None:
        lengths_k = lengths_q
    tq, tk = int(sum(lengths_q)), int(sum(lengths_k))
    bias = np.full((tq, tk), -np.inf)
    oq = ok = 0
    for lq, lk in zip(lengths_q, lengths_k):
        block = causal_bias(lq, lk) if causal else np.zeros((lq, lk))
        bias[oq:oq + lq, ok:ok + lk] = block
        oq += lq
        ok += lk
    return bias


def sdpa_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k=None, is_causal=False, scale=None,
                enable_gqa=False, dropout_p=0.0):
    """Packed variable-length attention with a block-diagonal mask.

    q (total_q, Hq, E), k (total_k, Hkv, E), v (total_k, Hkv, Ev) packed along
    the token axis; cu_seqlens are the n+1 cumulative segment offsets.  Returns
    out (total_q, Hq, Ev) and lse (Hq, total_q), float64.  Each segment is
    computed on its own, which equals the block-diagonal mask over the packed
    tensors exactly (see the module docstring).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cq = [int(x) for x in np.asarray(cu_seqlens_q).ravel()]
    ck = cq if cu_seqlens_k is None else [int(x) for x in np.asarray(cu_seqlens_k).ravel()]
    Hq, Ev = q.shape[1], v.shape[2]
    out = np.zeros((q.shape[0], Hq, Ev))
    lse = np.full((Hq, q.shape[0]), -np.inf)
    for s in range(len(cq) - 1):
        a, b = cq[s], cq[s + 1]
        c, d = ck[s], ck[s + 1]
        if b == a:
            continue
        qs = np.swapaxes(q[a:b], 0, 1)  # (Hq, lq, E)
        ks = np.swapaxes(k[c:d], 0, 1)
        vs = np.swapaxes(v[c:d], 0, 1)
        o, l_ = sdpa(qs, ks, vs, dropout_p=dropout_p, is_causal=is_causal, scale=scale,
                     enable_gqa=enable_gqa)
        out[a:b] = np.swapaxes(o, 0, 1)
        lse[:, a:b] = l_
    return out, lse


def sdpa_paged(q, k_cache, v_cache, block_table, seq_lens, is_causal=False, scale=None,
               enable_gqa=False):
    """Attention of new query rows against a paged key/value cache, float64.

    q (B, Hq, L, E); k_cache (n_pages, Hkv, page_size, E) and v_cache
    (n_pages, Hkv, page_size, Ev); block_table (B, max_blocks) ints: logical
    block j of sequence b lives in page block_table[b][j]; seq_lens (B,): the
    cached length n_b of each sequence (the L new rows' own keys included).
    Sequence b attends to its first n_b cached keys, gathered page by page
    (the paged KV cache the pages mention for vLLM/FlashInfer-style serving).
    is_causal aligns bottom-right: new row i (0-based of L) is the sequence's
    position n_b - L + i and keeps key j iff j <= n_b - L + i.  Returns out
    (B, Hq, L, Ev) and lse (B, Hq, L).  A table entry outside [0, n_pages) for
    a needed block raises ValueError (nothing is read from outside the cache).
    """
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    bt = np.asarray(block_table)
    lens = [int(x) for x in np.asarray(seq_lens).ravel()]
    B, Hq, L, E = q.shape
    n_pages, Hkv, ps, _ = kc.shape
    Ev = vc.shape[-1]
    out = np.zeros((B, Hq, L, Ev))
    lse = np.full((B, Hq, L), -np.inf)
    for b in range(B):
        n = lens[b]
        nblk = (n + ps - 1) // ps
        if nblk > bt.shape[1]:
            raise ValueError(f"sequence {b}: {n} keys need {nblk} blocks, the table has {bt.shape[1]}")
        pages = [int(x) for x in bt[b, :nblk]]
        if any(pg < 0 or pg >= n_pages for pg in pages):
            raise ValueError(f"sequence {b}: block table entry outside [0, {n_pages})")
        kb = np.concatenate([kc[pg] for pg in pages], axis=1)[:, :n] if nblk else np.zeros((Hkv, 0, E))
        vb = np.concatenate([vc[pg] for pg in pages], axis=1)[:, :n] if nblk else np.zeros((Hkv, 0, Ev))
        bias = None
        if is_causal:
            i = np.arange(L)[:, None]
            j = np.arange(n)[None, :]
            bias = np.where(j <= n - L + i, 0.0, -np.inf)
        o, l_ = sdpa(q[b], kb, vb, attn_mask=bias, scale=scale, enable_gqa=enable_gqa)
        out[b], lse[b] = o, l_
    return out, lse


def sdpa_paged_varlen(q, cu_seqlens_q, k_cache, v_cache, block_table, seq_lens, is_causal=False, scale=None,
                      enable_gqa=False):
    """Packed new rows of several sequences against a paged cache, float64.

    q (total_q, Hq, E) holds sequence b's new rows at tokens cu_seqlens_q[b] ..
    cu_seqlens_q[b + 1] - 1 (each sequence its own number L_b of new rows);
    the cache, block table and seq_lens are as for sdpa_paged, and each
    sequence is exactly sdpa_paged of its own rows (bottom-right causal over
    its n_b cached keys).  Returns out (total_q, Hq, Ev) and lse (Hq, total_q).
    """
    qq = _f64(q)
    cu = [int(x) for x in np.asarray(cu_seqlens_q).ravel()]
    bt = np.asarray(block_table)
    lens = np.asarray(seq_lens).ravel()
    total, Hq, _ = qq.shape
    Ev = v_cache.shape[-1]
    out = np.zeros((total, Hq, Ev))
    lse = np.full((Hq, total), -np.inf)
    for b in range(len(cu) - 1):
        a, e = cu[b], cu[b + 1]
        if e == a:
            continue
        qb = np.transpose(qq[a:e], (1, 0, 2))[None]            # (1, Hq, L_b, E)
        o, l_ = sdpa_paged(qb, k_cache, v_cache, bt[b:b + 1], lens[b:b + 1], is_causal=is_causal,
                           scale=scale, enable_gqa=enable_gqa)
        out[a:e] = np.transpose(o[0], (1, 0, 2))
        lse[:, a:e] = l_[0]
    return out, lse


def entropy(p):
    """Attention entropy -sum_j p_j log p_j per row, in nats (0 log 0 = 0)."""
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0)), 0.0)
    return -t.sum(axis=-1)
