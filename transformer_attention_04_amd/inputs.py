"""Seeded synthetic inputs shared by the HIP path's tests, the bench and the oracle's tests.

This module draws random numbers and lays out inputs. It holds none of the
attention arithmetic: no scores, no softmax, no weighting of values. The same
seed and shape always give the same bytes, so the oracle (host float64) and the
HIP kernels (device) receive exactly the same values.

Recipe (the pages fix none of it, so this is the plainest choice):
  * Q, K, V are drawn i.i.d. N(0, 1) in float32 from one CPU
    ``torch.Generator`` seeded with ``seed``, in the order Q, K, V, and then
    rounded to nearest-even into the working dtype (bf16 / fp16 / fp32).
  * Packed variable-length segment lengths are ``random.Random(seed).randint``
    draws, inclusive on both ends (Python's own seeded generator, the style the
    exactref.ai "Checking PyTorch" example uses).
  * The ALiBi-style bias of the GPT-NeoX-shaped workload is computed in float64
    and rounded once to float32: bias[h, i, j] = -(i - j) * 2**(-8 (h + 1) / H)
    for j <= i and -inf for j > i (0-based h, i, j).
"""
from __future__ import annotations

import random

import numpy as np
import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


def randn_qkv(q_shape, k_shape, v_shape, dtype="bf16", seed=0):
    """Q, K, V as CPU tensors of ``dtype``: N(0,1) float32 draws, Q then K then V, RNE cast."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    out = []
    for shape in (q_shape, k_shape, v_shape):
        t = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
        out.append(t.to(DTYPES[dtype]))
    return tuple(out)


def segment_lengths(n=32, lo=8, hi=2048, seed=1):
    """``n`` segment lengths drawn uniformly from [lo, hi] (both inclusive)."""
    r = random.Random(seed)
    return [r.randint(lo, hi) for _ in range(n)]


def cu_seqlens(lengths):
    """Cumulative offsets [0, l0, l0+l1, ...] as int32 (length n+1)."""
    c = np.zeros(len(lengths) + 1, dtype=np.int64)
    c[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return c.astype(np.int32)


def alibi_causal_bias(H, L, S):
    """(H, L, S) float32 ALiBi-style additive bias with -inf above the diagonal."""
    i = np.arange(L, dtype=np.float64)[:, None]
    j = np.arange(S, dtype=np.float64)[None, :]
    out = np.empty((H, L, S), dtype=np.float32)
    for h in range(H):
        slope = 2.0 ** (-8.0 * (h + 1) / H)
        b = -(i - j) * slope
        b = np.where(j <= i, b, -np.inf)
        out[h] = b.astype(np.float32)
    return torch.from_numpy(out)


# The five workloads, with their shapes in (B, H, L, E) order.  ``name`` is what
# the bench and the tests print.
WORKLOADS = {
    "fp32_single_head": dict(dtype="fp32", B=1, Hq=1, Hkv=1, L=128, S=128, E=64, causal=False, seed=0),
    "bf16_causal_e128": dict(dtype="bf16", B=4, Hq=16, Hkv=16, L=2048, S=2048, E=128, causal=True, seed=0),
    "bf16_neox_e96": dict(dtype="bf16", B=2, Hq=64, Hkv=64, L=2048, S=2048, E=96, causal=True, seed=0),
    "fp16_varlen_e64": dict(dtype="fp16", n_seqs=32, Hq=8, Hkv=8, E=64, causal=True, seed=0, len_seed=1),
    "bf16_gqa_decode": dict(dtype="bf16", B=64, Hq=32, Hkv=8, L=1, S=32768, E=128, causal=False, seed=0),
}


def workload_inputs(name, device="cpu"):
    """Q, K, V for a named batched workload, laid out (B, H, rows, E), on ``device``."""
    w = WORKLOADS[name]
    q, k, v = randn_qkv((w["B"], w["Hq"], w["L"], w["E"]),
                        (w["B"], w["Hkv"], w["S"], w["E"]),
                        (w["B"], w["Hkv"], w["S"], w["E"]), w["dtype"], w["seed"])
    return q.to(device), k.to(device), v.to(device)


def varlen_inputs(lengths, H, Hkv, E, dtype="fp16", seed=0, device="cpu"):
    """Packed Q, K, V of shape (1, total, H, E) (the BMHK layout) and int32 cu_seqlens."""
    total = int(sum(lengths))
    q, k, v = randn_qkv((1, total, H, E), (1, total, Hkv, E), (1, total, Hkv, E), dtype, seed)
    cu = torch.from_numpy(cu_seqlens(lengths))
    return q.to(device), k.to(device), v.to(device), cu.to(device)

