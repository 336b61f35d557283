"""sdpa_fwd_noalloc (the allocation-free entry point) against sdpa_fwd, through the C interface.

Both run the same kernels; the allocation-free one keeps the split-KV
partials in the library's own device array instead of a workspace.  Two
decode calls in a row (the second smaller, so stale partials of the first
would show), a single-pass call that needs no scratch, and a call whose
scratch would not fit, which must fail before anything runs.  Outputs must be
bit-identical to sdpa_fwd's and within the forward bars of the oracle.
"""
import numpy as np
import pytest
import torch

from oracle import sdpa_oracle as O
from transformer_attention_04_amd import inputs
from transformer_attention_04_amd import sdpa as S

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(q, k, v, **kw):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ref = S.sdpa_fwd(qd, kd, vd, **kw)
    out = torch.full_like(ref[0], float("nan"))
    lse = torch.full(ref[1].shape + (1,), float("nan"), dtype=torch.float32, device=DEV)
    got = S.sdpa_fwd_noalloc(qd, kd, vd, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    return ref, got


def _oracle_close(got, q, k, v, **kw):
    ro, rl = O.sdpa(q, k, v, enable_gqa=kw.get("enable_gqa", False), is_causal=kw.get("is_causal", False))
    assert np.abs(got[0].cpu().double().numpy() - ro).max() <= 2e-2
    assert np.abs(got[1].cpu().double().numpy() - rl).max() <= 1e-3


def test_noalloc_equals_workspace_entry_point():
    # decode with 5 splits: partials in the scratch array
    q, k, v = inputs.randn_qkv((4, 16, 1, 128), (4, 4, 3000, 128), (4, 4, 3000, 128), "bf16", seed=1)
    ref, got = _both(q, k, v, enable_gqa=True, num_splits=5)
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    _oracle_close(got, q, k, v, enable_gqa=True)
    # a second, smaller decode call right after (fewer rows, splits and keys)
    q, k, v = inputs.randn_qkv((2, 8, 1, 64), (2, 2, 700, 64), (2, 2, 700, 64), "fp16", seed=2)
    ref, got = _both(q, k, v, enable_gqa=True, num_splits=3)
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    _oracle_close(got, q, k, v, enable_gqa=True)
    # automatic split count at the decode workload's per-sequence shape (B reduced)
    q, k, v = inputs.randn_qkv((4, 32, 1, 128), (4, 8, 32768, 128), (4, 8, 32768, 128), "bf16", seed=3)
    ref, got = _both(q, k, v, enable_gqa=True)
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    # a single-pass call: no scratch at all
    q, k, v = inputs.randn_qkv((1, 2, 300, 96), (1, 2, 300, 96), (1, 2, 300, 96), "bf16", seed=4)
    ref, got = _both(q, k, v, is_causal=True)
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])


def test_noalloc_rejects_scratch_beyond_its_size():
    # 64 sequences x 32 query heads x 64 splits of 128 keys: 64*32*64*(128+1)*4 bytes > 8 MiB.
    # The key/value tensors are broadcast views (batch stride 0): nothing is launched.
    q = torch.zeros((64, 32, 1, 128), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((1, 8, 8192, 128), dtype=torch.bfloat16, device=DEV).expand(64, 8, 8192, 128)
    with pytest.raises(RuntimeError, match="scratch"):
        S.sdpa_fwd_noalloc(q, kv, kv, enable_gqa=True, num_splits=64)
    torch.cuda.synchronize()
