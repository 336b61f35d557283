"""Python binding of libsdpa (ctypes): argument marshalling only.

The functions here have the names of the C entry points in include/sdpa.h.
They turn torch tensors into device pointers, sizes and strides, allocate the
outputs (and the split-KV workspace) with torch, and enqueue the HIP kernels
on torch's current stream.  Every step of the attention itself runs in the
HIP kernels; there is no CPU or PyTorch fallback: without the built library,
or with tensors that are not on a ROCm device, these functions raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdpa.so")

SDPA_OK, SDPA_ERR_INVALID_ARGUMENT, SDPA_ERR_UNSUPPORTED, SDPA_ERR_DEVICE = 0, 1, 2, 3
SDPA_F32, SDPA_F16, SDPA_BF16, SDPA_BOOL = 0, 1, 2, 3
_DTYPE = {torch.float32: SDPA_F32, torch.float16: SDPA_F16, torch.bfloat16: SDPA_BF16}

EXPORTED = ("sdpa_fwd", "sdpa_fwd_workspace_size", "sdpa_fwd_noalloc", "sdpa_fwd_varlen", "sdpa_fwd_paged",
            "sdpa_fwd_paged_workspace_size", "sdpa_fwd_paged_varlen", "sdpa_bwd", "sdpa_bwd_workspace_size", "sdpa_bwd_varlen",
            "sdpa_bwd_varlen_workspace_size", "sdpa_last_error",
            "sdpa_abi_version")


class SdpaTensor4(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p),
                ("size", ctypes.c_int64 * 4),
                ("stride", ctypes.c_int64 * 4)]


class SdpaError(RuntimeError):
    """A non-zero status from libsdpa, with its message."""

    def __init__(self, status, message):
        super().__init__(f"libsdpa status {status}: {message}")
        self.status = status


_lib = None


def library_path():
    return _LIB_PATH


def load_library():
    """Load libsdpa.so from the package directory (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m transformer_attention_04_amd.build_lib`")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(SdpaTensor4)
    vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.sdpa_fwd.argtypes = [ctypes.c_int, P, P, P, P, ctypes.c_int, dbl, ctypes.c_int,
                             ctypes.POINTER(dbl), ctypes.c_int, P, P, vp, ctypes.c_size_t,
                             ctypes.c_int, vp]
    lib.sdpa_fwd.restype = ctypes.c_int
    lib.sdpa_fwd_noalloc.argtypes = [ctypes.c_int, P, P, P, P, ctypes.c_int, dbl, ctypes.c_int,
                                     ctypes.POINTER(dbl), ctypes.c_int, P, P, ctypes.c_int, vp]
    lib.sdpa_fwd_noalloc.restype = ctypes.c_int
    lib.sdpa_fwd_workspace_size.argtypes = [ctypes.c_int, P, P, P, P, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.sdpa_fwd_workspace_size.restype = ctypes.c_int
    lib.sdpa_fwd_varlen.argtypes = [ctypes.c_int, vp, i64, i64, vp, i64, i64, vp, i64, i64,
                                    vp, vp, i32, i32, i32, i32, i32, i32, i32, i64, i64,
                                    dbl, ctypes.c_int, ctypes.POINTER(dbl), ctypes.c_int,
                                    vp, i64, i64, vp, i64, vp]
    lib.sdpa_fwd_varlen.restype = ctypes.c_int
    lib.sdpa_fwd_paged.argtypes = [ctypes.c_int, P, P, P, vp, i64, i32, vp, i32, ctypes.c_int,
                                   ctypes.POINTER(dbl), ctypes.c_int, P, P, vp, ctypes.c_size_t,
                                   ctypes.c_int, vp]
    lib.sdpa_fwd_paged.restype = ctypes.c_int
    lib.sdpa_fwd_paged_workspace_size.argtypes = [ctypes.c_int, P, P, P, i32, ctypes.c_int, ctypes.c_int,
                                                  ctypes.POINTER(ctypes.c_size_t)]
    lib.sdpa_fwd_paged_workspace_size.restype = ctypes.c_int
    lib.sdpa_fwd_paged_varlen.argtypes = [ctypes.c_int, vp, i64, i64, vp, i32, i32, i64, i32, P, P, vp, i64, i32,
                                          vp, i32, ctypes.c_int, ctypes.POINTER(dbl), ctypes.c_int, vp, i64, i64,
                                          vp, i64, vp]
    lib.sdpa_fwd_paged_varlen.restype = ctypes.c_int
    lib.sdpa_bwd.argtypes = [ctypes.c_int, P, P, P, P, ctypes.c_int, P, P, P, ctypes.c_int,
                             ctypes.POINTER(dbl), ctypes.c_int, P, P, P, vp, ctypes.c_size_t, vp]
    lib.sdpa_bwd.restype = ctypes.c_int
    lib.sdpa_bwd_workspace_size.argtypes = [ctypes.c_int, P, P, P, ctypes.c_int,
                                            ctypes.POINTER(ctypes.c_size_t)]
    lib.sdpa_bwd_workspace_size.restype = ctypes.c_int
    lib.sdpa_bwd_varlen.argtypes = ([ctypes.c_int] + [vp, i64, i64] * 4 + [vp, i64] + [vp, i64, i64]
                                    + [vp, vp, i32, i32, i32, i32, i32, i32, i32, i64, i64, ctypes.c_int,
                                       ctypes.POINTER(dbl), ctypes.c_int] + [vp, i64, i64] * 3
                                    + [vp, ctypes.c_size_t, vp])
    lib.sdpa_bwd_varlen.restype = ctypes.c_int
    lib.sdpa_bwd_varlen_workspace_size.argtypes = [i32, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.sdpa_bwd_varlen_workspace_size.restype = ctypes.c_int
    lib.sdpa_last_error.argtypes = []
    lib.sdpa_last_error.restype = ctypes.c_char_p
    lib.sdpa_abi_version.argtypes = []
    lib.sdpa_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def sdpa_last_error():
    return load_library().sdpa_last_error().decode()


def sdpa_abi_version():
    return load_library().sdpa_abi_version()


def _check(status):
    if status != SDPA_OK:
        raise SdpaError(status, sdpa_last_error())


def _desc(t):
    d = SdpaTensor4()
    d.data = t.data_ptr() if t is not None and t.numel() > 0 else None
    for i in range(4):
        d.size[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _as4d(x):
    """(..., H, L, E) -> (B, H, L, E) with B the product of the leading dims (a view when possible)."""
    if x.dim() < 2:
        raise ValueError("attention inputs need at least 2 dimensions (..., L, E)")
    if x.dim() == 2:
        return x.unsqueeze(0).unsqueeze(0)
    if x.dim() == 3:
        return x.unsqueeze(0)
    if x.dim() == 4:
        return x
    return x.reshape(-1, *x.shape[-3:])


def _scale_arg(scale):
    return None if scale is None else ctypes.byref(ctypes.c_double(float(scale)))


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require_gpu(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("libsdpa runs on the GPU: every tensor must be on a ROCm device")


def _mask_4d(attn_mask, q4, S):
    if attn_mask is None:
        return None, SDPA_F32
    if attn_mask.dtype == torch.bool:
        m, mdt = attn_mask, SDPA_BOOL
    else:
        m, mdt = (attn_mask if attn_mask.dtype == torch.float32 else attn_mask.float()), SDPA_F32
    while m.dim() < 4:
        m = m.unsqueeze(0)
    if m.dim() > 4:
        m = m.reshape(-1, *m.shape[-3:])
    B, H, L = q4.shape[:3]
    m = torch.broadcast_to(m, (B if m.shape[0] != 1 else 1, H if m.shape[1] != 1 else 1,
                               L if m.shape[2] != 1 else 1, S))
    if S > 1 and m.stride(3) != 1:
        m = m.contiguous()
    return m, mdt


def sdpa_fwd_workspace_size(query, key, value, attn_mask=None, is_causal=False, enable_gqa=False,
                            num_splits=0):
    """Workspace bytes sdpa_fwd needs for these arguments (host only)."""
    lib = load_library()
    q4, k4, v4 = _as4d(query), _as4d(key), _as4d(value)
    k4, v4 = _expand_batch(q4, k4), _expand_batch(q4, v4)
    m4, _ = _mask_4d(attn_mask, q4, k4.shape[2])
    n = ctypes.c_size_t(0)
    dq, dk, dv = _desc(q4), _desc(k4), _desc(v4)
    dm = _desc(m4) if m4 is not None else None
    _check(lib.sdpa_fwd_workspace_size(_DTYPE[query.dtype], dq, dk, dv,
                                       ctypes.byref(dm) if dm is not None else None,
                                       int(bool(is_causal)), int(bool(enable_gqa)), int(num_splits),
                                       ctypes.byref(n)))
    return n.value


def _expand_batch(q4, t4):
    if t4.shape[0] == 1 and q4.shape[0] != 1:
        return t4.expand(q4.shape[0], *t4.shape[1:])
    return t4


def sdpa_fwd(query, key, value, attn_mask=None, dropout_p=0.0, is_causal=False, scale=None,
             enable_gqa=False, num_splits=0, out=None, lse=None, workspace=None):
    """Exact attention forward on the GPU.  Returns (out (..., Hq, L, Ev), lse (..., Hq, L) float32).

    Arguments follow the exactref.ai "scaled_dot_product_attention" Arguments
    table; ``num_splits`` selects the kernel (0 automatic, -1 single pass,
    k >= 1 split-KV decode with k splits).
    """
    lib = load_library()
    _require_gpu(query, key, value, attn_mask, out, lse)
    if query.dtype not in _DTYPE or key.dtype != query.dtype or value.dtype != query.dtype:
        raise ValueError("query, key and value must share one of float32, float16, bfloat16")
    q4, k4, v4 = _as4d(query), _as4d(key), _as4d(value)
    k4, v4 = _expand_batch(q4, k4), _expand_batch(q4, v4)
    B, Hq, L, _ = q4.shape
    S, Ev = v4.shape[2], v4.shape[3]
    m4, mdt = _mask_4d(attn_mask, q4, S)
    dev = query.device
    if out is None:
        out = torch.empty((B, Hq, L, Ev), dtype=query.dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq, L, 1), dtype=torch.float32, device=dev)
    if tuple(out.shape) != (B, Hq, L, Ev) or tuple(lse.shape) != (B, Hq, L, 1):
        raise ValueError("out must be (B, Hq, L, Ev) and lse (B, Hq, L, 1)")
    o4, l4 = out, lse
    dq, dk, dv, do, dl = _desc(q4), _desc(k4), _desc(v4), _desc(o4), _desc(l4)
    dm = _desc(m4) if m4 is not None else None
    pm = ctypes.byref(dm) if dm is not None else None
    with torch.cuda.device(dev):
        nbytes = ctypes.c_size_t(0)
        _check(lib.sdpa_fwd_workspace_size(_DTYPE[query.dtype], dq, dk, dv, pm, int(bool(is_causal)),
                                           int(bool(enable_gqa)), int(num_splits), ctypes.byref(nbytes)))
        if nbytes.value and (workspace is None or workspace.numel() < nbytes.value):
            workspace = torch.empty(nbytes.value, dtype=torch.uint8, device=dev)
        ws_ptr = workspace.data_ptr() if nbytes.value else None
        _check(lib.sdpa_fwd(_DTYPE[query.dtype], dq, dk, dv, pm, mdt, float(dropout_p),
                            int(bool(is_causal)), _scale_arg(scale), int(bool(enable_gqa)), do, dl,
                            ws_ptr, nbytes.value, int(num_splits), _stream(dev)))
    return o4.reshape(*query.shape[:-1], Ev), l4.reshape(*query.shape[:-1])


def sdpa_fwd_noalloc(query, key, value, attn_mask=None, dropout_p=0.0, is_causal=False, scale=None,
                     enable_gqa=False, num_splits=0, out=None, lse=None):
    """sdpa_fwd through the allocation-free C entry point: the split-KV scratch is
    the library's own device array (no workspace).  ``out`` and ``lse`` are
    allocated here only when not given; the C call allocates nothing."""
    lib = load_library()
    _require_gpu(query, key, value, attn_mask, out, lse)
    if query.dtype not in _DTYPE or key.dtype != query.dtype or value.dtype != query.dtype:
        raise ValueError("query, key and value must share one of float32, float16, bfloat16")
    q4, k4, v4 = _as4d(query), _as4d(key), _as4d(value)
    k4, v4 = _expand_batch(q4, k4), _expand_batch(q4, v4)
    B, Hq, L, _ = q4.shape
    S, Ev = v4.shape[2], v4.shape[3]
    m4, mdt = _mask_4d(attn_mask, q4, S)
    dev = query.device
    if out is None:
        out = torch.empty((B, Hq, L, Ev), dtype=query.dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq, L, 1), dtype=torch.float32, device=dev)
    if tuple(out.shape) != (B, Hq, L, Ev) or tuple(lse.shape) != (B, Hq, L, 1):
        raise ValueError("out must be (B, Hq, L, Ev) and lse (B, Hq, L, 1)")
    dm = _desc(m4) if m4 is not None else None
    with torch.cuda.device(dev):
        _check(lib.sdpa_fwd_noalloc(_DTYPE[query.dtype], _desc(q4), _desc(k4), _desc(v4),
                                    ctypes.byref(dm) if dm is not None else None, mdt, float(dropout_p),
                                    int(bool(is_causal)), _scale_arg(scale), int(bool(enable_gqa)), _desc(out),
                                    _desc(lse), int(num_splits), _stream(dev)))
    return out.reshape(*query.shape[:-1], Ev), lse.reshape(*query.shape[:-1])


def sdpa_fwd_paged(query, k_cache, v_cache, block_table, seq_lens, max_seq_len=None, is_causal=False,
                   scale=None, enable_gqa=False, num_splits=0, workspace=None):
    """Attention of new rows against a paged key/value cache on the GPU (decode
    steps through the split-KV kernel, longer chunks of new rows through the
    single-pass kernel).

    query (B, Hq, L, E); k_cache / v_cache (n_pages, Hkv, page_size, E);
    block_table (B, max_blocks) int32 and seq_lens (B,) int32 on the device;
    ``max_seq_len`` bounds seq_lens (read from the device when None, which
    synchronizes).  is_causal aligns the L new rows bottom-right.  Returns
    (out (B, Hq, L, Ev), lse (B, Hq, L) float32).
    """
    lib = load_library()
    _require_gpu(query, k_cache, v_cache, block_table, seq_lens)
    if query.dtype not in (torch.float16, torch.bfloat16) or k_cache.dtype != query.dtype \
            or v_cache.dtype != query.dtype:
        raise ValueError("the paged-cache kernel takes float16 or bfloat16 query and cache")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or block_table.dim() != 2:
        raise ValueError("block_table must be a 2-D int32 tensor and seq_lens int32")
    if block_table.stride(1) != 1:
        block_table = block_table.contiguous()
    seq_lens = seq_lens.contiguous()
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if seq_lens.numel() else 0
    B, Hq, L, E = query.shape
    Ev = v_cache.shape[3]
    dev = query.device
    out = torch.empty((B, Hq, L, Ev), dtype=query.dtype, device=dev)
    lse = torch.empty((B, Hq, L, 1), dtype=torch.float32, device=dev)
    dq, dk, dv = _desc(query), _desc(k_cache), _desc(v_cache)
    with torch.cuda.device(dev):
        n = ctypes.c_size_t(0)
        _check(lib.sdpa_fwd_paged_workspace_size(_DTYPE[query.dtype], dq, dk, dv, int(max_seq_len),
                                                 int(bool(enable_gqa)), int(num_splits), ctypes.byref(n)))
        if workspace is None or workspace.numel() < n.value:
            workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
        _check(lib.sdpa_fwd_paged(_DTYPE[query.dtype], dq, dk, dv, block_table.data_ptr(),
                                  block_table.stride(0), block_table.shape[1], seq_lens.data_ptr(),
                                  int(max_seq_len), int(bool(is_causal)), _scale_arg(scale),
                                  int(bool(enable_gqa)), _desc(out), _desc(lse), workspace.data_ptr(),
                                  n.value, int(num_splits), _stream(dev)))
    return out, lse.reshape(B, Hq, L)


def sdpa_fwd_paged_varlen(q, cu_seqlens_q, k_cache, v_cache, block_table, seq_lens, max_seqlen_q=None,
                          max_seq_len=None, is_causal=False, scale=None, enable_gqa=False):
    """Packed new rows of several sequences (each its own count) against a
    paged key/value cache on the GPU.

    q (total_q, Hq, E) or (1, total_q, Hq, E); cu_seqlens_q int32 (n_seqs + 1)
    offsets; k_cache / v_cache (n_pages, Hkv, page_size, E); block_table
    (n_seqs, max_blocks) and seq_lens (n_seqs,) int32, all on the device.
    is_causal aligns each sequence's rows bottom-right.  Returns out shaped
    like q (with Ev) and lse (Hq, total_q) (or (1, Hq, total_q)).
    """
    lib = load_library()
    _require_gpu(q, cu_seqlens_q, k_cache, v_cache, block_table, seq_lens)
    if q.dtype not in (torch.float16, torch.bfloat16) or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("the paged-cache kernels take float16 or bfloat16 query and cache")
    for t in (cu_seqlens_q, block_table, seq_lens):
        if t.dtype != torch.int32:
            raise ValueError("cu_seqlens_q, block_table and seq_lens must be int32")
    if block_table.dim() != 2:
        raise ValueError("block_table must be 2-D (n_seqs, max_blocks)")
    if block_table.stride(1) != 1:
        block_table = block_table.contiguous()
    cu_seqlens_q, seq_lens = cu_seqlens_q.contiguous(), seq_lens.contiguous()
    n_seqs = cu_seqlens_q.numel() - 1
    if max_seqlen_q is None:
        cq = cu_seqlens_q.cpu().long()
        max_seqlen_q = int((cq[1:] - cq[:-1]).max()) if n_seqs > 0 else 0
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if seq_lens.numel() else 0
    batched = q.dim() == 4
    q3 = q[0] if batched else q
    total_q, Hq, E = q3.shape
    Ev = v_cache.shape[3]
    dev = q.device
    out3 = torch.empty((total_q, Hq, Ev), dtype=q.dtype, device=dev)
    lse = torch.empty((Hq, total_q), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check(lib.sdpa_fwd_paged_varlen(
            _DTYPE[q.dtype], q3.data_ptr(), q3.stride(0), q3.stride(1), cu_seqlens_q.data_ptr(), n_seqs,
            int(max_seqlen_q), total_q, Hq, _desc(k_cache), _desc(v_cache), block_table.data_ptr(),
            block_table.stride(0), block_table.shape[1], seq_lens.data_ptr(), int(max_seq_len),
            int(bool(is_causal)), _scale_arg(scale), int(bool(enable_gqa)), out3.data_ptr(), out3.stride(0),
            out3.stride(1), lse.data_ptr(), lse.stride(0), _stream(dev)))
    if batched:
        return out3.unsqueeze(0), lse.unsqueeze(0)
    return out3, lse


def sdpa_bwd_workspace_size(query, key, value, enable_gqa=False):
    """Workspace bytes sdpa_bwd needs for these shapes (host only)."""
    lib = load_library()
    q4, k4, v4 = _as4d(query), _as4d(key), _as4d(value)
    n = ctypes.c_size_t(0)
    _check(lib.sdpa_bwd_workspace_size(_DTYPE[query.dtype], _desc(q4), _desc(k4), _desc(v4),
                                       int(bool(enable_gqa)), ctypes.byref(n)))
    return n.value


def sdpa_bwd(query, key, value, out, lse, grad, attn_mask=None, is_causal=False, scale=None,
             enable_gqa=False, workspace=None, grads=None, store_ds=True):
    """Gradients of exact attention on the GPU: returns (grad_query, grad_key, grad_value).

    ``out`` and ``lse`` are sdpa_fwd's results for the same arguments (the
    optional float or bool ``attn_mask`` included) and ``grad`` the gradient
    with respect to ``out`` (exactref.ai "scaled_dot_product_attention.backward";
    the mask gets no gradient).  The outputs have the shapes and dtype of
    query, key and value; ``grads`` may pass them in as a tuple of contiguous
    tensors (written in place).  ``store_ds=False`` hands the library only the
    workspace of the D values, so that dQ recomputes S and dP instead of reading
    the stored dS^T (the same values either way).
    """
    lib = load_library()
    _require_gpu(query, key, value, out, lse, grad, attn_mask)
    if query.dtype not in _DTYPE or any(t.dtype != query.dtype for t in (key, value, out, grad)):
        raise ValueError("query, key, value, out and grad must share one of float32, float16, bfloat16")
    q4, k4, v4 = _as4d(query), _as4d(key), _as4d(value)
    if k4.shape[0] != q4.shape[0] or v4.shape[0] != q4.shape[0]:
        raise ValueError("query, key and value must share the batch dimensions")
    B, Hq, L, E = q4.shape
    Hkv, S, Ev = k4.shape[1], v4.shape[2], v4.shape[3]
    o4, g4 = _as4d(out), _as4d(grad)
    l4 = lse.reshape(B, Hq, L, 1)
    m4, mdt = _mask_4d(attn_mask, q4, S)
    dm = _desc(m4) if m4 is not None else None
    dev = query.device
    if grads is None:
        dq4 = torch.empty((B, Hq, L, E), dtype=query.dtype, device=dev)
        dk4 = torch.empty((B, Hkv, S, E), dtype=query.dtype, device=dev)
        dv4 = torch.empty((B, Hkv, S, Ev), dtype=query.dtype, device=dev)
    else:
        want = ((B, Hq, L, E), (B, Hkv, S, E), (B, Hkv, S, Ev))
        dq4, dk4, dv4 = (_as4d(t) for t in grads)
        for t, shp in zip((dq4, dk4, dv4), want):
            if tuple(t.shape) != shp or t.dtype != query.dtype or not t.is_contiguous() or t.device != dev:
                raise ValueError(f"grads must be contiguous {query.dtype} tensors of shapes {want}")
    with torch.cuda.device(dev):
        nbytes = sdpa_bwd_workspace_size(q4, k4, v4, enable_gqa) if store_ds else B * Hq * L * 4 + 256
        if workspace is None or workspace.numel() < nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        _check(lib.sdpa_bwd(_DTYPE[query.dtype], _desc(q4), _desc(k4), _desc(v4),
                            ctypes.byref(dm) if dm is not None else None, mdt, _desc(o4), _desc(l4),
                            _desc(g4), int(bool(is_causal)), _scale_arg(scale), int(bool(enable_gqa)),
                            _desc(dq4), _desc(dk4), _desc(dv4), workspace.data_ptr(), nbytes,
                            _stream(dev)))
    return dq4.reshape(query.shape), dk4.reshape(key.shape), dv4.reshape(value.shape)


def sdpa_bwd_varlen(q, k, v, out, lse, grad, cu_seqlens_q, cu_seqlens_k=None, max_seqlen_q=None,
                    max_seqlen_k=None, is_causal=False, scale=None, enable_gqa=False, workspace=None):
    """Gradients of packed variable-length attention (sdpa_fwd_varlen's block-
    diagonal mask): returns (grad_q, grad_k, grad_v) shaped like q, k, v.

    Layouts as for sdpa_fwd_varlen: q, k, v, out and grad (total, heads, head
    dim) or (1, total, heads, head dim); lse (Hq, total_q) or (1, Hq, total_q)
    as sdpa_fwd_varlen returns it.
    """
    lib = load_library()
    _require_gpu(q, k, v, out, lse, grad, cu_seqlens_q, cu_seqlens_k)
    if q.dtype not in _DTYPE or any(t.dtype != q.dtype for t in (k, v, out, grad)):
        raise ValueError("q, k, v, out and grad must share one of float32, float16, bfloat16")
    batched = q.dim() == 4
    q3, k3, v3, o3, g3 = (t[0] if t.dim() == 4 else t for t in (q, k, v, out, grad))
    l2 = lse[0] if lse.dim() == 3 else lse
    if cu_seqlens_k is None:
        cu_seqlens_k = cu_seqlens_q
    for c in (cu_seqlens_q, cu_seqlens_k):
        if c.dtype != torch.int32 or c.dim() != 1 or not c.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous 1-D int32 device tensors")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    n_seqs = cu_seqlens_q.numel() - 1
    if max_seqlen_q is None or max_seqlen_k is None:
        cq, ck = cu_seqlens_q.cpu().long(), cu_seqlens_k.cpu().long()
        max_seqlen_q = int((cq[1:] - cq[:-1]).max()) if n_seqs > 0 else 0
        max_seqlen_k = int((ck[1:] - ck[:-1]).max()) if n_seqs > 0 else 0
    total_q, Hq, E = q3.shape
    total_k, Hkv, _ = k3.shape
    Ev = v3.shape[2]
    for t in (q3, k3, v3, o3, g3, l2):
        if t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError("the last dimension must have stride 1")
    dev = q.device
    dq3 = torch.empty((total_q, Hq, E), dtype=q.dtype, device=dev)
    dk3 = torch.empty((total_k, Hkv, E), dtype=q.dtype, device=dev)
    dv3 = torch.empty((total_k, Hkv, Ev), dtype=q.dtype, device=dev)
    with torch.cuda.device(dev):
        n = ctypes.c_size_t(0)
        _check(lib.sdpa_bwd_varlen_workspace_size(Hq, total_q, ctypes.byref(n)))
        if workspace is None or workspace.numel() < n.value:
            workspace = torch.empty(n.value, dtype=torch.uint8, device=dev)
        _check(lib.sdpa_bwd_varlen(
            _DTYPE[q.dtype], q3.data_ptr(), q3.stride(0), q3.stride(1), k3.data_ptr(), k3.stride(0), k3.stride(1),
            v3.data_ptr(), v3.stride(0), v3.stride(1), o3.data_ptr(), o3.stride(0), o3.stride(1),
            l2.data_ptr(), l2.stride(0), g3.data_ptr(), g3.stride(0), g3.stride(1),
            cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), n_seqs, int(max_seqlen_q), int(max_seqlen_k),
            Hq, Hkv, E, Ev, total_q, total_k, int(bool(is_causal)), _scale_arg(scale), int(bool(enable_gqa)),
            dq3.data_ptr(), dq3.stride(0), dq3.stride(1), dk3.data_ptr(), dk3.stride(0), dk3.stride(1),
            dv3.data_ptr(), dv3.stride(0), dv3.stride(1), workspace.data_ptr(), n.value, _stream(dev)))
    if batched:
        return dq3.unsqueeze(0), dk3.unsqueeze(0), dv3.unsqueeze(0)
    return dq3, dk3, dv3


def sdpa_fwd_bmhk(query, key, value, is_causal=False, scale=None, num_splits=0):
    """Attention in the xFormers layouts of the insureai360 tutorial: BMHK
    (B, M, H, K) with the sequence before the heads, or the 5-D grouped-query
    BMGHK (B, M, G, Hq, K) with key/value (B, M, G, 1, K) shared by the Hq
    query heads of each of the G groups (tutorial section 5).

    No copies: the tensors are handed to sdpa_fwd as strided (B, heads, M, K)
    views, query head g*Hq + j reading key/value head g (contiguous groups).
    Returns the output in the query's layout and lse (B, heads, M) float32.
    """
    if query.dim() == 4:
        q4, k4, v4 = (t.permute(0, 2, 1, 3) for t in (query, key, value))
        gqa = q4.shape[1] != k4.shape[1]
    elif query.dim() == 5:
        B, M, G, Hq, K = query.shape
        if key.dim() != 5 or key.shape[2] != G or key.shape[3] != 1 or value.shape[3] != 1:
            raise ValueError("BMGHK: key and value must be (B, M, G, 1, K) with the query's G")
        if query.stride(2) != Hq * query.stride(3):
            raise ValueError("BMGHK: the group and head axes of the query must be packed (G outer)")
        q4 = query.reshape(B, M, G * Hq, K).permute(0, 2, 1, 3) if query.is_contiguous() else \
            query.as_strided((B, G * Hq, M, K), (query.stride(0), query.stride(3), query.stride(1), query.stride(4)))
        k4 = key[:, :, :, 0].permute(0, 2, 1, 3)
        v4 = value[:, :, :, 0].permute(0, 2, 1, 3)
        gqa = Hq != 1
    else:
        raise ValueError("expected a 4-D BMHK or a 5-D BMGHK query")
    B, H, M = q4.shape[:3]
    Ev = v4.shape[3]
    out = torch.empty(query.shape[:-1] + (Ev,), dtype=query.dtype, device=query.device)
    o4 = out.permute(0, 2, 1, 3) if out.dim() == 4 else out.reshape(B, M, H, Ev).permute(0, 2, 1, 3)
    lse = torch.empty((B, H, M, 1), dtype=torch.float32, device=query.device)
    sdpa_fwd(q4, k4, v4, is_causal=is_causal, scale=scale, enable_gqa=gqa, num_splits=num_splits,
             out=o4, lse=lse)
    return out, lse.reshape(B, H, M)


def sdpa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None,
                    dropout_p=0.0, is_causal=False, scale=None, enable_gqa=False, out=None, lse=None):
    """Packed variable-length attention with a block-diagonal (optionally causal) mask.

    q (total_q, Hq, E) or (1, total_q, Hq, E) -- the BMHK layout of the
    insureai360 xFormers tutorial, section 4; k, v likewise; cu_seqlens are
    int32 device tensors of n_seqs + 1 offsets.  Returns out shaped like q
    (with Ev) and lse (Hq, total_q) (or (1, Hq, total_q) for 4-D input).
    ``out`` (total_q, Hq, Ev) and ``lse`` (Hq, total_q) may be passed in
    (written in place; the returned tensors are views of them).
    """
    lib = load_library()
    _require_gpu(q, k, v, cu_seqlens_q, cu_seqlens_k)
    if q.dtype not in _DTYPE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one of float32, float16, bfloat16")
    batched = q.dim() == 4
    q3, k3, v3 = (t[0] if t.dim() == 4 else t for t in (q, k, v))
    if cu_seqlens_k is None:
        cu_seqlens_k = cu_seqlens_q
    for c in (cu_seqlens_q, cu_seqlens_k):
        if c.dtype != torch.int32 or c.dim() != 1 or not c.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous 1-D int32 device tensors")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    n_seqs = cu_seqlens_q.numel() - 1
    if max_seqlen_q is None or max_seqlen_k is None:
        cq = cu_seqlens_q.cpu().long()
        ck = cu_seqlens_k.cpu().long()
        max_seqlen_q = int((cq[1:] - cq[:-1]).max()) if n_seqs > 0 else 0
        max_seqlen_k = int((ck[1:] - ck[:-1]).max()) if n_seqs > 0 else 0
    total_q, Hq, E = q3.shape
    total_k, Hkv, _ = k3.shape
    Ev = v3.shape[2]
    for t in (q3, k3, v3):
        if t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError("the last dimension must have stride 1")
    dev = q.device
    if out is None:
        out3 = torch.empty((total_q, Hq, Ev), dtype=q.dtype, device=dev)
    else:
        out3 = out[0] if out.dim() == 4 else out
        if tuple(out3.shape) != (total_q, Hq, Ev) or out3.dtype != q.dtype or out3.stride(-1) != 1:
            raise ValueError(f"out must be ({total_q}, {Hq}, {Ev}) {q.dtype} with unit last stride")
    if lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=dev)
    else:
        lse = lse[0] if lse.dim() == 3 else lse
        if tuple(lse.shape) != (Hq, total_q) or lse.dtype != torch.float32 or lse.stride(1) != 1:
            raise ValueError(f"lse must be ({Hq}, {total_q}) float32 with unit last stride")
    _require_gpu(out3, lse)
    with torch.cuda.device(dev):
        _check(lib.sdpa_fwd_varlen(
            _DTYPE[q.dtype], q3.data_ptr(), q3.stride(0), q3.stride(1),
            k3.data_ptr(), k3.stride(0), k3.stride(1), v3.data_ptr(), v3.stride(0), v3.stride(1),
            cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), n_seqs, int(max_seqlen_q),
            int(max_seqlen_k), Hq, Hkv, E, Ev, total_q, total_k, float(dropout_p),
            int(bool(is_causal)), _scale_arg(scale), int(bool(enable_gqa)),
            out3.data_ptr(), out3.stride(0), out3.stride(1), lse.data_ptr(), lse.stride(0),
            _stream(dev)))
    if batched:
        return out3.unsqueeze(0), lse.unsqueeze(0)
    return out3, lse


class PreparedSdpaFwd:
    """sdpa_fwd with its arguments marshalled once, for repeated calls on the same buffers.

    Calling the object enqueues the same C call again (one ctypes call per
    launch) on the stream that was current when it was prepared; the tensors
    must stay alive and keep their storage.  Returns (out, lse).
    """

    def __init__(self, query, key, value, attn_mask=None, dropout_p=0.0, is_causal=False, scale=None,
                 enable_gqa=False, num_splits=0, out=None, lse=None):
        lib = load_library()
        _require_gpu(query, key, value, attn_mask, out, lse)
        q4, k4, v4 = _as4d(query), _as4d(key), _as4d(value)
        k4, v4 = _expand_batch(q4, k4), _expand_batch(q4, v4)
        B, Hq, L, _ = q4.shape
        S, Ev = v4.shape[2], v4.shape[3]
        m4, mdt = _mask_4d(attn_mask, q4, S)
        dev = query.device
        self.out = out if out is not None else torch.empty((B, Hq, L, Ev), dtype=query.dtype, device=dev)
        self.lse = lse if lse is not None else torch.empty((B, Hq, L, 1), dtype=torch.float32, device=dev)
        self._keep = (q4, k4, v4, m4)
        self._d = [_desc(q4), _desc(k4), _desc(v4), _desc(self.out), _desc(self.lse)]
        self._dm = _desc(m4) if m4 is not None else None
        pm = ctypes.byref(self._dm) if self._dm is not None else None
        n = ctypes.c_size_t(0)
        _check(lib.sdpa_fwd_workspace_size(_DTYPE[query.dtype], self._d[0], self._d[1], self._d[2], pm,
                                           int(bool(is_causal)), int(bool(enable_gqa)), int(num_splits),
                                           ctypes.byref(n)))
        self.workspace = torch.empty(n.value, dtype=torch.uint8, device=dev) if n.value else None
        self._scale = ctypes.c_double(float(scale)) if scale is not None else None
        self._args = (_DTYPE[query.dtype], ctypes.byref(self._d[0]), ctypes.byref(self._d[1]),
                      ctypes.byref(self._d[2]), pm, mdt, float(dropout_p), int(bool(is_causal)),
                      ctypes.byref(self._scale) if self._scale is not None else None, int(bool(enable_gqa)),
                      ctypes.byref(self._d[3]), ctypes.byref(self._d[4]),
                      self.workspace.data_ptr() if self.workspace is not None else None, n.value,
                      int(num_splits), _stream(dev))
        self._fn = lib.sdpa_fwd

    def __call__(self):
        _check(self._fn(*self._args))
        return self.out, self.lse
