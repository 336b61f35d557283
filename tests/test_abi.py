"""The C interface, checked on the host: library loads, exports what include/sdpa.h
declares, and rejects bad arguments before enqueueing any GPU work.

Every call here fails validation on the host, so the (fake) device pointers
are never dereferenced and no kernel is launched; no GPU is needed.
"""
import ctypes
import os
import re

import pytest

from transformer_attention_04_amd import sdpa as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdpa.h")

FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced


@pytest.fixture(scope="module")
def lib():
    # SDPA_TEST_LIBRARY: another build of the same interface (the sanitized host
    # build of tests/test_abi_sanitized.py), loaded in place of libsdpa.so
    other = os.environ.get("SDPA_TEST_LIBRARY")
    if other:
        S._LIB_PATH, S._lib = other, None
    if not os.path.exists(S.library_path()):
        pytest.skip("libsdpa.so is not built (python -m transformer_attention_04_amd.build_lib)")
    return S.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdpa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert {"sdpa_fwd", "sdpa_fwd_varlen", "sdpa_fwd_workspace_size", "sdpa_last_error"} <= set(names)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(S.EXPORTED) == set(declared_functions())
    assert lib.sdpa_abi_version() == 5


def t4(shape, strides=None, data=FAKE):
    d = S.SdpaTensor4()
    d.data = data
    if strides is None:
        strides, acc = [0] * 4, 1
        for i in range(3, -1, -1):
            strides[i] = acc
            acc *= shape[i]
    for i in range(4):
        d.size[i] = shape[i]
        d.stride[i] = strides[i]
    return d


def call(lib, q, k, v, out=None, lse=None, mask=None, mask_dtype=S.SDPA_F32, dtype=S.SDPA_BF16,
         dropout=0.0, causal=0, scale=None, gqa=0, ws=None, ws_bytes=0, splits=0):
    if out is None:
        out = t4((q.size[0], q.size[1], q.size[2], v.size[3]))
    if lse is None:
        lse = t4((q.size[0], q.size[1], q.size[2], 1))
    sc = ctypes.byref(ctypes.c_double(scale)) if scale is not None else None
    st = lib.sdpa_fwd(dtype, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                      ctypes.byref(mask) if mask is not None else None, mask_dtype, dropout, causal,
                      sc, gqa, ctypes.byref(out), ctypes.byref(lse), ws, ws_bytes, splits, None)
    return st, lib.sdpa_last_error().decode()


def qkv(B=2, Hq=4, Hkv=4, L=16, S_=32, E=64, Ev=None):
    Ev = E if Ev is None else Ev
    return t4((B, Hq, L, E)), t4((B, Hkv, S_, E)), t4((B, Hkv, S_, Ev))


def test_dropout_is_rejected(lib):
    st, msg = call(lib, *qkv(), dropout=0.1)
    assert st == S.SDPA_ERR_INVALID_ARGUMENT and "dropout" in msg


def test_bad_dtype(lib):
    st, _ = call(lib, *qkv(), dtype=S.SDPA_BOOL)
    assert st == S.SDPA_ERR_INVALID_ARGUMENT


def test_shape_mismatches(lib):
    q, k, v = qkv()
    k.size[3] = 32
    assert call(lib, q, k, v)[0] == S.SDPA_ERR_INVALID_ARGUMENT  # E differs
    q, k, v = qkv()
    v.size[2] = 31
    assert call(lib, q, k, v)[0] == S.SDPA_ERR_INVALID_ARGUMENT  # S differs
    q, k, v = qkv()
    st, _ = call(lib, q, k, v, out=t4((2, 4, 16, 32)))
    assert st == S.SDPA_ERR_INVALID_ARGUMENT  # out shape
    st, _ = call(lib, q, k, v, lse=t4((2, 4, 16, 2)))
    assert st == S.SDPA_ERR_INVALID_ARGUMENT  # lse shape


def test_gqa_rules(lib):
    st, msg = call(lib, *qkv(Hq=8, Hkv=2))
    assert st == S.SDPA_ERR_INVALID_ARGUMENT and "enable_gqa" in msg
    st, _ = call(lib, *qkv(Hq=8, Hkv=3), gqa=1)
    assert st == S.SDPA_ERR_INVALID_ARGUMENT


def test_head_dim_limits(lib):
    """Head dims E and Ev must be multiples of 8 up to 128 (E = 0 included); calls
    outside that are refused before anything is launched."""
    for e in (4, 84, 136, 256):
        st, _ = call(lib, *qkv(E=e))
        assert st == S.SDPA_ERR_UNSUPPORTED, e
        st, _ = call(lib, *qkv(E=e), dtype=S.SDPA_F32)
        assert st == S.SDPA_ERR_UNSUPPORTED, e
    for ev in (12, 132):
        st, msg = call(lib, *qkv(E=64, Ev=ev))
        assert st == S.SDPA_ERR_UNSUPPORTED and "Ev" in msg, ev
        st, msg = call(lib, *qkv(E=128, Ev=ev), dtype=S.SDPA_F32, mask=t4((1, 1, 16, 32)))
        assert st == S.SDPA_ERR_UNSUPPORTED and "Ev" in msg, ev
    # the split-KV decode takes head dims 64, 96, 128 only; others run single-pass (no workspace)
    for E, Ev in ((80, 80), (0, 64), (64, 40)):
        q, k, v = qkv(L=1, E=E, Ev=Ev)
        n = ctypes.c_size_t(0)
        st = lib.sdpa_fwd_workspace_size(S.SDPA_BF16, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                         None, 0, 0, 2, ctypes.byref(n))
        assert st == S.SDPA_ERR_UNSUPPORTED, (E, Ev)
        st = lib.sdpa_fwd_workspace_size(S.SDPA_BF16, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                         None, 0, 0, 0, ctypes.byref(n))
        assert st == S.SDPA_OK and n.value == 0, (E, Ev)


def test_layout_requirements(lib):
    q, k, v = qkv()
    q.data = FAKE + 2
    assert call(lib, q, k, v)[0] == S.SDPA_ERR_UNSUPPORTED  # misaligned base
    q, k, v = qkv()
    k.stride[3] = 2
    assert call(lib, q, k, v)[0] == S.SDPA_ERR_UNSUPPORTED  # non-unit last stride
    q, k, v = qkv()
    v.stride[2] = 68
    assert call(lib, q, k, v)[0] == S.SDPA_ERR_UNSUPPORTED  # row stride not a multiple of 8


def test_mask_checks(lib):
    q, k, v = qkv()
    st, _ = call(lib, q, k, v, mask=t4((2, 4, 16, 31)))
    assert st == S.SDPA_ERR_INVALID_ARGUMENT  # key dim must match
    st, _ = call(lib, q, k, v, mask=t4((3, 4, 16, 32)))
    assert st == S.SDPA_ERR_INVALID_ARGUMENT  # batch neither 1 nor B
    st, _ = call(lib, q, k, v, mask=t4((1, 1, 16, 32)), mask_dtype=S.SDPA_BF16)
    assert st == S.SDPA_ERR_INVALID_ARGUMENT  # mask dtype
    st, _ = call(lib, q, k, v, mask=t4((1, 1, 16, 32)), splits=2)
    assert st == S.SDPA_ERR_UNSUPPORTED  # the decode kernel takes no mask


def test_non_finite_scale(lib):
    st, msg = call(lib, *qkv(), scale=float("inf"))
    assert st == S.SDPA_ERR_INVALID_ARGUMENT and "scale" in msg


def test_workspace_size_and_too_small(lib):
    q, k, v = qkv(B=64, Hq=32, Hkv=8, L=1, S_=32768, E=128)
    n = ctypes.c_size_t(0)
    st = lib.sdpa_fwd_workspace_size(S.SDPA_BF16, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                     None, 0, 1, 0, ctypes.byref(n))
    assert st == S.SDPA_OK and n.value > 64 * 32 * 129 * 4
    st, msg = call(lib, q, k, v, gqa=1, ws=FAKE, ws_bytes=n.value - 1)
    assert st == S.SDPA_ERR_INVALID_ARGUMENT and "workspace" in msg
    # the single-pass kernel needs none
    st = lib.sdpa_fwd_workspace_size(S.SDPA_BF16, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                     None, 0, 1, -1, ctypes.byref(n))
    assert st == S.SDPA_OK and n.value == 0
    # causal calls are not eligible for the split kernel
    st = lib.sdpa_fwd_workspace_size(S.SDPA_BF16, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                     None, 1, 1, 4, ctypes.byref(n))
    assert st == S.SDPA_ERR_UNSUPPORTED
    st = lib.sdpa_fwd_workspace_size(S.SDPA_BF16, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                     None, 0, 1, -2, ctypes.byref(n))
    assert st == S.SDPA_ERR_INVALID_ARGUMENT


def test_varlen_argument_errors(lib):
    def varlen(**kw):
        a = dict(dtype=S.SDPA_F16, q=FAKE, qt=512, qh=64, k=FAKE, kt=512, kh=64, v=FAKE, vt=512,
                 vh=64, cq=FAKE, ck=FAKE, n=4, mq=200, mk=200, Hq=8, Hkv=8, E=64, Ev=64, tq=365,
                 tk=365, drop=0.0, causal=1, gqa=0, o=FAKE, ot=512, oh=64, lse=FAKE, lh=365)
        a.update(kw)
        st = lib.sdpa_fwd_varlen(a["dtype"], a["q"], a["qt"], a["qh"], a["k"], a["kt"], a["kh"],
                                 a["v"], a["vt"], a["vh"], a["cq"], a["ck"], a["n"], a["mq"], a["mk"],
                                 a["Hq"], a["Hkv"], a["E"], a["Ev"], a["tq"], a["tk"], a["drop"],
                                 a["causal"], None, a["gqa"], a["o"], a["ot"], a["oh"], a["lse"],
                                 a["lh"], None)
        return st
    assert varlen(drop=0.5) == S.SDPA_ERR_INVALID_ARGUMENT
    assert varlen(Hkv=2) == S.SDPA_ERR_INVALID_ARGUMENT
    assert varlen(Hkv=3, gqa=1) == S.SDPA_ERR_INVALID_ARGUMENT
    assert varlen(cq=None) == S.SDPA_ERR_INVALID_ARGUMENT
    assert varlen(E=84, Ev=84) == S.SDPA_ERR_UNSUPPORTED
    assert varlen(E=64, Ev=136) == S.SDPA_ERR_UNSUPPORTED
    assert varlen(dtype=S.SDPA_F32, E=132, Ev=128) == S.SDPA_ERR_UNSUPPORTED
    assert varlen(q=FAKE + 4) == S.SDPA_ERR_UNSUPPORTED
    assert varlen(kt=510) == S.SDPA_ERR_UNSUPPORTED
    assert varlen(n=-1) == S.SDPA_ERR_INVALID_ARGUMENT
    # nothing to do is not an error and launches nothing
    assert varlen(n=0) == S.SDPA_OK
    assert varlen(tq=0) == S.SDPA_OK


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    if not os.path.exists(S.library_path()):
        pytest.skip("libsdpa.so is not built")
    with pytest.raises(ValueError, match="GPU"):
        S.sdpa_fwd(q, q, q)


def test_paged_plan_rules(lib):
    """sdpa_fwd_paged_workspace_size (host only): decode steps get a split-KV
    workspace, longer chunks of new rows (chunked prefill) need none and take no
    split count; page size, head dims and dtype are checked."""
    def ws(L=1, Hq=8, Hkv=2, E=128, Ev=128, ps=64, dtype=S.SDPA_BF16, splits=0, max_len=4096):
        q, kc, vc = t4((4, Hq, L, E)), t4((100, Hkv, ps, E)), t4((100, Hkv, ps, Ev))
        n = ctypes.c_size_t(12345)
        st = lib.sdpa_fwd_paged_workspace_size(dtype, ctypes.byref(q), ctypes.byref(kc), ctypes.byref(vc),
                                               max_len, 1, splits, ctypes.byref(n))
        return st, n.value
    st, n = ws(L=4)                        # 16 rows per cache head: split-KV decode
    assert st == S.SDPA_OK and n > 4 * 8 * 4 * 128 * 4
    st, n = ws(L=5)                        # 20 rows: chunked prefill, no workspace
    assert st == S.SDPA_OK and n == 0
    st, n = ws(L=512, Hq=32, Hkv=8)
    assert st == S.SDPA_OK and n == 0
    assert ws(L=512, splits=2)[0] == S.SDPA_ERR_UNSUPPORTED
    assert ws(L=4, splits=2)[0] == S.SDPA_OK
    assert ws(ps=48)[0] == S.SDPA_ERR_UNSUPPORTED
    assert ws(ps=8)[0] == S.SDPA_ERR_UNSUPPORTED
    st, n = ws(L=4, E=64, Ev=128)          # Ev != E decode: split-KV with Ev-wide partials
    assert st == S.SDPA_OK and n > 4 * 8 * 4 * 128 * 4
    assert ws(L=1, E=40, Ev=40) == (S.SDPA_OK, 0)   # other head dims: single pass, decode steps too
    assert ws(L=1, E=40, Ev=40, splits=2)[0] == S.SDPA_ERR_UNSUPPORTED
    assert ws(E=84, Ev=84)[0] == S.SDPA_ERR_UNSUPPORTED
    assert ws(dtype=S.SDPA_F32)[0] == S.SDPA_ERR_UNSUPPORTED
    assert ws(splits=-1)[0] == S.SDPA_ERR_INVALID_ARGUMENT


def test_varlen_backward_argument_errors(lib):
    def call(**kw):
        a = dict(dtype=S.SDPA_BF16, ptr=FAKE, st=1024, sh=128, lse=FAKE, lsh=365, cq=FAKE, ck=FAKE, n=4,
                 mq=200, mk=200, Hq=8, Hkv=8, E=128, Ev=128, tq=365, tk=365, causal=1, gqa=0, ws=FAKE,
                 wsb=1 << 20)
        a.update(kw)
        p, st, sh = a["ptr"], a["st"], a["sh"]
        return lib.sdpa_bwd_varlen(a["dtype"], p, st, sh, p, st, sh, p, st, sh, p, st, sh, a["lse"], a["lsh"],
                                   p, st, sh, a["cq"], a["ck"], a["n"], a["mq"], a["mk"], a["Hq"], a["Hkv"],
                                   a["E"], a["Ev"], a["tq"], a["tk"], a["causal"], None, a["gqa"],
                                   p, st, sh, p, st, sh, p, st, sh, a["ws"], a["wsb"], None)
    assert call(dtype=S.SDPA_BOOL) == S.SDPA_ERR_INVALID_ARGUMENT
    assert call(Hkv=2) == S.SDPA_ERR_INVALID_ARGUMENT        # grouped heads need enable_gqa
    assert call(Hkv=3, gqa=1) == S.SDPA_ERR_INVALID_ARGUMENT
    assert call(cq=None) == S.SDPA_ERR_INVALID_ARGUMENT
    assert call(E=128, Ev=136) == S.SDPA_ERR_UNSUPPORTED       # head dims up to 128
    assert call(E=12, Ev=12) == S.SDPA_ERR_UNSUPPORTED         # multiples of 8
    assert call(ptr=FAKE + 8) == S.SDPA_ERR_UNSUPPORTED       # misaligned base
    assert call(st=1020) == S.SDPA_ERR_UNSUPPORTED            # stride not a multiple of 8
    assert call(wsb=8 * 365 * 4) == S.SDPA_ERR_INVALID_ARGUMENT   # workspace too small
    assert call(n=-1) == S.SDPA_ERR_INVALID_ARGUMENT
    assert call(n=0) == S.SDPA_OK                              # nothing to do
    n = ctypes.c_size_t(0)
    assert lib.sdpa_bwd_varlen_workspace_size(8, 365, ctypes.byref(n)) == S.SDPA_OK
    assert n.value == 8 * 365 * 4 + 256


def test_paged_varlen_argument_errors(lib):
    def call(**kw):
        a = dict(dtype=S.SDPA_BF16, q=FAKE, qt=1024, qh=128, cu=FAKE, n=3, mq=100, tq=250, Hq=8,
                 kc=t4((64, 2, 64, 128)), vc=t4((64, 2, 64, 128)), bt=FAKE, bts=16, mb=16, sl=FAKE, ms=1000,
                 causal=1, gqa=1, o=FAKE, ot=1024, oh=128, lse=FAKE, lh=250)
        a.update(kw)
        return lib.sdpa_fwd_paged_varlen(a["dtype"], a["q"], a["qt"], a["qh"], a["cu"], a["n"], a["mq"], a["tq"],
                                         a["Hq"], ctypes.byref(a["kc"]), ctypes.byref(a["vc"]), a["bt"], a["bts"],
                                         a["mb"], a["sl"], a["ms"], a["causal"], None, a["gqa"], a["o"], a["ot"],
                                         a["oh"], a["lse"], a["lh"], None)
    assert call(dtype=S.SDPA_F32) == S.SDPA_ERR_UNSUPPORTED
    assert call(gqa=0) == S.SDPA_ERR_INVALID_ARGUMENT          # 8 query heads over 2 cache heads
    assert call(Hq=5) == S.SDPA_ERR_INVALID_ARGUMENT           # not a multiple of the cache heads
    assert call(kc=t4((64, 2, 48, 128)), vc=t4((64, 2, 48, 128))) == S.SDPA_ERR_UNSUPPORTED  # page size
    assert call(vc=t4((64, 2, 64, 84))) == S.SDPA_ERR_UNSUPPORTED                           # Ev % 8 != 0
    assert call(vc=t4((63, 2, 64, 128))) == S.SDPA_ERR_INVALID_ARGUMENT                     # pools differ
    assert call(bts=8) == S.SDPA_ERR_INVALID_ARGUMENT           # max_blocks > table stride
    assert call(cu=None) == S.SDPA_ERR_INVALID_ARGUMENT
    assert call(q=FAKE + 8) == S.SDPA_ERR_UNSUPPORTED           # misaligned base
    assert call(qt=1020) == S.SDPA_ERR_UNSUPPORTED              # stride not a multiple of 8
    assert call(n=0) == S.SDPA_OK                               # nothing to do
