"""Host-side checks of the C ABI that need no GPU: the library loads, exports every
entry point include/libattn.h declares, and rejects bad arguments with the documented
status code before touching the device (so these calls never launch anything)."""
import ctypes
import os
import re

import numpy as np
import pytest

import attention_flash_attn_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libattn.h")

OK, NULL, SHAPE, UNSUP, SEQ = 0, 1, 2, 3, 4
# A non-null address that is never dereferenced: every call below fails validation
# (or is zero-sized) before any device work.
P = ctypes.c_void_p(0x1000)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(A.LIB_PATH):
        pytest.skip("libattn.so not built")
    return A.lib()


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(attn_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(L):
    names = declared()
    assert {"attn_fwd", "attn_bwd_preprocess", "attn_bwd", "attn_varlen_fwd",
            "attn_varlen_bwd", "attn_lse_merge", "attn_bwd_accum", "attn_cast_bf16",
            "attn_fwd_gqa", "attn_bwd_gqa", "attn_fwd_ex", "attn_bwd_ex", "attn_varlen_fwd_ex",
            "attn_varlen_bwd_ex"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert L.attn_abi_version() == 5
    assert L.attn_status_str(0) == b"ok"
    assert L.attn_status_str(4) == b"invalid cu_seqlens"


def test_status_enum_matches_header():
    text = open(HEADER).read()
    block = re.search(r"typedef\s+enum\s*\{(.*?)\}\s*attn_status\s*;", text, re.S)
    assert block, "attn_status enum not found"
    enum = dict((k, int(v)) for k, v in re.findall(r"(ATTN_\w+)\s*=\s*(\d+)", block.group(1)))
    assert {v: k for k, v in enum.items()} == A.STATUS


def fwd(L, B=1, Sq=8, Sk=8, H=2, D=64, scale=0.125, q=P, k=P, v=P, m=None, out=P, lse=P):
    return L.attn_fwd(B, Sq, Sk, H, D, scale, q, k, v, m, out, lse, None)


def test_fwd_validation(L):
    assert fwd(L, q=None) == NULL
    assert fwd(L, lse=None) == NULL
    assert fwd(L, B=-1) == SHAPE
    assert fwd(L, Sk=-3) == SHAPE
    assert fwd(L, scale=0.0) == SHAPE
    assert fwd(L, scale=float("nan")) == SHAPE
    assert fwd(L, scale=float("inf")) == SHAPE
    assert fwd(L, scale=1e-30) == SHAPE  # below 2^-64
    for D in (0, 32, 96, 256):
        assert fwd(L, D=D) == UNSUP
    assert fwd(L, B=2, Sq=2 ** 30 + 1) == UNSUP
    # rows wider than 2^22 elements (H * D): tile copies use 32-bit byte offsets
    assert fwd(L, H=2 ** 15, D=128) == UNSUP
    assert fwd(L, H=2 ** 16, D=64) == UNSUP
    # zero-sized problems succeed without launching anything
    assert fwd(L, B=0) == OK
    assert fwd(L, Sq=0) == OK
    assert fwd(L, H=0) == OK


def test_preprocess_and_bwd_validation(L):
    assert L.attn_bwd_preprocess(1, 8, 2, 64, P, None, P, None) == NULL
    assert L.attn_bwd_preprocess(1, -8, 2, 64, P, P, P, None) == SHAPE
    assert L.attn_bwd_preprocess(1, 8, 2, 80, P, P, P, None) == UNSUP
    assert L.attn_bwd_preprocess(0, 8, 2, 64, P, P, P, None) == OK
    args = [1, 8, 8, 2, 64, 0.125, P, P, P, None, P, P, P, P, P, P, None]
    for i in (6, 7, 8, 10, 11, 12, 13, 14, 15):  # every tensor but the mask is required
        a = list(args)
        a[i] = None
        assert L.attn_bwd(*a) == NULL, i
    a = list(args)
    a[4] = 48
    assert L.attn_bwd(*a) == UNSUP
    a = list(args)
    a[5] = -1.0
    assert L.attn_bwd(*a) == SHAPE
    a = list(args)
    a[0] = 0
    assert L.attn_bwd(*a) == OK


def test_merge_accum_cast_validation(L):
    n2 = (ctypes.c_void_p * 2)(P.value, P.value)
    n1null = (ctypes.c_void_p * 2)(P.value, None)

    def merge(n=2, B=1, S=8, H=2, D=128, outs=n2, lses=n2, out=P, lse=P):
        return L.attn_lse_merge(n, B, S, H, D, outs, lses, out, lse, None)

    assert merge(n=0) == SHAPE
    assert merge(n=17) == UNSUP
    assert merge(B=-1) == SHAPE
    assert merge(D=96) == UNSUP
    assert merge(outs=None) == NULL
    assert merge(lses=n1null) == NULL
    assert merge(out=None) == NULL
    assert merge(B=0, outs=n1null, lses=n1null, out=None, lse=None) == OK  # nothing to merge

    args = [1, 8, 8, 2, 64, 0.125, P, P, P, None, P, P, P, P, P, P, 3, None]
    for i in (6, 7, 8, 10, 11, 12, 13, 14, 15):
        a = list(args)
        a[i] = None
        assert L.attn_bwd_accum(*a) == NULL, i
    a = list(args)
    a[16] = 4  # unknown flag bit
    assert L.attn_bwd_accum(*a) == SHAPE
    a = list(args)
    a[4] = 96
    assert L.attn_bwd_accum(*a) == UNSUP
    a = list(args)
    a[5] = 0.0
    assert L.attn_bwd_accum(*a) == SHAPE
    a = list(args)
    a[3] = 0
    assert L.attn_bwd_accum(*a) == OK

    assert L.attn_cast_bf16(-1, P, P, None) == SHAPE
    assert L.attn_cast_bf16(4, None, P, None) == NULL
    assert L.attn_cast_bf16(4, P, None, None) == NULL
    assert L.attn_cast_bf16(0, None, None, None) == OK


def test_gqa_validation(L):
    def fwd(H=8, Hk=2, B=1, S=8):
        return L.attn_fwd_gqa(B, S, S, H, Hk, 64, 0.125, P, P, P, None, P, P, None)

    def bwd(H=8, Hk=2, B=1, S=8):
        return L.attn_bwd_gqa(B, S, S, H, Hk, 64, 0.125, P, P, P, None, P, P, P, P, P, P, None)

    for f in (fwd, bwd):
        assert f(Hk=3) == SHAPE   # must divide H
        assert f(Hk=0) == SHAPE
        assert f(Hk=-2) == SHAPE
        assert f(Hk=16) == SHAPE  # more key/value heads than query heads
        assert f(H=0, Hk=0) == OK
        assert f(B=0) == OK
    assert L.attn_fwd_gqa(1, 8, 8, 8, 2, 64, 0.125, P, None, P, None, P, P, None) == NULL
    # flags: only ATTN_CAUSAL (1) is defined
    assert L.attn_fwd_ex(1, 8, 8, 8, 2, 64, 0.125, 2, P, P, P, None, P, P, None) == SHAPE
    assert L.attn_bwd_ex(1, 8, 8, 8, 2, 64, 0.125, 4, P, P, P, None, P, P, P, P, P, P, None) == SHAPE
    assert L.attn_fwd_ex(0, 8, 8, 8, 2, 64, 0.125, 1, P, P, P, None, P, P, None) == OK
    arr = np.array([0, 4], dtype=np.int32)
    cu = arr.ctypes.data_as(ctypes.c_void_p)
    assert L.attn_varlen_fwd_ex(1, cu, P, 2, 64, 0.1, 8, P, P, P, P, P, None) == SHAPE
    assert L.attn_varlen_bwd_ex(1, cu, P, 2, 64, 0.1, 8, P, P, P, P, P, P, P, P, P, None) == SHAPE


def _cu(vals):
    arr = np.array(vals, dtype=np.int32)
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def test_varlen_validation(L):
    def call(vals, nseq=None, H=2, D=128):
        arr, p = _cu(vals)
        n = len(vals) - 1 if nseq is None else nseq
        f = L.attn_varlen_fwd(n, p, P, H, D, 0.1, P, P, P, P, P, None)
        b = L.attn_varlen_bwd(n, p, P, H, D, 0.1, P, P, P, P, P, P, P, P, P, None)
        return f, b

    assert call([1, 5, 9]) == (SEQ, SEQ)        # must start at 0
    assert call([0, 5, 4]) == (SEQ, SEQ)        # must not decrease
    assert call([0, 5, 9], D=72) == (UNSUP, UNSUP)
    assert call([0, 5, 9], H=2 ** 15) == (UNSUP, UNSUP)
    assert call([0, 5, 9], nseq=-1) == (SHAPE, SHAPE)
    assert call([0]) == (OK, OK)                # no sequences: nothing to do
    assert call([0, 0, 0]) == (OK, OK)          # empty sequences: T = 0
    assert call([0, 5, 9], H=0) == (OK, OK)
    # grouped-query heads: Hk must divide H
    arr, p = _cu([0, 5, 9])
    for Hk, want in ((3, SHAPE), (0, SHAPE), (-1, SHAPE)):
        assert L.attn_varlen_fwd_gqa(2, p, P, 4, Hk, 128, 0.1, 0, P, P, P, P, P, None) == want
        assert L.attn_varlen_bwd_gqa(2, p, P, 4, Hk, 128, 0.1, 0, P, P, P, P, P, P, P, P, P,
                                     None) == want
    assert L.attn_varlen_fwd_gqa(2, p, P, 4, 2, 128, 0.1, 2, P, P, P, P, P, None) == SHAPE
    assert L.attn_varlen_fwd_gqa(2, p, P, 4, 2, 128, 0.1, 0, P, None, P, P, P, None) == NULL
    arr, p = _cu([0, 4])
    assert L.attn_varlen_fwd(1, None, P, 2, 64, 0.1, P, P, P, P, P, None) == NULL
    assert L.attn_varlen_fwd(1, p, None, 2, 64, 0.1, P, P, P, P, P, None) == NULL


def test_binding_rejects_per_head_mask_and_bad_shapes():
    torch = pytest.importorskip("torch")
    # Shape checks run before any device use; a CPU meta tensor is enough to reach them.
    B, S, H, D = 2, 16, 4, 64
    m = torch.ones((B, H, 1, S), dtype=torch.bool)
    with pytest.raises(ValueError, match="head-broadcast"):
        A._mask_arg(m, B, S, H)
    with pytest.raises(ValueError):
        A._mask_arg(torch.ones((B, S + 1), dtype=torch.bool), B, S, H)
    q = torch.empty((B, S, H, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device"):
        A._want(q, "q", (B, S, H, D), torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        A._want(q, "k", (B, H, S, D), torch.bfloat16)  # a K/V handed over in BHSD
    with pytest.raises(TypeError):
        A._want(q.float(), "q", (B, S, H, D), torch.bfloat16)
