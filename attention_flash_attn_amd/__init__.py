"""libattn: MI355X (gfx950) attention forward/backward behind a C ABI.

Thin ctypes binding over ``libattn.so`` with the same entry-point names as
``include/libattn.h``.  This layer only checks shapes, allocates outputs with
torch (device memory and the current stream are torch's only role) and
passes raw pointers; every step of the computation runs in the HIP kernels.
There is no fallback: if ``libattn.so`` has not been built the calls raise.

Tensors are bf16 CUDA(HIP) tensors, contiguous, BSHD (dense) or (T, H, D) /
(1, T, H, D) (varlen).  LSE and delta are fp32 (B, H, Sq) or (H, T).
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "LibAttnError", "lib", "attn_fwd", "attn_bwd_preprocess", "attn_bwd", "attn_varlen_fwd",
    "attn_varlen_bwd", "STATUS",
]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED",
          4: "ATTN_ERR_SEQLENS", 5: "ATTN_ERR_HIP"}

_lib = None


class LibAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")


def lib():
    """Load libattn.so (built in-tree by ``__graft_entry__.build()``) and declare its ABI."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with attention_flash_attn_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    i, f, vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    L.attn_status_str.argtypes = [i]
    L.attn_status_str.restype = ctypes.c_char_p
    L.attn_abi_version.argtypes = []
    L.attn_fwd.argtypes = [i, i, i, i, i, f, vp, vp, vp, vp, vp, vp, vp]
    L.attn_bwd_preprocess.argtypes = [i, i, i, i, vp, vp, vp, vp]
    L.attn_bwd.argtypes = [i, i, i, i, i, f, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.attn_varlen_fwd.argtypes = [i, vp, vp, i, i, f, vp, vp, vp, vp, vp, vp]
    L.attn_varlen_bwd.argtypes = [i, vp, vp, i, i, f, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.attn_lse_merge.argtypes = [i, i, i, i, i, vp, vp, vp, vp, vp]
    L.attn_fwd_gqa.argtypes = [i, i, i, i, i, i, f, vp, vp, vp, vp, vp, vp, vp]
    L.attn_fwd_ex.argtypes = [i, i, i, i, i, i, f, i, vp, vp, vp, vp, vp, vp, vp]
    L.attn_bwd_ex.argtypes = [i, i, i, i, i, i, f, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.attn_varlen_fwd_ex.argtypes = [i, vp, vp, i, i, f, i, vp, vp, vp, vp, vp, vp]
    L.attn_varlen_bwd_ex.argtypes = [i, vp, vp, i, i, f, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.attn_varlen_fwd_gqa.argtypes = [i, vp, vp, i, i, i, f, i, vp, vp, vp, vp, vp, vp]
    L.attn_varlen_bwd_gqa.argtypes = [i, vp, vp, i, i, i, f, i, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp]
    L.attn_bwd_gqa.argtypes = [i, i, i, i, i, i, f, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.attn_bwd_accum.argtypes = [i, i, i, i, i, f, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, vp]
    L.attn_cast_bf16.argtypes = [ctypes.c_int64, vp, vp, vp]
    for name in ("attn_abi_version", "attn_fwd", "attn_bwd_preprocess", "attn_bwd",
                 "attn_varlen_fwd", "attn_varlen_bwd", "attn_lse_merge", "attn_bwd_accum",
                 "attn_cast_bf16", "attn_fwd_gqa", "attn_bwd_gqa", "attn_fwd_ex", "attn_bwd_ex",
                 "attn_varlen_fwd_ex", "attn_varlen_bwd_ex", "attn_varlen_fwd_gqa",
                 "attn_varlen_bwd_gqa"):
        getattr(L, name).restype = i
    _lib = L
    return L


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _check(fn, status):
    if status != 0:
        raise LibAttnError(fn, status)


def _want(t, name, shape, dtype):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _mask_arg(key_mask, B, Sk, H):
    """Accept (B, Sk) or (B, 1, 1, Sk) bool/uint8; reject per-head (B, H, 1, Sk) masks."""
    torch = _torch()
    if key_mask is None:
        return None
    m = key_mask
    if m.dim() == 4:
        if m.shape[1] != 1 or m.shape[2] != 1:
            raise ValueError(f"only head-broadcast key masks (B,1,1,Sk) are supported, got "
                             f"{tuple(m.shape)}")
        m = m.reshape(m.shape[0], m.shape[3])
    if tuple(m.shape) != (B, Sk):
        raise ValueError(f"key_mask has shape {tuple(key_mask.shape)}, expected ({B}, {Sk})")
    if m.dtype == torch.bool:
        m = m.contiguous().view(torch.uint8)
    elif m.dtype != torch.uint8:
        raise TypeError("key_mask must be bool or uint8")
    if not m.is_cuda or not m.is_contiguous():
        raise ValueError("key_mask must be a contiguous device tensor")
    return m


def _dims(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D BSHD tensors")
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    return B, Sq, Sk, H, D


def _kv_heads(q, k):
    """Key/value heads of k (grouped-query attention when fewer than q's heads)."""
    H, Hk = q.shape[2], k.shape[2]
    if Hk < 1 or H % Hk:
        raise ValueError(f"k/v have {Hk} heads, which must divide the {H} query heads")
    return Hk


CAUSAL = 1


def attn_fwd(q, k, v, key_mask=None, scale=None, out=None, lse=None, causal=False):
    """out, lse = attn_fwd(q, k, v): q (B,Sq,H,D), k/v (B,Sk,Hk,D) bf16 (Hk dividing H:
    grouped-query attention, query head h reading key/value head h // (H/Hk))
    -> out bf16, lse fp32 (B,H,Sq).  causal: query i sees keys j <= i only."""
    torch = _torch()
    B, Sq, Sk, H, D = _dims(q, k)
    Hk = _kv_heads(q, k)
    _want(q, "q", (B, Sq, H, D), torch.bfloat16)
    _want(k, "k", (B, Sk, Hk, D), torch.bfloat16)
    _want(v, "v", (B, Sk, Hk, D), torch.bfloat16)
    m = _mask_arg(key_mask, B, Sk, H)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _want(out, "out", (B, Sq, H, D), torch.bfloat16)
    _want(lse, "lse", (B, H, Sq), torch.float32)
    _check("attn_fwd", lib().attn_fwd_ex(B, Sq, Sk, H, Hk, D, scale, CAUSAL if causal else 0,
                                         _ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(out),
                                         _ptr(lse), _stream()))
    return out, lse


def attn_bwd_preprocess(out, dout, delta=None):
    """delta = rowsum(dout * out) in fp32, (B, H, S); for varlen pass (1, T, H, D) tensors."""
    torch = _torch()
    if out.dim() == 3:
        out, dout = out[None], dout[None]
    B, S, H, D = out.shape
    _want(out, "out", (B, S, H, D), torch.bfloat16)
    _want(dout, "dout", (B, S, H, D), torch.bfloat16)
    if delta is None:
        delta = torch.empty((B, H, S), dtype=torch.float32, device=out.device)
    _want(delta, "delta", (B, H, S), torch.float32)
    _check("attn_bwd_preprocess", lib().attn_bwd_preprocess(B, S, H, D, _ptr(out), _ptr(dout),
                                                            _ptr(delta), _stream()))
    return delta


def attn_bwd(q, k, v, lse, delta, dout, key_mask=None, scale=None, dq=None, dk=None, dv=None,
             causal=False):
    """dq, dk, dv = attn_bwd(q, k, v, lse, delta, dout) (bf16 BSHD grads; dk, dv have k's
    Hk heads, each summing its query heads' contributions)."""
    torch = _torch()
    B, Sq, Sk, H, D = _dims(q, k)
    Hk = _kv_heads(q, k)
    _want(q, "q", (B, Sq, H, D), torch.bfloat16)
    _want(k, "k", (B, Sk, Hk, D), torch.bfloat16)
    _want(v, "v", (B, Sk, Hk, D), torch.bfloat16)
    _want(dout, "dout", (B, Sq, H, D), torch.bfloat16)
    _want(lse, "lse", (B, H, Sq), torch.float32)
    _want(delta, "delta", (B, H, Sq), torch.float32)
    m = _mask_arg(key_mask, B, Sk, H)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _want(dq, "dq", (B, Sq, H, D), torch.bfloat16)
    _want(dk, "dk", (B, Sk, Hk, D), torch.bfloat16)
    _want(dv, "dv", (B, Sk, Hk, D), torch.bfloat16)
    _check("attn_bwd", lib().attn_bwd_ex(B, Sq, Sk, H, Hk, D, scale, CAUSAL if causal else 0,
                                         _ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(lse),
                                         _ptr(delta), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                         _stream()))
    return dq, dk, dv


def _cu_args(cu_seqlens, device):
    """Host int32 copy (validated by the library) and a device copy of cu_seqlens.

    Accepts one array (host or device; the other copy is made here) or a
    (host_int32_tensor, device_int32_tensor) pair holding the same values, which
    avoids any copy per call."""
    torch = _torch()
    if isinstance(cu_seqlens, tuple) and len(cu_seqlens) == 2:
        host, dev = cu_seqlens
        if (host.device.type != "cpu" or host.dtype != torch.int32 or not host.is_contiguous()
                or not dev.is_cuda or dev.dtype != torch.int32 or not dev.is_contiguous()
                or host.numel() != dev.numel()):
            raise ValueError("cu_seqlens pair must be (host int32, device int32) of equal length")
        return host, dev
    cu = torch.as_tensor(cu_seqlens)
    host = cu.detach().to("cpu", torch.int32).contiguous()
    dev = cu if (cu.is_cuda and cu.dtype == torch.int32 and cu.is_contiguous()) else host.to(device)
    return host, dev


def _thd(x, name):
    if x.dim() == 4:
        if x.shape[0] != 1:
            raise ValueError(f"{name}: packed varlen tensors are (T,H,D) or (1,T,H,D)")
        x = x[0]
    if x.dim() != 3:
        raise ValueError(f"{name}: packed varlen tensors are (T,H,D) or (1,T,H,D)")
    return x


def attn_varlen_fwd(q, k, v, cu_seqlens, scale=None, out=None, lse=None, causal=False):
    """Packed varlen forward: q (T,H,D), k/v (T,Hk,D) bf16 (Hk dividing H: grouped-query
    heads), cu_seqlens int32[nseq+1] -> out (T,H,D), lse (H,T)."""
    torch = _torch()
    q3, k3, v3 = _thd(q, "q"), _thd(k, "k"), _thd(v, "v")
    T, H, D = q3.shape
    Hk = _kv_heads(q3[None], k3[None])
    _want(q3, "q", (T, H, D), torch.bfloat16)
    for t, n in ((k3, "k"), (v3, "v")):
        _want(t, n, (T, Hk, D), torch.bfloat16)
    host, dev = _cu_args(cu_seqlens, q.device)
    nseq = host.numel() - 1
    if nseq < 0 or int(host[-1]) != T:
        raise ValueError(f"cu_seqlens must end at T={T}")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device) if lse is None else lse
    _want(_thd(out, "out"), "out", (T, H, D), torch.bfloat16)
    _want(lse, "lse", (H, T), torch.float32)
    _check("attn_varlen_fwd", lib().attn_varlen_fwd_gqa(nseq, _ptr(host), _ptr(dev), H, Hk, D,
                                                        scale, CAUSAL if causal else 0, _ptr(q3),
                                                        _ptr(k3), _ptr(v3), _ptr(out), _ptr(lse),
                                                        _stream()))
    return out, lse


def attn_varlen_bwd(q, k, v, lse, delta, dout, cu_seqlens, scale=None, dq=None, dk=None, dv=None,
                    causal=False):
    """Packed varlen backward -> dq (T,H,D), dk, dv (T,Hk,D).  delta = attn_bwd_preprocess(out,
    dout)[0]."""
    torch = _torch()
    q3, k3, v3, o3 = _thd(q, "q"), _thd(k, "k"), _thd(v, "v"), _thd(dout, "dout")
    T, H, D = q3.shape
    Hk = _kv_heads(q3[None], k3[None])
    for t, n in ((q3, "q"), (o3, "dout")):
        _want(t, n, (T, H, D), torch.bfloat16)
    for t, n in ((k3, "k"), (v3, "v")):
        _want(t, n, (T, Hk, D), torch.bfloat16)
    if delta.dim() == 3:
        delta = delta[0]
    _want(lse, "lse", (H, T), torch.float32)
    _want(delta, "delta", (H, T), torch.float32)
    host, dev = _cu_args(cu_seqlens, q.device)
    nseq = host.numel() - 1
    if nseq < 0 or int(host[-1]) != T:
        raise ValueError(f"cu_seqlens must end at T={T}")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _want(_thd(dq, "dq"), "dq", (T, H, D), torch.bfloat16)
    for t, n in ((dk, "dk"), (dv, "dv")):
        _want(_thd(t, n), n, (T, Hk, D), torch.bfloat16)
    _check("attn_varlen_bwd", lib().attn_varlen_bwd_gqa(nseq, _ptr(host), _ptr(dev), H, Hk, D,
                                                        scale, CAUSAL if causal else 0, _ptr(q3),
                                                        _ptr(k3), _ptr(v3), _ptr(lse), _ptr(delta),
                                                        _ptr(o3), _ptr(dq), _ptr(dk), _ptr(dv),
                                                        _stream()))
    return dq, dk, dv


MAX_MERGE_CHUNKS = 16


def attn_lse_merge(outs, lses, out=None, lse=None):
    """out, lse = attn_lse_merge([out_c], [lse_c]): merge partial results of disjoint key
    chunks (each out_c (B,S,H,D) bf16 normalised over its chunk, lse_c (B,H,S) fp32).
    out / lse may be one chunk's own tensors (in-place accumulation)."""
    torch = _torch()
    n = len(outs)
    if n != len(lses) or not 1 <= n <= MAX_MERGE_CHUNKS:
        raise ValueError(f"need 1..{MAX_MERGE_CHUNKS} chunks with one lse each, got {n}/{len(lses)}")
    B, S, H, D = outs[0].shape
    for c in range(n):
        _want(outs[c], f"outs[{c}]", (B, S, H, D), torch.bfloat16)
        _want(lses[c], f"lses[{c}]", (B, H, S), torch.float32)
    out = torch.empty_like(outs[0]) if out is None else out
    lse = torch.empty_like(lses[0]) if lse is None else lse
    _want(out, "out", (B, S, H, D), torch.bfloat16)
    _want(lse, "lse", (B, H, S), torch.float32)
    optr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in outs])
    lptr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in lses])
    _check("attn_lse_merge", lib().attn_lse_merge(n, B, S, H, D, optr, lptr, _ptr(out), _ptr(lse),
                                                  _stream()))
    return out, lse


ACC_DQ, ACC_DKDV = 1, 2


def attn_bwd_accum(q, k, v, lse, delta, dout, dq_acc, dk_acc, dv_acc, key_mask=None, scale=None,
                   add_dq=True, add_dkdv=True):
    """One key chunk's dQ, dK, dV into fp32 buffers (q, dout of all rows with the whole key
    set's lse and delta; k, v, key_mask of the chunk): added to the buffers' contents
    (add_dq / add_dkdv) or written over them."""
    torch = _torch()
    B, Sq, Sk, H, D = _dims(q, k)
    _want(q, "q", (B, Sq, H, D), torch.bfloat16)
    _want(k, "k", (B, Sk, H, D), torch.bfloat16)
    _want(v, "v", (B, Sk, H, D), torch.bfloat16)
    _want(dout, "dout", (B, Sq, H, D), torch.bfloat16)
    _want(lse, "lse", (B, H, Sq), torch.float32)
    _want(delta, "delta", (B, H, Sq), torch.float32)
    _want(dq_acc, "dq_acc", (B, Sq, H, D), torch.float32)
    _want(dk_acc, "dk_acc", (B, Sk, H, D), torch.float32)
    _want(dv_acc, "dv_acc", (B, Sk, H, D), torch.float32)
    m = _mask_arg(key_mask, B, Sk, H)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check("attn_bwd_accum", lib().attn_bwd_accum(B, Sq, Sk, H, D, scale, _ptr(q), _ptr(k), _ptr(v),
                                                  _ptr(m), _ptr(lse), _ptr(delta), _ptr(dout),
                                                  _ptr(dq_acc), _ptr(dk_acc), _ptr(dv_acc),
                                                  (ACC_DQ if add_dq else 0) |
                                                  (ACC_DKDV if add_dkdv else 0), _stream()))
    return dq_acc, dk_acc, dv_acc


def attn_cast_bf16(src, dst=None):
    """bf16 copy (nearest even) of an fp32 tensor, e.g. an accumulated gradient."""
    torch = _torch()
    if not isinstance(src, torch.Tensor) or src.dtype != torch.float32:
        raise TypeError("src must be a float32 tensor")
    dst = torch.empty(src.shape, dtype=torch.bfloat16, device=src.device) if dst is None else dst
    _want(src, "src", tuple(src.shape), torch.float32)
    _want(dst, "dst", tuple(src.shape), torch.bfloat16)
    _check("attn_cast_bf16", lib().attn_cast_bf16(src.numel(), _ptr(src), _ptr(dst), _stream()))
    return dst
