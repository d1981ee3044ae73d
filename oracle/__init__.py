"""fp64 CPU oracle for attention forward/backward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never touches it.

Thin ctypes wrapper over ``attn_oracle.c`` (plain C, fp64, OpenMP).  All arrays
are float64 numpy arrays in BSHD (dense) or packed THD (varlen) layout; LSE and
delta are (B, H, Sq) or (H, T).  See ``attn_oracle.c`` for the definition each
function follows.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_dp = ctypes.POINTER(ctypes.c_double)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i32p = ctypes.POINTER(ctypes.c_int32)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    i, d = ctypes.c_int, ctypes.c_double
    lib.oracle_attn_fwd.argtypes = [i, i, i, i, i, d, _dp, _dp, _dp, _u8p, _dp, _dp]
    lib.oracle_attn_fwd_ex.argtypes = [i, i, i, i, i, d, _dp, _dp, _dp, _u8p, _dp, _dp, i]
    lib.oracle_attn_delta.argtypes = [i, i, i, i, _dp, _dp, _dp]
    lib.oracle_attn_bwd.argtypes = [i, i, i, i, i, d, _dp, _dp, _dp, _u8p, _dp, _dp, _dp, _dp,
                                    _dp, _dp, _dp]
    lib.oracle_attn_bwd_ex.argtypes = lib.oracle_attn_bwd.argtypes + [i]
    lib.oracle_set_num_threads.argtypes = [i]
    lib.oracle_attn_lse_merge.argtypes = [i, i, i, i, i, ctypes.POINTER(_dp), ctypes.POINTER(_dp),
                                          _dp, _dp]
    lib.oracle_attn_varlen_fwd.argtypes = [i, _i32p, i, i, d, _dp, _dp, _dp, _dp, _dp]
    lib.oracle_attn_varlen_fwd_ex.argtypes = [i, _i32p, i, i, d, _dp, _dp, _dp, _dp, _dp, i]
    lib.oracle_attn_varlen_bwd.argtypes = [i, _i32p, i, i, d, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                           _dp, _dp, _dp]
    lib.oracle_attn_varlen_bwd_ex.argtypes = lib.oracle_attn_varlen_bwd.argtypes + [i]
    for f in ("oracle_attn_fwd", "oracle_attn_delta", "oracle_attn_bwd", "oracle_attn_varlen_fwd",
              "oracle_attn_varlen_bwd", "oracle_num_threads", "oracle_set_num_threads",
              "oracle_attn_lse_merge", "oracle_attn_fwd_ex", "oracle_attn_bwd_ex",
              "oracle_attn_varlen_fwd_ex", "oracle_attn_varlen_bwd_ex"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> int:
    """Threads for the following calls (OpenMP); returns the count now in effect."""
    return _load().oracle_set_num_threads(int(n))


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _m(mask):
    if mask is None:
        return None
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    return mask


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle rejected arguments (code {rc})")


def attn_fwd(q, k, v, key_mask=None, scale=None, causal=False):
    """q (B,Sq,H,D), k/v (B,Sk,H,D) -> out (B,Sq,H,D), lse (B,H,Sq); causal: query i sees
    keys j <= i only."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    assert k.shape == (B, Sk, H, D) and v.shape == k.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    mask = _m(key_mask)
    if mask is not None:
        assert mask.shape == (B, Sk)
    out = np.empty_like(q)
    lse = np.empty((B, H, Sq), dtype=np.float64)
    _check(_load().oracle_attn_fwd_ex(B, Sq, Sk, H, D, scale, _p(q), _p(k), _p(v),
                                      None if mask is None else mask.ctypes.data_as(_u8p), _p(out),
                                      _p(lse), int(causal)))
    return out, lse


def attn_delta(out, dout):
    """delta[b,h,i] = <dO[b,i,h,:], out[b,i,h,:]> -> (B,H,S)."""
    out, dout = _f64(out), _f64(dout)
    B, S, H, D = out.shape
    delta = np.empty((B, H, S), dtype=np.float64)
    _check(_load().oracle_attn_delta(B, S, H, D, _p(out), _p(dout), _p(delta)))
    return delta


def attn_bwd(q, k, v, out, lse, dout, key_mask=None, scale=None, want_dq=True, want_dkdv=True,
             causal=False):
    """Return (delta, dq, dk, dv); dq or dk/dv are None when not requested.

    ``out`` and ``lse`` must come from :func:`attn_fwd` on the same inputs (or,
    for key-column sampling, from the full forward while k/v are a key subset).
    """
    q, k, v, out, lse, dout = map(_f64, (q, k, v, out, lse, dout))
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    mask = _m(key_mask)
    delta = np.empty((B, H, Sq), dtype=np.float64)
    dq = np.empty_like(q) if want_dq else None
    dk = np.empty_like(k) if want_dkdv else None
    dv = np.empty_like(v) if want_dkdv else None
    _check(_load().oracle_attn_bwd_ex(B, Sq, Sk, H, D, scale, _p(q), _p(k), _p(v),
                                      None if mask is None else mask.ctypes.data_as(_u8p), _p(out),
                                      _p(lse), _p(dout), _p(delta), _p(dq), _p(dk), _p(dv),
                                      int(causal)))
    return delta, dq, dk, dv


def attn_varlen_fwd(q, k, v, cu_seqlens, scale=None, causal=False):
    """Packed q/k/v (T,H,D) (a leading batch dim of 1 is accepted) -> out (T,H,D), lse (H,T)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    shp = q.shape
    T, H, D = shp[-3:]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    assert cu[-1] == T
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.empty_like(q)
    lse = np.empty((H, T), dtype=np.float64)
    _check(_load().oracle_attn_varlen_fwd_ex(len(cu) - 1, cu.ctypes.data_as(_i32p), H, D, scale,
                                             _p(q), _p(k), _p(v), _p(out), _p(lse), int(causal)))
    return out, lse


def attn_varlen_bwd(q, k, v, out, lse, dout, cu_seqlens, scale=None, causal=False):
    """-> (delta (H,T), dq, dk, dv) for packed inputs."""
    q, k, v, out, lse, dout = map(_f64, (q, k, v, out, lse, dout))
    T, H, D = q.shape[-3:]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    delta = np.empty((H, T), dtype=np.float64)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    _check(_load().oracle_attn_varlen_bwd_ex(len(cu) - 1, cu.ctypes.data_as(_i32p), H, D, scale,
                                             _p(q), _p(k), _p(v), _p(out), _p(lse), _p(dout),
                                             _p(delta), _p(dq), _p(dk), _p(dv), int(causal)))
    return delta, dq, dk, dv


def attn_lse_merge(outs, lses):
    """Merge partial results of disjoint key chunks: outs[c] (B,S,H,D), lses[c] (B,H,S)
    -> (out, lse) of attention over all the chunks' keys."""
    outs = [_f64(o) for o in outs]
    lses = [_f64(l) for l in lses]
    n = len(outs)
    assert n >= 1 and len(lses) == n
    B, S, H, D = outs[0].shape
    for o, l in zip(outs, lses):
        assert o.shape == (B, S, H, D) and l.shape == (B, H, S)
    out = np.empty_like(outs[0])
    lse = np.empty_like(lses[0])
    op = (_dp * n)(*[_p(o) for o in outs])
    lp = (_dp * n)(*[_p(l) for l in lses])
    _check(_load().oracle_attn_lse_merge(n, B, S, H, D, op, lp, _p(out), _p(lse)))
    return out, lse


# ---------------------------------------------------------------- grouped-query attention
#
# GQA (diffusers PR #14834 names it as not extended; the cuDNN / flash messages quoted in
# diffusers PR #14341, reporter's tables, state the constraint that the key/value head count
# divides the query head count).  Query head h reads key/value head h // G, G = H / Hk.
# Written out as its definition: attention with each key/value head repeated over its
# group of G query heads; the gradient of a repeated tensor is the sum of the gradients of
# its copies (chain rule), so dK, dV of head g sum the G expanded heads' dK, dV.


def _gqa_group(H, Hk):
    assert Hk >= 1 and H % Hk == 0, (H, Hk)
    return H // Hk


def attn_fwd_gqa(q, k, v, key_mask=None, scale=None, causal=False):
    """q (B,Sq,H,D), k/v (B,Sk,Hk,D) -> out (B,Sq,H,D), lse (B,H,Sq)."""
    G = _gqa_group(q.shape[2], k.shape[2])
    return attn_fwd(q, np.repeat(_f64(k), G, axis=2), np.repeat(_f64(v), G, axis=2), key_mask, scale,
                    causal)


def attn_bwd_gqa(q, k, v, out, lse, dout, key_mask=None, scale=None, causal=False):
    """-> (delta, dq (B,Sq,H,D), dk, dv (B,Sk,Hk,D))."""
    B, Sk, Hk, D = k.shape
    G = _gqa_group(q.shape[2], Hk)
    delta, dq, dke, dve = attn_bwd(q, np.repeat(_f64(k), G, axis=2), np.repeat(_f64(v), G, axis=2),
                                   out, lse, dout, key_mask, scale, causal=causal)
    return (delta, dq, dke.reshape(B, Sk, Hk, G, D).sum(axis=3),
            dve.reshape(B, Sk, Hk, G, D).sum(axis=3))
