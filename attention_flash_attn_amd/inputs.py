"""Seeded synthetic inputs for attention forward/backward.

This module only draws numbers and builds index metadata; it holds none of the
attention arithmetic.  Both the fp64 oracle and the GPU path are fed from here.

Recipe (the pages publish no seeds or tensors, so this is a stated choice):
  * ``numpy.random.default_rng(seed)``; q, k, v, dO drawn in that order as full
    BSHD (or packed THD) float32 tensors with ``standard_normal``, then rounded
    to bfloat16 with round-to-nearest-even.  The oracle upcasts the very same
    bf16 values exactly to fp64.
  * Key-padding masks are prefixes: key j of batch b is attended iff
    ``j < valid_len[b]`` (byte 1 = attend, 0 = masked).
  * Varlen batches are packed in the listed order; ``cu_seqlens`` is int32.

The workloads below carry the shapes the pages discuss: the H == S layout probe
and the H != S shape from the K/V double-transpose fix (diffusers PR #14341,
"Test" and reporter's tables), a masked long-sequence case, the per-rank shard
of the Wan attention layer timed in LightX2V PR #1234 ("Performance" table:
N=27280, 40 heads over 4 sequence-parallel ranks, D=128), and a packed varlen
batch (the FA3-varlen path named in diffusers PR #14834, "Model test coverage").
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r = r.copy()
        r[nan] = 0x7FC0
    return r


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f64_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return f32_from_bf16_bits(b).astype(np.float64)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention problem.  Dense problems are BSHD; varlen ones are packed THD (B=1)."""

    name: str
    B: int
    S: int  # Sq == Sk for every named workload
    H: int
    D: int
    valid_lens: Optional[Sequence[int]] = None  # per-batch key prefix lengths (mask)
    seqlens: Optional[Sequence[int]] = None  # varlen sequence lengths (packed)
    seed: int = 0
    Hk: Optional[int] = None  # key/value heads (grouped-query attention); None = H
    causal: bool = False  # query i sees keys j <= i only

    @property
    def kv_heads(self) -> int:
        return self.H if self.Hk is None else self.Hk

    @property
    def varlen(self) -> bool:
        return self.seqlens is not None

    @property
    def T(self) -> int:
        return int(sum(self.seqlens)) if self.varlen else self.B * self.S

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def shape(self):
        return (1, self.T, self.H, self.D) if self.varlen else (self.B, self.S, self.H, self.D)

    @property
    def kv_shape(self):
        return self.shape[:2] + (self.kv_heads, self.D)

    def cu_seqlens(self) -> Optional[np.ndarray]:
        if not self.varlen:
            return None
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    def key_mask(self) -> Optional[np.ndarray]:
        if self.valid_lens is None:
            return None
        m = np.zeros((self.B, self.S), dtype=np.uint8)
        for b, n in enumerate(self.valid_lens):
            m[b, :n] = 1
        return m

    def fwd_flops(self) -> float:
        """Algorithmic forward FLOPs: 4*H*D per (query, key) pair attended, over (b | sequence):
        Sq*Sk pairs (dense count for masks), or S(S+1)/2 when causal."""
        pairs = (lambda n: n * (n + 1) // 2) if self.causal else (lambda n: n * n)
        if self.varlen:
            return 4.0 * self.H * self.D * float(sum(pairs(int(n)) for n in self.seqlens))
        return 4.0 * self.B * self.H * self.D * float(pairs(self.S))

    def fwd_bwd_flops(self) -> float:
        return 3.5 * self.fwd_flops()


# The five named workloads; the seed of each is its ordinal.
WORKLOADS = {
    "probe_hs16": Workload("probe_hs16", B=2, S=16, H=16, D=64, seed=1),
    "dit_s1024": Workload("dit_s1024", B=2, S=1024, H=24, D=64, seed=2),
    "mask_s4096": Workload("mask_s4096", B=2, S=4096, H=24, D=128, valid_lens=(3001, 4096), seed=3),
    "wan_shard": Workload("wan_shard", B=1, S=27280, H=10, D=128, seed=4),
    "varlen4": Workload("varlen4", B=1, S=27330, H=24, D=128, seqlens=(4096, 7000, 1234, 15000), seed=5),
    # Grouped-query attention (named as not yet extended in diffusers PR #14834, description;
    # the pages give no GQA workload): the Wan shard's query heads over 2 key/value heads.
    "wan_shard_gqa": Workload("wan_shard_gqa", B=1, S=27280, H=10, D=128, seed=6, Hk=2),
    # Causal attention (also named as not yet extended there; the pages give no causal
    # workload): the Wan shard's shape with query i seeing keys 0..i.
    "wan_shard_causal": Workload("wan_shard_causal", B=1, S=27280, H=10, D=128, seed=7, causal=True),
}


@dataclasses.dataclass
class Tensors:
    """bf16 bit patterns (uint16) of q, k, v, dO in BSHD/THD, plus metadata."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    key_mask: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]


def draw(shape, seed: int, key_mask=None, cu_seqlens=None, kv_shape=None) -> Tensors:
    """Draw q, k, v, dO i.i.d. N(0,1) (in that order) and round each to bf16; k and v take
    kv_shape when given (fewer key/value heads)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(4):
        shp = kv_shape if (kv_shape is not None and i in (1, 2)) else shape
        out.append(bf16_bits_from_f32(rng.standard_normal(shp, dtype=np.float32)))
    return Tensors(out[0], out[1], out[2], out[3], key_mask, cu_seqlens)


def draw_workload(w: Workload, seed: Optional[int] = None) -> Tensors:
    return draw(w.shape, w.seed if seed is None else seed, w.key_mask(), w.cu_seqlens(),
                w.kv_shape if w.Hk is not None else None)


def small_case(B, Sq, Sk, H, D, seed, valid_lens=None, Hk=None):
    """Dense inputs with Sq != Sk allowed: q/dO get Sq rows, k/v get Sk rows (and Hk heads
    when given).

    Draw order is still q, k, v, dO."""
    rng = np.random.default_rng(seed)
    Hk = H if Hk is None else Hk
    q = bf16_bits_from_f32(rng.standard_normal((B, Sq, H, D), dtype=np.float32))
    k = bf16_bits_from_f32(rng.standard_normal((B, Sk, Hk, D), dtype=np.float32))
    v = bf16_bits_from_f32(rng.standard_normal((B, Sk, Hk, D), dtype=np.float32))
    do = bf16_bits_from_f32(rng.standard_normal((B, Sq, H, D), dtype=np.float32))
    mask = None
    if valid_lens is not None:
        mask = np.zeros((B, Sk), dtype=np.uint8)
        for b, n in enumerate(valid_lens):
            mask[b, :n] = 1
    return Tensors(q, k, v, do, mask, None)
