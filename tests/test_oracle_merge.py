"""Pins for the oracle's chunk merge and the chunked backward (ring / context-parallel
attention, the backward diffusers PR #14834 names as missing in its description).

Each check ties the merge to something other than itself:
* the full forward over all keys (a different function of the oracle) equals the merge of
  the forwards over disjoint key chunks, with and without a mask, for ragged splits;
* closed forms written out by hand: one chunk is the identity, two chunks with equal LSE
  average their outputs and add ln 2 to the LSE, a chunk with LSE = -inf adds nothing,
  all chunks empty give out = 0 and LSE = -inf;
* the backward of each chunk with the whole key set's LSE and delta sums (dQ) or
  concatenates (dK, dV) to the full backward.
"""
import numpy as np
import pytest

import oracle


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


SPLITS = {
    1: [(0, 11)],
    2: [(0, 5), (5, 11)],
    3: [(0, 3), (3, 9), (9, 11)],
    4: [(0, 1), (1, 4), (4, 10), (10, 11)],
}


def chunk_forwards(q, k, v, mask, bounds, scale=None):
    outs, lses = [], []
    for a, b in bounds:
        m = None if mask is None else mask[:, a:b]
        o, l = oracle.attn_fwd(q, k[:, a:b], v[:, a:b], m, scale)
        outs.append(o)
        lses.append(l)
    return outs, lses


@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("masked", [False, True])
def test_merge_equals_full_forward(n, masked):
    B, Sq, Sk, H, D = 2, 7, 11, 3, 8
    q, k, v = rnd((B, Sq, H, D), 11), rnd((B, Sk, H, D), 12), rnd((B, Sk, H, D), 13)
    mask = None
    if masked:
        mask = np.ones((B, Sk), dtype=np.uint8)
        mask[0, 6:] = 0
        mask[1, :2] = 0
    out, lse = oracle.attn_fwd(q, k, v, mask, 0.4)
    outs, lses = chunk_forwards(q, k, v, mask, SPLITS[n], 0.4)
    mo, ml = oracle.attn_lse_merge(outs, lses)
    assert np.max(np.abs(mo - out)) < 1e-12
    assert np.max(np.abs(ml - lse)) < 1e-12


def test_merge_closed_forms():
    B, S, H, D = 1, 4, 2, 3
    o1, o2 = rnd((B, S, H, D), 21), rnd((B, S, H, D), 22)
    l1 = rnd((B, H, S), 23)
    # one chunk: identity
    mo, ml = oracle.attn_lse_merge([o1], [l1])
    assert np.array_equal(mo, o1) and np.array_equal(ml, l1)
    # two chunks of equal mass: mean of the outputs, LSE + ln 2
    mo, ml = oracle.attn_lse_merge([o1, o2], [l1, l1.copy()])
    assert np.max(np.abs(mo - 0.5 * (o1 + o2))) < 1e-15
    assert np.max(np.abs(ml - (l1 + np.log(2.0)))) < 1e-15
    # mass ratio 1 : 3 -> weights 1/4, 3/4
    mo, ml = oracle.attn_lse_merge([o1, o2], [l1, l1 + np.log(3.0)])
    assert np.max(np.abs(mo - (0.25 * o1 + 0.75 * o2))) < 1e-14
    assert np.max(np.abs(ml - (l1 + np.log(4.0)))) < 1e-14
    # a chunk with no keys (LSE = -inf, out = 0) adds nothing
    ninf = np.full_like(l1, -np.inf)
    mo, ml = oracle.attn_lse_merge([o1, np.zeros_like(o2)], [l1, ninf])
    assert np.array_equal(mo, o1) and np.array_equal(ml, l1)
    # no keys anywhere: out = 0, LSE = -inf
    mo, ml = oracle.attn_lse_merge([np.zeros_like(o1), np.zeros_like(o2)], [ninf, ninf])
    assert np.array_equal(mo, np.zeros_like(o1)) and np.all(np.isneginf(ml))


def test_merge_with_fully_masked_chunk():
    B, Sq, Sk, H, D = 2, 5, 9, 2, 8
    q, k, v = rnd((B, Sq, H, D), 31), rnd((B, Sk, H, D), 32), rnd((B, Sk, H, D), 33)
    mask = np.ones((B, Sk), dtype=np.uint8)
    mask[:, 3:6] = 0  # the middle chunk has no key to attend to
    bounds = [(0, 3), (3, 6), (6, 9)]
    outs, lses = chunk_forwards(q, k, v, mask, bounds)
    assert np.all(np.isneginf(lses[1])) and not np.any(outs[1])
    mo, ml = oracle.attn_lse_merge(outs, lses)
    out, lse = oracle.attn_fwd(q, k, v, mask)
    assert np.max(np.abs(mo - out)) < 1e-12 and np.max(np.abs(ml - lse)) < 1e-12


@pytest.mark.parametrize("masked", [False, True])
def test_chunked_backward_equals_full(masked):
    B, Sq, Sk, H, D = 2, 6, 10, 2, 8
    q, k, v, do = (rnd((B, Sq, H, D), 41), rnd((B, Sk, H, D), 42), rnd((B, Sk, H, D), 43),
                   rnd((B, Sq, H, D), 44))
    mask = None
    if masked:
        mask = np.ones((B, Sk), dtype=np.uint8)
        mask[0, 7:] = 0
    out, lse = oracle.attn_fwd(q, k, v, mask)
    _, dq, dk, dv = oracle.attn_bwd(q, k, v, out, lse, do, mask)
    dq_sum = np.zeros_like(dq)
    dks, dvs = [], []
    bounds = [(0, 4), (4, 7), (7, 10)]
    for a, b in bounds:
        m = None if mask is None else mask[:, a:b]
        _, dq_c, dk_c, dv_c = oracle.attn_bwd(q, k[:, a:b], v[:, a:b], out, lse, do, m)
        dq_sum += dq_c
        dks.append(dk_c)
        dvs.append(dv_c)
    assert np.max(np.abs(dq_sum - dq)) < 1e-12
    assert np.max(np.abs(np.concatenate(dks, axis=1) - dk)) < 1e-12
    assert np.max(np.abs(np.concatenate(dvs, axis=1) - dv)) < 1e-12
