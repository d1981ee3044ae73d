"""Pins for the fp64 oracle: each check ties it to something other than itself.

* finite differences of L = sum(dO * out) against the analytic backward;
* invariants the mathematics fixes (softmax rows sum to one, shift invariance
  of softmax -> sum_j dK_j = 0, sum_j dV_j = sum_i dO_i, <Q,dQ> = <K,dK>);
* closed forms (one key, two keys = logistic, zero queries = uniform weights,
  identical keys -> dQ = 0, fully masked rows);
* equivalences (all-ones mask = no mask, masked = sliced, varlen = per-sequence
  dense, key permutation, per-(b,h) independence);
* an independent library implementation (torch CPU fp64 SDPA + autograd);
* the H == S layout probe of diffusers PR #14341 ("Test"): a K/V read with S
  and H swapped must fail the parity bar by a wide margin;
* the gradient magnitudes printed on that page for its two shapes.
"""
import json
import os

import numpy as np
import pytest

import oracle
from attention_flash_attn_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def fwd_bwd(q, k, v, do, mask=None, scale=None):
    out, lse = oracle.attn_fwd(q, k, v, mask, scale)
    delta, dq, dk, dv = oracle.attn_bwd(q, k, v, out, lse, do, mask, scale)
    return out, lse, delta, dq, dk, dv


# ---------------------------------------------------------------- finite differences

@pytest.mark.parametrize("masked", [False, True])
def test_finite_differences(masked):
    B, Sq, Sk, H, D = 2, 3, 5, 2, 4
    q, k, v, do = rnd((B, Sq, H, D), 1), rnd((B, Sk, H, D), 2), rnd((B, Sk, H, D), 3), rnd((B, Sq, H, D), 4)
    mask = None
    if masked:
        mask = np.array([[1, 0, 1, 1, 0], [0, 1, 1, 1, 1]], dtype=np.uint8)
    scale = 0.7

    def loss(q_, k_, v_):
        out, _ = oracle.attn_fwd(q_, k_, v_, mask, scale)
        return float(np.sum(out * do))

    _, _, _, dq, dk, dv = fwd_bwd(q, k, v, do, mask, scale)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.max(np.abs(num - g)) / max(1e-300, np.max(np.abs(g)))
        assert err < 1e-7, (name, err)
    if masked:  # masked keys receive exactly zero gradient
        assert np.all(dk[0, [1, 4]] == 0) and np.all(dv[0, [1, 4]] == 0)
        assert np.all(dk[1, 0] == 0) and np.all(dv[1, 0] == 0)


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("shape,lens", [((2, 37, 3, 16), (29, 37)), ((1, 64, 2, 64), None),
                                        ((3, 20, 4, 128), (1, 7, 20))])
def test_invariants(shape, lens):
    B, S, H, D = shape
    q, k, v, do = (rnd(shape, s) for s in (11, 12, 13, 14))
    mask = None
    if lens is not None:
        mask = np.zeros((B, S), np.uint8)
        for b, n in enumerate(lens):
            mask[b, :n] = 1
    scale = 1 / np.sqrt(D)
    out, lse, delta, dq, dk, dv = fwd_bwd(q, k, v, do, mask)
    keep = np.ones((B, S), bool) if mask is None else mask.astype(bool)
    for b in range(B):
        for h in range(H):
            s = scale * q[b, :, h] @ k[b, :, h].T
            s[:, ~keep[b]] = -np.inf
            P = np.exp(s - lse[b, h][:, None])
            np.testing.assert_allclose(P.sum(1), 1.0, rtol=0, atol=1e-13)
            np.testing.assert_allclose(dv[b, :, h], P.T @ do[b, :, h], rtol=0, atol=1e-12)
            dP = do[b, :, h] @ v[b, :, h].T
            np.testing.assert_allclose(delta[b, h], (P * dP).sum(1), rtol=0, atol=1e-12)
            # softmax is shift invariant in each row -> gradients w.r.t. keys sum to zero
            np.testing.assert_allclose(dk[b, :, h].sum(0), 0.0, rtol=0, atol=1e-12)
            np.testing.assert_allclose(dv[b, :, h].sum(0), do[b, :, h].sum(0), rtol=0, atol=1e-11)
            # s is bilinear in (q, k): <Q, dQ> = <K, dK> = sum dS * s
            a = np.sum(q[b, :, h] * dq[b, :, h])
            c = np.sum(k[b, :, h] * dk[b, :, h])
            assert abs(a - c) < 1e-11 * max(1.0, abs(a))
            assert np.all(dk[b, ~keep[b], h] == 0) and np.all(dv[b, ~keep[b], h] == 0)


# ---------------------------------------------------------------- closed forms

def test_single_key():
    B, Sq, H, D = 2, 7, 3, 16
    q, k, v, do = rnd((B, Sq, H, D), 1), rnd((B, 1, H, D), 2), rnd((B, 1, H, D), 3), rnd((B, Sq, H, D), 4)
    out, lse, _, dq, dk, dv = fwd_bwd(q, k, v, do, scale=0.3)
    np.testing.assert_allclose(out, np.broadcast_to(v, out.shape), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.3 * np.einsum("bshd,bhd->bhs", q, k[:, 0]), rtol=0, atol=1e-13)
    assert np.max(np.abs(dq)) < 1e-14 and np.max(np.abs(dk)) < 1e-13
    np.testing.assert_allclose(dv[:, 0], do.sum(1), rtol=0, atol=1e-13)


def test_two_keys_is_logistic():
    B, Sq, H, D = 1, 9, 2, 8
    q, k, v, do = rnd((B, Sq, H, D), 5), rnd((B, 2, H, D), 6), rnd((B, 2, H, D), 7), rnd((B, Sq, H, D), 8)
    out, lse, *_ = fwd_bwd(q, k, v, do, scale=0.5)
    for h in range(H):
        z = 0.5 * q[0, :, h] @ (k[0, 0, h] - k[0, 1, h])
        w = 1 / (1 + np.exp(-z))
        np.testing.assert_allclose(out[0, :, h], w[:, None] * v[0, 0, h] + (1 - w)[:, None] * v[0, 1, h],
                                   rtol=0, atol=1e-14)
        s1 = 0.5 * q[0, :, h] @ k[0, 1, h]
        np.testing.assert_allclose(lse[0, h], s1 + np.log1p(np.exp(z)), rtol=0, atol=1e-13)


def test_zero_queries_uniform_weights():
    B, S, H, D = 2, 33, 2, 64
    q = np.zeros((B, S, H, D))
    k, v, do = rnd((B, S, H, D), 1), rnd((B, S, H, D), 2), rnd((B, S, H, D), 3)
    mask = np.zeros((B, S), np.uint8)
    mask[0, :20] = 1
    mask[1, :] = 1
    out, lse, *_ = fwd_bwd(q, k, v, do, mask)
    for b, n in ((0, 20), (1, 33)):
        np.testing.assert_allclose(lse[b], np.log(n), rtol=0, atol=1e-15)
        np.testing.assert_allclose(out[b], np.broadcast_to(v[b, :n].mean(0), (S, H, D)), rtol=0, atol=1e-14)


def test_identical_keys_give_zero_dq():
    # every row of dS sums to zero, so dQ_i = scale * sum_j dS_ij * k vanishes when all k_j agree
    B, S, H, D = 1, 25, 2, 32
    q, v, do = rnd((B, S, H, D), 1), rnd((B, S, H, D), 2), rnd((B, S, H, D), 3)
    k = np.broadcast_to(rnd((B, 1, H, D), 4), (B, S, H, D)).copy()
    *_, dq, dk, dv = fwd_bwd(q, k, v, do)
    assert np.max(np.abs(dq)) < 1e-13


def test_fully_masked_rows():
    B, S, H, D = 2, 10, 2, 16
    q, k, v, do = (rnd((B, S, H, D), s) for s in (1, 2, 3, 4))
    mask = np.ones((B, S), np.uint8)
    mask[1] = 0
    out, lse, delta, dq, dk, dv = fwd_bwd(q, k, v, do, mask)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1])) and np.all(delta[1] == 0)
    assert np.all(dq[1] == 0) and np.all(dk[1] == 0) and np.all(dv[1] == 0)
    ref = fwd_bwd(q[:1], k[:1], v[:1], do[:1])
    for a, r in zip((out, lse, delta, dq, dk, dv), ref):
        np.testing.assert_array_equal(a[:1], r)


# ---------------------------------------------------------------- equivalences

def test_all_ones_mask_equals_no_mask():
    shape = (2, 30, 3, 32)
    q, k, v, do = (rnd(shape, s) for s in (1, 2, 3, 4))
    a = fwd_bwd(q, k, v, do)
    b = fwd_bwd(q, k, v, do, np.ones((2, 30), np.uint8))
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_mask_equals_slice():
    B, S, H, D, n = 1, 40, 2, 16, 23
    q, k, v, do = (rnd((B, S, H, D), s) for s in (5, 6, 7, 8))
    mask = np.zeros((B, S), np.uint8)
    mask[0, :n] = 1
    out, lse, delta, dq, dk, dv = fwd_bwd(q, k, v, do, mask)
    o2, l2, d2, dq2, dk2, dv2 = fwd_bwd(q, k[:, :n], v[:, :n], do)
    for a, r in ((out, o2), (lse, l2), (delta, d2), (dq, dq2), (dk[:, :n], dk2), (dv[:, :n], dv2)):
        np.testing.assert_allclose(a, r, rtol=0, atol=1e-13)


def test_key_permutation_invariance():
    B, S, H, D = 1, 31, 2, 16
    q, k, v, do = (rnd((B, S, H, D), s) for s in (9, 10, 11, 12))
    perm = np.random.default_rng(0).permutation(S)
    out, lse, _, dq, dk, dv = fwd_bwd(q, k, v, do)
    o2, l2, _, dq2, dk2, dv2 = fwd_bwd(q, k[:, perm], v[:, perm], do)
    np.testing.assert_allclose(o2, out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dq2, dq, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk2, dk[:, perm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv2, dv[:, perm], rtol=0, atol=1e-13)


def test_slices_are_independent():
    shape = (3, 21, 4, 32)
    q, k, v, do = (rnd(shape, s) for s in (1, 2, 3, 4))
    full = fwd_bwd(q, k, v, do)
    b, h = 2, 1
    sub = fwd_bwd(*(x[b:b + 1, :, h:h + 1] for x in (q, k, v, do)))
    for a, r, kind in zip(full, sub, ("t", "r", "r", "t", "t", "t")):
        a = a[b:b + 1, :, h:h + 1] if kind == "t" else a[b:b + 1, h:h + 1]
        np.testing.assert_array_equal(a, r)


def test_varlen_equals_per_sequence_dense():
    lens = (5, 17, 1, 12)
    H, D = 3, 16
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v, do = (rnd((T, H, D), s) for s in (21, 22, 23, 24))
    out, lse = oracle.attn_varlen_fwd(q, k, v, cu)
    delta, dq, dk, dv = oracle.attn_varlen_bwd(q, k, v, out, lse, do, cu)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        o, l, d, gq, gk, gv = fwd_bwd(*(x[None, a:b] for x in (q, k, v, do)))
        np.testing.assert_allclose(out[a:b], o[0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[:, a:b], l[0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(delta[:, a:b], d[0], rtol=0, atol=1e-14)
        for x, y in ((dq, gq), (dk, gk), (dv, gv)):
            np.testing.assert_allclose(x[a:b], y[0], rtol=0, atol=1e-14)


# ---------------------------------------------------------------- independent library

def _torch_ref(q, k, v, do, mask, scale):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    tq, tk, tv = (torch.tensor(x).permute(0, 2, 1, 3).contiguous().requires_grad_(True) for x in (q, k, v))
    am = None
    if mask is not None:
        am = torch.tensor(mask.astype(bool))[:, None, None, :]
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, scale=scale)
    out.backward(torch.tensor(do).permute(0, 2, 1, 3))
    s = scale * tq.detach() @ tk.detach().transpose(-1, -2)
    if am is not None:
        s = s.masked_fill(~am, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    t = lambda x: x.permute(0, 2, 1, 3).numpy()
    return t(out.detach()), lse.numpy(), t(tq.grad), t(tk.grad), t(tv.grad)


@pytest.mark.parametrize("shape,lens", [((2, 16, 16, 64), None), ((2, 128, 4, 64), None),
                                        ((2, 100, 3, 128), (61, 100))])
def test_against_torch_fp64_sdpa(shape, lens):
    B, S, H, D = shape
    t = I.small_case(B, S, S, H, D, seed=7, valid_lens=lens)
    q, k, v, do = (I.f64_from_bf16_bits(x) for x in (t.q, t.k, t.v, t.do))
    scale = 1 / np.sqrt(D)
    out, lse, _, dq, dk, dv = fwd_bwd(q, k, v, do, t.key_mask)
    r = _torch_ref(q, k, v, do, t.key_mask, scale)
    for name, a, b in zip(("out", "lse", "dq", "dk", "dv"), (out, lse, dq, dk, dv), r):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11, err_msg=name)


# ---------------------------------------------------------------- layout probe + page numbers

def test_hs_layout_probe_fails_parity():
    """K/V read with S and H swapped (the double transpose) must be caught by values, since
    with H == S the shapes still agree (diffusers PR #14341, "Test")."""
    w = I.WORKLOADS["probe_hs16"]
    t = I.draw_workload(w)
    q, k, v, do = (I.f64_from_bf16_bits(x) for x in (t.q, t.k, t.v, t.do))
    out, lse, _, dq, dk, dv = fwd_bwd(q, k, v, do)
    kt, vt = (np.ascontiguousarray(x.transpose(0, 2, 1, 3)) for x in (k, v))
    _, dq2, dk2, dv2 = oracle.attn_bwd(q, kt, vt, out, lse, do)
    page = json.load(open(os.path.join(GOLDEN, "page_reported_errors.json")))["probe_hs16"]
    for a, b, bug in zip((dq, dk, dv), (dq2, dk2, dv2), page["double_transposed_kv_max_abs_error_dq_dk_dv"]):
        err = np.max(np.abs(a - b))
        assert err > 50 * 2e-2 and err > 0.25 * np.max(np.abs(a))
        assert bug / 5 < err < bug * 5  # same order as the page's buggy-path errors


def test_magnitudes_match_page():
    page = json.load(open(os.path.join(GOLDEN, "page_reported_errors.json")))
    for key, seeds in (("probe_hs16", range(1, 7)), ("dit_s1024", (2,))):
        w = I.WORKLOADS[key]
        mags = []
        for seed in seeds:
            t = I.draw_workload(w, seed)
            q, k, v, do = (I.f64_from_bf16_bits(x) for x in (t.q, t.k, t.v, t.do))
            *_, dq, dk, dv = fwd_bwd(q, k, v, do)
            mags.append([np.max(np.abs(x)) for x in (dq, dk, dv)])
        mags = np.mean(mags, axis=0)
        ref = np.array(page[key]["reference_max_magnitude_dq_dk_dv"])
        assert np.all(mags > ref / 2) and np.all(mags < ref * 2), (key, mags, ref)


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(3).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 65504.0]  # ties and a large value
    ours = I.bf16_bits_from_f32(x)
    ref = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
