"""Pins for the oracle's causal mode (query i sees keys j <= i, top-left aligned when
Sq != Sk; named as not extended in diffusers PR #14834, description, defined on no page).

* central differences of L = sum(dO * out) against the causal backward, with and without
  a key mask, Sq == Sk and Sq != Sk;
* torch CPU fp64 scaled_dot_product_attention with the causal (and key) mask as an explicit
  boolean mask, plus autograd, and logsumexp for the LSE;
* the prefix identity: causal row i equals plain attention of q_i over keys 0..i;
* varlen causal equals per-sequence dense causal calls.
"""
import numpy as np
import pytest

import oracle
from attention_flash_attn_amd import inputs as I


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("Sq,Sk,masked", [(4, 4, False), (4, 4, True), (3, 5, False), (5, 3, True)])
def test_causal_finite_differences(Sq, Sk, masked):
    B, H, D = 1, 2, 4
    q, k, v, do = rnd((B, Sq, H, D), 1), rnd((B, Sk, H, D), 2), rnd((B, Sk, H, D), 3), rnd((B, Sq, H, D), 4)
    mask = None
    if masked:
        mask = np.ones((B, Sk), dtype=np.uint8)
        mask[0, 1] = 0
    scale = 0.7

    def loss(q_, k_, v_):
        out, _ = oracle.attn_fwd(q_, k_, v_, mask, scale, causal=True)
        return float(np.sum(out * do))

    out, lse = oracle.attn_fwd(q, k, v, mask, scale, causal=True)
    _, dq, dk, dv = oracle.attn_bwd(q, k, v, out, lse, do, mask, scale, causal=True)
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
        assert np.max(np.abs(num - g)) < 1e-7 * max(1.0, np.max(np.abs(g))), name


@pytest.mark.parametrize("Sq,Sk", [(33, 33), (20, 37), (37, 20)])
def test_causal_against_torch_fp64(Sq, Sk):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    B, H, D = 2, 3, 16
    t = I.small_case(B, Sq, Sk, H, D, seed=23, valid_lens=(Sk, Sk - 3))
    q, k, v, do = (I.f64_from_bf16_bits(x) for x in (t.q, t.k, t.v, t.do))
    scale = 1 / np.sqrt(D)
    out, lse = oracle.attn_fwd(q, k, v, t.key_mask, scale, causal=True)
    _, dq, dk, dv = oracle.attn_bwd(q, k, v, out, lse, do, t.key_mask, scale, causal=True)
    tq, tk, tv = (torch.tensor(x).permute(0, 2, 1, 3).contiguous().requires_grad_(True) for x in (q, k, v))
    allowed = torch.ones(Sq, Sk, dtype=torch.bool).tril()[None, None] & \
        torch.tensor(t.key_mask.astype(bool))[:, None, None, :]
    tout = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=allowed, scale=scale)
    tout.backward(torch.tensor(do).permute(0, 2, 1, 3))
    s = (scale * tq.detach() @ tk.detach().transpose(-1, -2)).masked_fill(~allowed, float("-inf"))
    tl = torch.logsumexp(s, dim=-1).numpy()
    tt = lambda x: x.permute(0, 2, 1, 3).detach().numpy()
    for name, a, b in (("out", out, tt(tout)), ("lse", lse, tl), ("dq", dq, tt(tq.grad)),
                       ("dk", dk, tt(tk.grad)), ("dv", dv, tt(tv.grad))):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11, err_msg=name)


def test_causal_rows_are_prefix_attention():
    B, S, H, D = 2, 9, 2, 8
    q, k, v = rnd((B, S, H, D), 5), rnd((B, S, H, D), 6), rnd((B, S, H, D), 7)
    out, lse = oracle.attn_fwd(q, k, v, causal=True)
    for i in range(S):
        o_i, l_i = oracle.attn_fwd(q[:, i:i + 1], k[:, :i + 1], v[:, :i + 1])
        assert np.max(np.abs(out[:, i:i + 1] - o_i)) < 1e-14
        assert np.max(np.abs(lse[:, :, i:i + 1] - l_i)) < 1e-14


def test_varlen_causal_equals_dense_per_sequence():
    H, D = 2, 8
    lens = [5, 1, 8]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v, do = (rnd((T, H, D), s) for s in (8, 9, 10, 11))
    out, lse = oracle.attn_varlen_fwd(q, k, v, cu, causal=True)
    _, dq, dk, dv = oracle.attn_varlen_bwd(q, k, v, out, lse, do, cu, causal=True)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        sl = lambda x: x[None, a:b]
        o, l = oracle.attn_fwd(sl(q), sl(k), sl(v), causal=True)
        _, gq, gk, gv = oracle.attn_bwd(sl(q), sl(k), sl(v), o, l, sl(do), causal=True)
        assert np.max(np.abs(out[a:b] - o[0])) < 1e-14 and np.max(np.abs(lse[:, a:b] - l[0])) < 1e-14
        for x, y in ((dq, gq), (dk, gk), (dv, gv)):
            assert np.max(np.abs(x[a:b] - y[0])) < 1e-14
