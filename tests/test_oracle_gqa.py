"""Pins for the oracle's grouped-query attention (query head h reads key/value head
h // G, G = H / Hk; named as not yet extended in diffusers PR #14834, description).

* central differences of L = sum(dO * out) with respect to q, k, v (k and v with Hk heads)
  against the oracle's backward, which sums the gradients of each key/value head's copies;
* torch CPU fp64 scaled_dot_product_attention with enable_gqa=True plus autograd, an
  independent implementation of the same grouping;
* G = 1 is plain multi-head attention.
"""
import numpy as np
import pytest

import oracle
from attention_flash_attn_amd import inputs as I


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("masked", [False, True])
def test_gqa_finite_differences(masked):
    B, Sq, Sk, H, Hk, D = 1, 3, 4, 4, 2, 4
    q, k, v, do = rnd((B, Sq, H, D), 1), rnd((B, Sk, Hk, D), 2), rnd((B, Sk, Hk, D), 3), rnd((B, Sq, H, D), 4)
    mask = np.array([[1, 0, 1, 1]], dtype=np.uint8) if masked else None
    scale = 0.6

    def loss(q_, k_, v_):
        out, _ = oracle.attn_fwd_gqa(q_, k_, v_, mask, scale)
        return float(np.sum(out * do))

    out, lse = oracle.attn_fwd_gqa(q, k, v, mask, scale)
    _, dq, dk, dv = oracle.attn_bwd_gqa(q, k, v, out, lse, do, mask, scale)
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
    if masked:  # the masked key gets no gradient
        assert not np.any(dk[:, 1]) and not np.any(dv[:, 1])


@pytest.mark.parametrize("shape", [(2, 40, 8, 2, 64), (1, 33, 6, 3, 32), (2, 17, 4, 1, 16)])
def test_gqa_against_torch_fp64_sdpa(shape):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    B, S, H, Hk, D = shape
    t = I.small_case(B, S, S, H, D, seed=17, valid_lens=(S - 5,) + (S,) * (B - 1), Hk=Hk)
    q, k, v, do = (I.f64_from_bf16_bits(x) for x in (t.q, t.k, t.v, t.do))
    scale = 1 / np.sqrt(D)
    out, lse = oracle.attn_fwd_gqa(q, k, v, t.key_mask, scale)
    _, dq, dk, dv = oracle.attn_bwd_gqa(q, k, v, out, lse, do, t.key_mask, scale)
    tq, tk, tv = (torch.tensor(x).permute(0, 2, 1, 3).contiguous().requires_grad_(True) for x in (q, k, v))
    am = torch.tensor(t.key_mask.astype(bool))[:, None, None, :]
    tout = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, scale=scale, enable_gqa=True)
    tout.backward(torch.tensor(do).permute(0, 2, 1, 3))
    tt = lambda x: x.permute(0, 2, 1, 3).detach().numpy()
    for name, a, b in (("out", out, tt(tout)), ("dq", dq, tt(tq.grad)), ("dk", dk, tt(tk.grad)),
                       ("dv", dv, tt(tv.grad))):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11, err_msg=name)


def test_gqa_with_one_group_is_mha():
    B, Sq, Sk, H, D = 2, 9, 7, 3, 8
    q, k, v, do = rnd((B, Sq, H, D), 5), rnd((B, Sk, H, D), 6), rnd((B, Sk, H, D), 7), rnd((B, Sq, H, D), 8)
    o1, l1 = oracle.attn_fwd_gqa(q, k, v)
    o2, l2 = oracle.attn_fwd(q, k, v)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    g1 = oracle.attn_bwd_gqa(q, k, v, o1, l1, do)
    g2 = oracle.attn_bwd(q, k, v, o2, l2, do)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)
