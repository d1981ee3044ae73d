"""GPU parity of causal attention (query i sees keys j <= i, top-left aligned when Sq != Sk,
per sequence in varlen; named as not yet extended in diffusers PR #14834, description)
through the C ABI against the fp64 oracle's causal mode on the same seeded bf16 inputs.

The kernels skip key tiles past a workgroup's last query row and mask per element only on
the tiles that cross the diagonal, so the cases put the diagonal inside and across tiles
(64-key forward/dQ tiles, 256-key dK/dV blocks, 128/256-row query tiles), with ragged
tails, Sq != Sk both ways, key masks (rows whose visible keys are all masked get out = 0,
LSE = -inf), grouped-query heads and packed sequences.
"""
import numpy as np
import pytest

import oracle
from attention_flash_attn_amd import inputs as I
from parity import assert_lse, assert_parity, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_flash_attn_amd as A
    A.lib()  # raise loudly if the HIP library is missing
    return A


def f64(bits):
    return I.f64_from_bf16_bits(bits)


def gpu(A, t, causal=True):
    import torch
    q, k, v, do = (to_dev(x) for x in (t.q, t.k, t.v, t.do))
    m = None if t.key_mask is None else torch.from_numpy(t.key_mask).cuda()
    nan = float("nan")
    B, Sq, H, _ = q.shape
    out, lse = A.attn_fwd(q, k, v, m, out=torch.full_like(q, nan),
                          lse=torch.full((B, H, Sq), nan, device="cuda"), causal=causal)
    delta = A.attn_bwd_preprocess(out, do)
    dq, dk, dv = (torch.full_like(x, nan) for x in (q, k, v))
    A.attn_bwd(q, k, v, lse, delta, do, m, dq=dq, dk=dk, dv=dv, causal=causal)
    torch.cuda.synchronize()
    return dict(out=out, lse=lse, dq=dq, dk=dk, dv=dv)


def check(g, t, H, Hk):
    q, k, v, do = (f64(x) for x in (t.q, t.k, t.v, t.do))
    if Hk == H:
        out, lse = oracle.attn_fwd(q, k, v, t.key_mask, causal=True)
        _, dq, dk, dv = oracle.attn_bwd(q, k, v, out, lse, do, t.key_mask, causal=True)
    else:
        out, lse = oracle.attn_fwd_gqa(q, k, v, t.key_mask, causal=True)
        _, dq, dk, dv = oracle.attn_bwd_gqa(q, k, v, out, lse, do, t.key_mask, causal=True)
    assert_parity("out", to_f64(g["out"]), out, True)
    assert_lse(to_f64(g["lse"]), lse)
    for n, r in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_parity(n, to_f64(g[n]), r, True)
    if t.key_mask is not None:
        off = t.key_mask == 0
        for n in ("dk", "dv"):
            assert np.all(to_f64(g[n])[off] == 0.0), f"{n} of masked keys must be exactly 0"
    # keys that no query row sees (Sq < Sk: keys Sq..Sk-1) get exactly zero gradients
    Sq, Sk = q.shape[1], k.shape[1]
    if Sq < Sk:
        for n in ("dk", "dv"):
            assert np.all(to_f64(g[n])[:, Sq:] == 0.0), f"{n} of unseen keys must be exactly 0"


CASES = [
    # (B, Sq, Sk, H, Hk, D, valid_lens)
    (2, 300, 300, 3, 3, 128, None),
    (1, 513, 513, 2, 2, 64, None),
    (2, 200, 333, 2, 2, 128, (333, 150)),   # Sq < Sk: keys 200.. seen by no row
    (1, 333, 200, 2, 2, 64, None),          # Sq > Sk: rows 199.. see every key
    (2, 257, 257, 8, 2, 128, (64, 257)),    # grouped-query heads (G = 4)
    (1, 130, 130, 10, 5, 64, None),
    (1, 1, 1, 2, 2, 128, None),
    (1, 64, 64, 2, 2, 128, None),           # one tile, the diagonal inside it
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Sq{}_Sk{}_H{}_Hk{}_D{}_m{}".format(*c))
def test_causal_small(A, case):
    B, Sq, Sk, H, Hk, D, lens = case
    t = I.small_case(B, Sq, Sk, H, D, seed=500 + Sq + Sk + H + D, valid_lens=lens, Hk=Hk)
    check(gpu(A, t), t, H, Hk)


def test_causal_rows_with_no_visible_key(A):
    """Keys 0..69 masked: rows 0..69 see no key (out 0, LSE -inf), rows 70.. see 70..i."""
    B, S, H, D = 1, 300, 2, 128
    t = I.small_case(B, S, S, H, D, seed=531)
    mask = np.ones((B, S), dtype=np.uint8)
    mask[:, :70] = 0
    t = I.Tensors(t.q, t.k, t.v, t.do, mask, None)
    g = gpu(A, t)
    check(g, t, H, H)
    assert np.all(np.isneginf(to_f64(g["lse"])[:, :, :70]))
    for n in ("out", "dq"):
        assert np.all(to_f64(g[n])[:, :70] == 0.0), n


def test_causal_last_row_equals_full_attention(A):
    """The last row of a square causal problem sees every key: its output, LSE and dQ are
    those of the non-causal call, within the parity bar of each (different tile paths)."""
    t = I.small_case(1, 400, 400, 2, 128, seed=532)
    c, n = gpu(A, t), gpu(A, t, causal=False)
    for name in ("out", "dq"):
        assert_parity(name, to_f64(c[name][:, -1:]), to_f64(n[name][:, -1:]))
    assert_lse(to_f64(c["lse"][:, :, -1:]), to_f64(n["lse"][:, :, -1:]))


@pytest.mark.parametrize("D", [64, 128])
def test_causal_varlen(A, D):
    import torch
    lens = (5, 130, 1, 64, 300, 0, 77, 257)
    H = 2
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    t = I.draw((T, H, D), seed=540 + D, cu_seqlens=cu)
    q, k, v, do = (to_dev(x) for x in (t.q, t.k, t.v, t.do))
    nan = float("nan")
    out, lse = A.attn_varlen_fwd(q, k, v, cu, out=torch.full_like(q, nan),
                                 lse=torch.full((H, T), nan, device="cuda"), causal=True)
    delta = A.attn_bwd_preprocess(out, do)
    dq, dk, dv = (torch.full_like(x, nan) for x in (q, k, v))
    A.attn_varlen_bwd(q, k, v, lse, delta, do, cu, dq=dq, dk=dk, dv=dv, causal=True)
    torch.cuda.synchronize()
    qf, kf, vf, dof = (f64(x) for x in (t.q, t.k, t.v, t.do))
    ro, rl = oracle.attn_varlen_fwd(qf, kf, vf, cu, causal=True)
    _, rdq, rdk, rdv = oracle.attn_varlen_bwd(qf, kf, vf, ro, rl, dof, cu, causal=True)
    assert_parity("out", to_f64(out), ro)
    assert_lse(to_f64(lse), rl)
    for n, a, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        assert_parity(n, to_f64(a), r)
    # each sequence equals the dense causal call on it alone, bit for bit
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        if b == a:
            continue
        sub = I.Tensors(*(x[None, a:b] for x in (t.q, t.k, t.v, t.do)), None, None)
        d = gpu(A, sub)
        for name, x in (("out", out), ("dq", dq), ("dk", dk), ("dv", dv)):
            assert torch.equal(d[name][0], x[a:b]), (n, name)
