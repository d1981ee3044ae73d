"""GPU parity of grouped-query attention (query head h reads key/value head h // G,
G = H / Hk; named as not yet extended in diffusers PR #14834, description) through the C
ABI against the fp64 oracle's grouped-query definition on the same seeded bf16 inputs."""
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


def gpu(A, t):
    import torch
    q, k, v, do = (to_dev(x) for x in (t.q, t.k, t.v, t.do))
    m = None if t.key_mask is None else torch.from_numpy(t.key_mask).cuda()
    nan = float("nan")
    B, Sq, H, _ = q.shape
    out, lse = A.attn_fwd(q, k, v, m, out=torch.full_like(q, nan),
                          lse=torch.full((B, H, Sq), nan, device="cuda"))
    delta = A.attn_bwd_preprocess(out, do)
    dq, dk, dv = (torch.full_like(x, nan) for x in (q, k, v))
    A.attn_bwd(q, k, v, lse, delta, do, m, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return dict(out=out, lse=lse, dq=dq, dk=dk, dv=dv)


CASES = [
    # (B, Sq, Sk, H, Hk, D, valid_lens)
    (2, 300, 300, 8, 2, 128, None),
    (1, 200, 333, 6, 3, 64, None),
    (2, 257, 257, 4, 1, 128, (64, 200)),   # one key/value head (multi-query)
    (1, 129, 129, 12, 4, 64, None),
    (2, 130, 70, 10, 5, 128, (70, 1)),     # G = 2, Sq > Sk, a single valid key
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Sq{}_Sk{}_H{}_Hk{}_D{}_m{}".format(*c))
def test_gqa_small(A, case):
    B, Sq, Sk, H, Hk, D, lens = case
    t = I.small_case(B, Sq, Sk, H, D, seed=400 + Sq + H + Hk, valid_lens=lens, Hk=Hk)
    g = gpu(A, t)
    q, k, v, do = (f64(x) for x in (t.q, t.k, t.v, t.do))
    out, lse = oracle.attn_fwd_gqa(q, k, v, t.key_mask)
    _, dq, dk, dv = oracle.attn_bwd_gqa(q, k, v, out, lse, do, t.key_mask)
    assert_parity("out", to_f64(g["out"]), out, True)
    assert_lse(to_f64(g["lse"]), lse)
    for n, r in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_parity(n, to_f64(g[n]), r, True)
    if t.key_mask is not None:
        off = t.key_mask == 0
        for n in ("dk", "dv"):
            assert np.all(to_f64(g[n])[off] == 0.0), f"{n} of masked keys must be exactly 0"


def test_gqa_forward_equals_mha_on_repeated_kv(A):
    """Same arithmetic on the same data: out, LSE and dQ bit for bit."""
    import torch
    t = I.small_case(2, 333, 333, 8, 128, seed=91, Hk=2)
    g = gpu(A, t)
    rep = lambda x: np.repeat(x, 4, axis=2)
    m = gpu(A, I.Tensors(t.q, rep(t.k), rep(t.v), t.do, None, None))
    for n in ("out", "lse", "dq"):
        assert torch.equal(g[n], m[n]), n


def _sampled(A, t, H, Hk, rows, cols, kv_head):
    g = gpu(A, t)
    G = H // Hk
    q, k, v, do = (f64(x) for x in (t.q, t.k, t.v, t.do))
    heads = list(range(kv_head * G, (kv_head + 1) * G))
    kq, vq = k[:, :, kv_head:kv_head + 1], v[:, :, kv_head:kv_head + 1]
    # out, LSE, dQ of sampled rows of the group's first query head
    h = heads[0]
    o_r, l_r = oracle.attn_fwd(q[:, rows, h:h + 1], kq, vq)
    assert_parity("out", to_f64(g["out"][:, rows, h:h + 1]), o_r)
    assert_lse(to_f64(g["lse"][:, h:h + 1][:, :, rows]), l_r)
    _, dq_r, _, _ = oracle.attn_bwd(q[:, rows, h:h + 1], kq, vq, o_r, l_r, do[:, rows, h:h + 1],
                                    want_dkdv=False)
    assert_parity("dq", to_f64(g["dq"][:, rows, h:h + 1]), dq_r)
    # dK, dV of sampled key columns of the key/value head: every row of its G query heads
    qg, dog = q[:, :, heads], do[:, :, heads]
    out_g, lse_g = oracle.attn_fwd_gqa(qg, kq, vq)
    _, _, dk_r, dv_r = oracle.attn_bwd_gqa(qg, kq[:, cols], vq[:, cols], out_g, lse_g, dog)
    assert_parity("dk", to_f64(g["dk"][:, cols, kv_head:kv_head + 1]), dk_r)
    assert_parity("dv", to_f64(g["dv"][:, cols, kv_head:kv_head + 1]), dv_r)


def test_gqa_s8192_sampled(A):
    S, H, Hk = 8192, 8, 2
    t = I.small_case(1, S, S, H, 128, seed=92, Hk=Hk)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, S - 1], rng.integers(0, S, 24)]))
    cols = np.unique(np.concatenate([[0, S - 1], rng.integers(0, S, 24)]))
    _sampled(A, t, H, Hk, rows, cols, kv_head=1)


@pytest.mark.parametrize("D,causal", [(64, False), (128, False), (128, True)],
                         ids=["D64", "D128", "D128_causal"])
def test_varlen_gqa(A, D, causal):
    """Packed sequences with grouped-query heads (H = 8, Hk = 2): every sequence against
    the oracle's grouped-query attention over that sequence alone (causal inside it).  The
    short sequences make dK/dV sums over few rows of four heads, up to ~4 in magnitude, so
    the bar carries the bf16 quantisation slack of the synthetic cases (tests/parity.py)."""
    import torch
    lens = (5, 130, 1, 64, 300, 0, 77, 257)
    H, Hk = 8, 2
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    t = I.small_case(1, T, T, H, D, seed=700 + D + int(causal), Hk=Hk)
    q, k, v, do = (to_dev(x[0]) for x in (t.q, t.k, t.v, t.do))
    nan = float("nan")
    out, lse = A.attn_varlen_fwd(q, k, v, cu, out=torch.full_like(q, nan),
                                 lse=torch.full((H, T), nan, device="cuda"), causal=causal)
    delta = A.attn_bwd_preprocess(out, do)
    dq, dk, dv = (torch.full_like(x, nan) for x in (q, k, v))
    A.attn_varlen_bwd(q, k, v, lse, delta, do, cu, dq=dq, dk=dk, dv=dv, causal=causal)
    torch.cuda.synchronize()
    qf, kf, vf, dof = (f64(x) for x in (t.q, t.k, t.v, t.do))
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        if a == b:
            continue
        qs, ks, vs, ds = (x[:, a:b] for x in (qf, kf, vf, dof))
        ro, rl = oracle.attn_fwd_gqa(qs, ks, vs, None, causal=causal)
        _, rdq, rdk, rdv = oracle.attn_bwd_gqa(qs, ks, vs, ro, rl, ds, None, causal=causal)
        assert_parity(f"out[seq{n}]", to_f64(out[a:b])[None], ro, True)
        assert_lse(to_f64(lse[:, a:b])[None], rl)
        for nm, x, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            assert_parity(f"{nm}[seq{n}]", to_f64(x[a:b])[None], r, True)
