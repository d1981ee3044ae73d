"""GPU parity of the ring / context-parallel pieces (the backward diffusers PR #14834
names as missing in its description): per-chunk forwards merged by attn_lse_merge and
the per-chunk accumulating backward attn_bwd_accum (+ attn_cast_bf16), all through the C
ABI, against the fp64 oracle of attention over ALL keys on the same seeded bf16 inputs.

The chunked path rounds each chunk's output to bf16 before the merge, so its outputs
carry one more bf16 rounding than the one-launch path; the parity bar is the same.
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


def gpu_chunked(A, t, bounds, scale=None, inplace=False):
    """Forward per key chunk -> merge -> delta -> accumulating backward per chunk -> bf16."""
    import torch
    q, k, v, do = (to_dev(x) for x in (t.q, t.k, t.v, t.do))
    m = None if t.key_mask is None else torch.from_numpy(t.key_mask).cuda()
    chunks = []
    for a, b in bounds:
        mc = None if m is None else m[:, a:b].contiguous()
        chunks.append((k[:, a:b].contiguous(), v[:, a:b].contiguous(), mc))
    outs, lses = [], []
    for kc, vc, mc in chunks:
        o, l = A.attn_fwd(q, kc, vc, mc, scale)
        outs.append(o)
        lses.append(l)
    parts = ([o.clone() for o in outs], [l.clone() for l in lses])
    if inplace:
        out, lse = A.attn_lse_merge(outs, lses, out=outs[0], lse=lses[0])
    else:
        out, lse = A.attn_lse_merge(outs, lses)
    delta = A.attn_bwd_preprocess(out, do)
    # NaN-filled buffers: the first chunk must overwrite dq_acc, every chunk its dk/dv_acc
    dq_acc = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    dks, dvs = [], []
    for c, (kc, vc, mc) in enumerate(chunks):
        dk_acc = torch.full(kc.shape, float("nan"), dtype=torch.float32, device="cuda")
        dv_acc = torch.full(vc.shape, float("nan"), dtype=torch.float32, device="cuda")
        A.attn_bwd_accum(q, kc, vc, lse, delta, do, dq_acc, dk_acc, dv_acc, mc, scale,
                         add_dq=c > 0, add_dkdv=False)
        dks.append(A.attn_cast_bf16(dk_acc))
        dvs.append(A.attn_cast_bf16(dv_acc))
    dq = A.attn_cast_bf16(dq_acc)
    torch.cuda.synchronize()
    g = dict(out=out, lse=lse, delta=delta, dq=dq, dk=torch.cat(dks, 1), dv=torch.cat(dvs, 1))
    return g, parts


def oracle_dense(t, scale=None):
    q, k, v, do = (f64(x) for x in (t.q, t.k, t.v, t.do))
    out, lse = oracle.attn_fwd(q, k, v, t.key_mask, scale)
    delta, dq, dk, dv = oracle.attn_bwd(q, k, v, out, lse, do, t.key_mask, scale)
    return dict(out=out, lse=lse, delta=delta, dq=dq, dk=dk, dv=dv)


def check(g, r, t):
    assert_parity("out", to_f64(g["out"]), r["out"], True)
    assert_lse(to_f64(g["lse"]), r["lse"])
    for n in ("dq", "dk", "dv"):
        assert_parity(n, to_f64(g[n]), r[n], True)
    if t.key_mask is not None:
        off = t.key_mask == 0
        for n in ("dk", "dv"):
            assert np.all(to_f64(g[n])[off] == 0.0), f"{n} of masked keys must be exactly 0"


CASES = [
    # (B, S, H, D, valid_lens, chunk bounds over the keys)
    (2, 300, 3, 128, None, [(0, 100), (100, 250), (250, 300)]),
    (2, 300, 2, 64, (120, 300), [(0, 64), (64, 200), (200, 300)]),  # batch 0: last chunk empty
    (1, 257, 2, 128, None, [(0, 1), (1, 128), (128, 129), (129, 257)]),  # one-key chunks
    (2, 200, 2, 128, (150, 37), [(0, 200)]),  # a single chunk
    (1, 96, 1, 64, None, [(i, i + 6) for i in range(0, 96, 6)]),  # 16 chunks, the maximum
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_S{}_H{}_D{}_m{}_n{}".format(*c[:5], len(c[5])))
def test_chunked_path_matches_oracle(A, case):
    B, S, H, D, lens, bounds = case
    t = I.small_case(B, S, S, H, D, seed=300 + S + D + len(bounds), valid_lens=lens)
    g, _ = gpu_chunked(A, t, bounds)
    check(g, oracle_dense(t), t)


def test_merge_in_place_is_bitwise_equal(A):
    import torch
    t = I.small_case(2, 333, 333, 2, 128, seed=77, valid_lens=(333, 200))
    bounds = [(0, 111), (111, 222), (222, 333)]
    g1, _ = gpu_chunked(A, t, bounds)
    g2, _ = gpu_chunked(A, t, bounds, inplace=True)
    for n in g1:
        assert torch.equal(g1[n], g2[n]), n


def test_merge_kernel_vs_oracle_merge(A):
    """Same partial inputs (the GPU's bf16 chunk outputs, fp32 LSEs) into both merges: only
    fp32 arithmetic and the final bf16 rounding (half an ulp, 2^-9 relative) may differ."""
    t = I.small_case(2, 250, 250, 3, 64, seed=78, valid_lens=(90, 250))
    bounds = [(0, 80), (80, 100), (100, 250)]  # batch 0: keys 90.. masked, last chunk empty
    g, (outs, lses) = gpu_chunked(A, t, bounds)
    ro, rl = oracle.attn_lse_merge([to_f64(o) for o in outs], [to_f64(l) for l in lses])
    go, gl = to_f64(g["out"]), to_f64(g["lse"])
    assert np.all(np.abs(go - ro) <= 2.0 ** -8 * np.abs(ro) + 1e-6), np.max(np.abs(go - ro))
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    fin = ~np.isneginf(rl)
    assert np.max(np.abs(gl[fin] - rl[fin])) < 1e-5


def test_merge_of_empty_chunks(A):
    import torch
    t = I.small_case(1, 64, 64, 2, 128, seed=79, valid_lens=(0,))
    g, _ = gpu_chunked(A, t, [(0, 32), (32, 64)])
    assert torch.all(g["out"] == 0) and torch.all(torch.isneginf(g["lse"]))
    for n in ("dq", "dk", "dv"):
        assert torch.all(g[n] == 0), n


def test_bwd_accum_adds_when_asked(A):
    """add_dkdv / add_dq: a second call on the same buffers doubles them; rounded with
    attn_cast_bf16 the fp32 results equal the one-launch backward's bf16 outputs bit for
    bit (same arithmetic, one rounding)."""
    import torch
    t = I.small_case(1, 200, 150, 2, 128, seed=81)
    q, k, v, do = (to_dev(x) for x in (t.q, t.k, t.v, t.do))
    out, lse = A.attn_fwd(q, k, v)
    delta = A.attn_bwd_preprocess(out, do)
    acc = [torch.empty(x.shape, dtype=torch.float32, device="cuda") for x in (q, k, v)]
    A.attn_bwd_accum(q, k, v, lse, delta, do, *acc, add_dq=False, add_dkdv=False)
    once = [a.clone() for a in acc]
    A.attn_bwd_accum(q, k, v, lse, delta, do, *acc, add_dq=True, add_dkdv=True)
    for a, o in zip(acc, once):
        assert torch.equal(a, 2 * o)  # x + x is exact in fp32
    dq, dk, dv = A.attn_bwd(q, k, v, lse, delta, do)
    torch.cuda.synchronize()
    for a, b in zip(once, (dq, dk, dv)):
        assert torch.equal(A.attn_cast_bf16(a), b)  # same arithmetic, same rounding


@pytest.mark.parametrize("n", [1, 7, 2048, 2049, 100003])
def test_cast_rounds_to_nearest_even(A, n):
    import torch
    x = np.random.default_rng(n).standard_normal(n).astype(np.float32) * 3.0
    x[: min(n, 4)] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0][: min(n, 4)]
    ref = I.bf16_bits_from_f32(x)  # RNE on the host
    got = A.attn_cast_bf16(torch.from_numpy(x).cuda()).cpu().view(torch.int16).numpy()
    assert np.array_equal(got, ref.view(np.int16))


def test_wan_shard_in_four_chunks(A):
    """The 27280-token shard with its keys in 4 ring chunks: sampled query rows and key
    columns of one head against the oracle over all keys."""
    w = I.WORKLOADS["wan_shard"]
    t = I.draw_workload(w)
    S = w.S
    bounds = [(i * S // 4, (i + 1) * S // 4) for i in range(4)]
    g, _ = gpu_chunked(A, t, bounds)
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([[0, S // 4 - 1, S // 4, S - 1], rng.integers(0, S, 20)]))
    cols = np.unique(np.concatenate([[0, S // 4 - 1, S // 4, S - 1], rng.integers(0, S, 20)]))
    h = 3
    q, k, v, do = (f64(x[:, :, h:h + 1]) for x in (t.q, t.k, t.v, t.do))
    gh = {n: to_f64(g[n][:, :, h:h + 1]) for n in ("out", "dq", "dk", "dv")}
    o_r, l_r = oracle.attn_fwd(q[:, rows], k, v)
    assert_parity("out", gh["out"][:, rows], o_r)
    assert_lse(to_f64(g["lse"][:, h:h + 1])[:, :, rows], l_r)
    _, dq_r, _, _ = oracle.attn_bwd(q[:, rows], k, v, o_r, l_r, do[:, rows], want_dkdv=False)
    assert_parity("dq", gh["dq"][:, rows], dq_r)
    out_full, lse_full = oracle.attn_fwd(q, k, v)
    _, _, dk_r, dv_r = oracle.attn_bwd(q, k[:, cols], v[:, cols], out_full, lse_full, do,
                                       want_dq=False)
    assert_parity("dk", gh["dk"][:, cols], dk_r)
    assert_parity("dv", gh["dv"][:, cols], dv_r)
