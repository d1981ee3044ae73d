"""Full-tensor GPU parity on the large named workloads: every element of out, LSE, dQ, dK
and dV of the 27280-token Wan shard (B=1 N=27280 H=10 D=128) and of the packed varlen batch
(lengths 4096, 7000, 1234, 15000; H=24 D=128) against the fp64 oracle, in the launch
configuration the benchmark times.  The page's own test compares all three gradients of
the whole problem against a higher-precision reference (diffusers PR #14341, "Test").

Each workload runs once on the GPU (module fixture, results copied to the host); the oracle
then goes head by head (one test per head, so every test ends within seconds and host
memory stays bounded).  The bar is applied per head, which is at least as strict as over
the whole tensor (a head's max |oracle| is at most the tensor's).

The grouped-query and causal variants of the Wan shard are compared in full for out, LSE
and dQ (every query head), and on sampled key columns for dK/dV (a dK/dV column of the
grouped-query shard gathers five query heads' rows; its oracle cost is the same per column).
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


def run_dense(A, t, causal=False):
    """fwd -> preprocess -> bwd on the device (outputs pre-filled with NaN, so an unwritten
    element fails), results moved to host memory."""
    import torch
    q, k, v, do = (to_dev(x) for x in (t.q, t.k, t.v, t.do))
    nan = float("nan")
    B, Sq, H, _ = q.shape
    out, lse = A.attn_fwd(q, k, v, None, out=torch.full_like(q, nan),
                          lse=torch.full((B, H, Sq), nan, device="cuda"), causal=causal)
    delta = A.attn_bwd_preprocess(out, do)
    dq, dk, dv = (torch.full_like(x, nan) for x in (q, k, v))
    A.attn_bwd(q, k, v, lse, delta, do, None, dq=dq, dk=dk, dv=dv, causal=causal)
    torch.cuda.synchronize()
    res = {n: x.cpu() for n, x in (("out", out), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}
    del q, k, v, do, out, lse, delta, dq, dk, dv
    torch.cuda.empty_cache()
    return res


# Per-head oracle forwards (out, lse) of the grouped-query and causal shards, kept for the
# sampled-column tests that need every row's out and LSE: the oracle treats each (batch,
# head) alone, so a head's forward is the same arithmetic wherever it is computed.
_FWD = {}


def oracle_fwd_head(name, t, h, kh=None, causal=False):
    if (name, h) not in _FWD:
        q, k, v, _ = head(t, h, kh)
        _FWD[(name, h)] = oracle.attn_fwd(q, k, v, causal=causal)
    return _FWD[(name, h)]


def head(t, h, kh=None):
    kh = h if kh is None else kh
    return (f64(t.q[:, :, h:h + 1]), f64(t.k[:, :, kh:kh + 1]), f64(t.v[:, :, kh:kh + 1]),
            f64(t.do[:, :, h:h + 1]))


# ---------------------------------------------------------------- Wan shard, every element

@pytest.fixture(scope="module")
def wan(A):
    w = I.WORKLOADS["wan_shard"]
    t = I.draw_workload(w)
    return w, t, run_dense(A, t)


@pytest.mark.parametrize("h", range(10))
def test_wan_shard_full_head(wan, h):
    """Head h of the Wan shard, every element of out, LSE, dQ, dK, dV.  Head 9's rows
    15616.. are the forward's split tail workgroups and its last dQ tiles the backward's
    split dQ workgroups (in the grid of a 256-CU device)."""
    w, t, g = wan
    q, k, v, do = head(t, h)
    out, lse = oracle.attn_fwd(q, k, v)
    _, dq, dk, dv = oracle.attn_bwd(q, k, v, out, lse, do)
    sl = slice(h, h + 1)
    assert_parity(f"out[h{h}]", to_f64(g["out"][:, :, sl]), out)
    assert_lse(to_f64(g["lse"][:, sl]), lse)
    for n, r in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_parity(f"{n}[h{h}]", to_f64(g[n][:, :, sl]), r)


# ---------------------------------------------------------------- varlen4, every element

@pytest.fixture(scope="module")
def varlen4(A):
    import torch
    w = I.WORKLOADS["varlen4"]
    t = I.draw_workload(w)
    H, T = w.H, w.T
    q, k, v, do = (to_dev(x[0]) for x in (t.q, t.k, t.v, t.do))
    nan = float("nan")
    out, lse = A.attn_varlen_fwd(q, k, v, t.cu_seqlens, out=torch.full_like(q, nan),
                                 lse=torch.full((H, T), nan, device="cuda"))
    delta = A.attn_bwd_preprocess(out, do)
    dq, dk, dv = (torch.full_like(x, nan) for x in (q, k, v))
    A.attn_varlen_bwd(q, k, v, lse, delta, do, t.cu_seqlens, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    g = {n: x.cpu() for n, x in (("out", out), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}
    del q, k, v, do, out, lse, delta, dq, dk, dv
    torch.cuda.empty_cache()
    return w, t, g


@pytest.mark.parametrize("h", range(24))
def test_varlen4_full_head(varlen4, h):
    """Head h of the packed batch, every sequence, every element (the oracle's varlen
    calls apply the definition to each sequence alone)."""
    w, t, g = varlen4
    cu = t.cu_seqlens
    q, k, v, do = (f64(x[0, :, h:h + 1]) for x in (t.q, t.k, t.v, t.do))
    out, lse = oracle.attn_varlen_fwd(q, k, v, cu)
    _, dq, dk, dv = oracle.attn_varlen_bwd(q, k, v, out, lse, do, cu)
    sl = slice(h, h + 1)
    assert_parity(f"out[h{h}]", to_f64(g["out"][:, sl]), out)
    assert_lse(to_f64(g["lse"][sl]), lse)
    for n, r in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_parity(f"{n}[h{h}]", to_f64(g[n][:, sl]), r)


# ---------------------------------------------------------------- grouped-query Wan shard

@pytest.fixture(scope="module")
def wan_gqa(A):
    w = I.WORKLOADS["wan_shard_gqa"]
    t = I.draw_workload(w)
    return w, t, run_dense(A, t)


@pytest.mark.parametrize("h", range(10))
def test_wan_shard_gqa_rows_full_head(wan_gqa, h):
    """Query head h (key/value head h // 5): every element of out, LSE and dQ."""
    w, t, g = wan_gqa
    G = w.H // w.Hk
    q, k, v, do = head(t, h, h // G)
    out, lse = oracle_fwd_head(w.name, t, h, h // G)
    _, dq, _, _ = oracle.attn_bwd(q, k, v, out, lse, do, want_dkdv=False)
    sl = slice(h, h + 1)
    assert_parity(f"out[h{h}]", to_f64(g["out"][:, :, sl]), out)
    assert_lse(to_f64(g["lse"][:, sl]), lse)
    assert_parity(f"dq[h{h}]", to_f64(g["dq"][:, :, sl]), dq)


@pytest.mark.parametrize("kv_head", [0, 1])
def test_wan_shard_gqa_sampled_key_columns(wan_gqa, kv_head):
    """dK, dV of sampled key columns of each key/value head: each column sums every row
    of the group's five query heads (grouped-query oracle over the whole group)."""
    w, t, g = wan_gqa
    G, S = w.H // w.Hk, w.S
    rng = np.random.default_rng(40 + kv_head)
    cols = np.unique(np.concatenate([[0, 255, 256, S - 1], rng.integers(0, S, 20)]))
    heads = slice(kv_head * G, (kv_head + 1) * G)
    q, do = f64(t.q[:, :, heads]), f64(t.do[:, :, heads])
    k, v = f64(t.k[:, :, kv_head:kv_head + 1]), f64(t.v[:, :, kv_head:kv_head + 1])
    # the group's forward, head by head (as attn_fwd_gqa computes it)
    fw = [oracle_fwd_head(w.name, t, h, kv_head) for h in range(heads.start, heads.stop)]
    out = np.concatenate([o for o, _ in fw], axis=2)
    lse = np.concatenate([l for _, l in fw], axis=1)
    _, _, dk, dv = oracle.attn_bwd_gqa(q, k[:, cols], v[:, cols], out, lse, do)
    sl = slice(kv_head, kv_head + 1)
    assert_parity(f"dk[kv{kv_head}]", to_f64(g["dk"][:, cols, sl]), dk)
    assert_parity(f"dv[kv{kv_head}]", to_f64(g["dv"][:, cols, sl]), dv)


# ---------------------------------------------------------------- causal Wan shard

@pytest.fixture(scope="module")
def wan_causal(A):
    w = I.WORKLOADS["wan_shard_causal"]
    t = I.draw_workload(w)
    return w, t, run_dense(A, t, causal=True)


@pytest.mark.parametrize("h", range(10))
def test_wan_shard_causal_rows_full_head(wan_causal, h):
    """Head h of the causal shard: every element of out, LSE and dQ (row i is attention
    over keys 0..i)."""
    w, t, g = wan_causal
    q, k, v, do = head(t, h)
    out, lse = oracle_fwd_head(w.name, t, h, causal=True)
    _, dq, _, _ = oracle.attn_bwd(q, k, v, out, lse, do, want_dkdv=False, causal=True)
    sl = slice(h, h + 1)
    assert_parity(f"out[h{h}]", to_f64(g["out"][:, :, sl]), out)
    assert_lse(to_f64(g["lse"][:, sl]), lse)
    assert_parity(f"dq[h{h}]", to_f64(g["dq"][:, :, sl]), dq)


@pytest.mark.parametrize("h", [0, 4, 9])
def test_wan_shard_causal_sampled_key_columns(wan_causal, h):
    """dK, dV of sampled key columns: column j gathers the rows i >= j, with every row's
    LSE and out from the full causal forward."""
    w, t, g = wan_causal
    S = w.S
    rng = np.random.default_rng(50 + h)
    cols = np.unique(np.concatenate([[0, 1, 63, 64, 255, 256, S - 2, S - 1],
                                     rng.integers(0, S, 16)]))
    q, k, v, do = head(t, h)
    out, lse = oracle_fwd_head(w.name, t, h, causal=True)
    rdk, rdv = [], []
    for j in cols:
        _, _, dk, dv = oracle.attn_bwd(q[:, j:], k[:, j:j + 1], v[:, j:j + 1], out[:, j:],
                                       lse[:, :, j:], do[:, j:], want_dq=False)
        rdk.append(dk)
        rdv.append(dv)
    sl = slice(h, h + 1)
    assert_parity(f"dk[h{h}]", to_f64(g["dk"][:, cols, sl]), np.concatenate(rdk, axis=1))
    assert_parity(f"dv[h{h}]", to_f64(g["dv"][:, cols, sl]), np.concatenate(rdv, axis=1))
