"""The fwd -> delta -> bwd step captured as one HIP graph and replayed (what `bench.py
--graph` times): every replay must give the eager results bit for bit.  The step's calls
take every output buffer from the caller and record no memset, so a replay is the same
three kernels on the same buffers.  Replays alternate with eager work on the same buffers
(NaN fills, and an eager step on other inputs), with a synchronization before each check.
"""
import pytest

from attention_flash_attn_amd import inputs as I
from parity import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_flash_attn_amd as A
    A.lib()  # raise loudly if the HIP library is missing
    return A


@pytest.mark.parametrize("B,S,H,D,lens", [(1, 300, 2, 128, None), (2, 1024, 3, 64, None),
                                         (2, 520, 2, 128, [400, 520])])
def test_graph_replay_matches_eager(A, B, S, H, D, lens):
    import torch
    t = I.small_case(B, S, S, H, D, seed=900 + S + D, valid_lens=lens)
    o = I.small_case(B, S, S, H, D, seed=901 + S + D, valid_lens=lens)  # other inputs
    q, k, v, do = (to_dev(x) for x in (t.q, t.k, t.v, t.do))
    q2, k2, v2, do2 = (to_dev(x) for x in (o.q, o.k, o.v, o.do))
    m = None if t.key_mask is None else torch.from_numpy(t.key_mask).cuda()
    out, dq, dk, dv = (torch.empty_like(x) for x in (q, q, k, v))
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    delta = torch.empty_like(lse)
    bufs = (out, lse, delta, dq, dk, dv)

    def step(q, k, v, do):
        A.attn_fwd(q, k, v, m, None, out=out, lse=lse)
        A.attn_bwd_preprocess(out, do, delta=delta)
        A.attn_bwd(q, k, v, lse, delta, do, m, None, dq=dq, dk=dk, dv=dv)

    step(q, k, v, do)
    torch.cuda.synchronize()
    ref = [x.clone() for x in bufs]

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(q, k, v, do)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step(q, k, v, do)
    for r in range(3):
        for x in bufs:
            x.fill_(float("nan"))
        if r == 1:
            step(q2, k2, v2, do2)  # eager work on other inputs between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("out", "lse", "delta", "dq", "dk", "dv"), bufs, ref):
            assert torch.equal(x, y), f"replay {r}: {name} differs from the eager step"
