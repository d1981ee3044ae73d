"""Shared helpers for the GPU parity tests: moving seeded inputs to the device and
the parity bar.

Bar (per output tensor, over every compared element):
  max|gpu - oracle| <= 2e-2  and  <= 1% of max|oracle|;  LSE: max|gpu - oracle| <= 1e-3.
-inf LSE entries (rows with no key to attend to) must match exactly.

The named workloads (N(0,1) inputs, outputs below ~3 in magnitude) are held to that bar
as is.  Synthetic edge cases can produce outputs far larger (one valid key makes dV a sum
of every dO row); a bf16 output of magnitude m is itself only exact to 2^-8 * m, which
exceeds 2e-2 once m > 5, so for those cases the absolute part becomes
2e-2 + 2^-8 * |oracle| per element (``quant_slack=True``).  The 1%-of-max part is kept.

The absolute 2e-2 was set for the named workloads' softmax scale 1/sqrt(D), where the
gradients stay below ~1.2.  A larger scale makes rows peakier and the gradients larger
(scale 0.3 at D = 64: max |dQ| ~ 5), and the backward's delta, formed from the stored bf16
out as the method prescribes, then differs from the oracle's (fp64 out) by up to
sum_d |dO_d| 2^-9 |out_d| ~ 0.05, which moves dQ_i by scale * that * |(P K)_i| ~ 0.05 on its
own.  Such synthetic-scale cases are held to the scale-free part of the bar, 1% of
max|oracle| (``rel_only=True``), LSE unchanged.

A tensor the oracle gives as identically zero is a gradient that cancels exactly (a
query row that sees a single key has P = 1 and dP = delta, so its dS is 0 and so is the
dK it feeds).  1% of its max would demand an exact zero from fp32 arithmetic that
subtracts two O(10) sums rounded in different orders; there the bound is that
rounding, ZERO_REF_TOL = 1e-5 (the cancelled terms carry ~2^-24 relative error each).
"""
from __future__ import annotations

import numpy as np

ABS_TOL = 2e-2
REL_OF_MAX = 0.01
LSE_TOL = 1e-3
ZERO_REF_TOL = 1e-5


def to_dev(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_f64(t):
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy().astype(np.float64)


def max_err(gpu, ref):
    return float(np.max(np.abs(gpu - ref))) if ref.size else 0.0


def assert_parity(name, gpu, ref, quant_slack=False, rel_only=False):
    """rel_only: only the 1%-of-max part of the bar (see the module docstring on scales)."""
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    if ref.size == 0:
        return
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite values"
    err = max_err(gpu, ref)
    mx = float(np.max(np.abs(ref)))
    if rel_only:
        pass
    elif quant_slack:
        excess = float(np.max(np.abs(gpu - ref) - (ABS_TOL + 2.0 ** -8 * np.abs(ref))))
        assert excess <= 0, f"{name}: error exceeds 2e-2 + 2^-8|ref| by {excess:.3e}"
    else:
        assert err <= ABS_TOL, f"{name}: max abs err {err:.3e} > {ABS_TOL}"
    if mx == 0.0:
        assert err <= ZERO_REF_TOL, f"{name}: oracle is identically 0, max |gpu| {err:.3e}"
        return
    assert err <= REL_OF_MAX * mx, f"{name}: max abs err {err:.3e} > 1% of max |ref| {mx:.3e}"


def assert_lse(gpu, ref):
    assert gpu.shape == ref.shape
    inf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(gpu), inf), "LSE: -inf pattern differs"
    if (~inf).any():
        err = float(np.max(np.abs(gpu[~inf] - ref[~inf])))
        assert err <= LSE_TOL, f"LSE: max abs err {err:.3e} > {LSE_TOL}"
