"""Register budget of the HIP kernels (no GPU needed: hipcc cross-compiles for gfx950).

The attention kernels run two waves per SIMD, so each wave has at most 256 registers, and
the dense D = 128 backward sits at that ceiling.  A change that makes the compiler spill
inside a loop costs far more than it looks, and nothing at run time reports it.  This
compiles the kernel sources the way the library build does, reads the compiler's
per-kernel resource report (-Rpass-analysis=kernel-resource-usage) and fails when any
kernel's private scratch (spill space) grows beyond the amount recorded below, or when a
kernel needs more than 256 registers per wave.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_flash_attn_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Spill bytes per lane allowed per kernel instance (demangled name).  The D = 128 backward
# runs all its products on 16x16x32 MFMAs with two keys (dK/dV) or two queries (dQ) per
# lane at the 256-register ceiling: the dense instances (plain and accumulating) store
# five registers before their loops and reload two per dQ key tile; the varlen instance
# fits without spilling.  Every other kernel must not spill at all.
MAX_SCRATCH = {
    "attn::bwd_kernel<128, false, false>": 20,
    "attn::bwd_kernel<128, false, true>": 20,
}


def resource_report(src):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--offload-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[bytes/lane\])?: (\d+)", line)
        if m and cur:
            kernels[cur][m.group(1).strip()] = int(m.group(2))
    names = list(kernels)
    demangled = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True,
                               text=True).stdout.splitlines()
    out = {}
    for mangled, dm in zip(names, demangled):
        dm = re.sub(r"^void\s+", "", dm)
        dm = re.sub(r"\(.*\)$", "", dm)
        out[dm] = kernels[mangled]
    return out


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("c++filt") is None,
                    reason="hipcc or c++filt not available")
@pytest.mark.parametrize("src", ["fwd.hip", "bwd.hip", "merge.hip"])
def test_no_new_spills(src):
    rep = resource_report(src)
    assert rep, f"no kernel resource report for {src}"
    for name, r in rep.items():
        if "kernel" not in name:
            continue
        scratch = r.get("ScratchSize", 0)
        allowed = MAX_SCRATCH.get(name, 0)
        assert scratch <= allowed, f"{name}: {scratch} B/lane of scratch (spills), allowed {allowed}"
        assert r.get("VGPRs", 0) + r.get("AGPRs", 0) <= 256, (name, r)
