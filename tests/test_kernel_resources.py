"""Register budgets of the MFMA kernels, checked at compile time (no GPU).

The large GEMMs and the prefill attention run two waves per SIMD, so each
has at most 256 registers per lane; a kernel that crosses that spills to
scratch memory and slows down many times over while its results stay the
same (the parity tests cannot see it).  This compiles their sources for
gfx950 with the compiler's resource remarks and fails on any spill, except
the fp32-residual epilogue of the bf16 DMA GEMM, whose 32 spilled registers
sit after the K loop.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_gqa_transformer_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# kernel (mangled-name fragment) -> VGPR spills allowed
ALLOWED = {"gemm_dma_kernelILi1ELb0E": 32}


def _resources(src):
    cmd = [HIPCC, "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs Spill|ScratchSize \[bytes/lane\]|VGPRs): (\d+)", line)
        if m and name:
            out[name][m.group(1)] = int(m.group(2))
    return out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["gemm_f8.hip", "gemm_dma.hip", "attn_fa.hip"])
def test_mfma_kernels_do_not_spill(src):
    res = _resources(src)
    assert res, "no kernels reported"
    for name, r in res.items():
        allowed = next((v for k, v in ALLOWED.items() if k in name), 0)
        assert r.get("VGPRs Spill", 0) <= allowed, f"{src}: {name} spills {r.get('VGPRs Spill')} VGPRs"
