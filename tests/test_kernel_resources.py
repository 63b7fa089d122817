"""Compile-time resource check of the HIP kernels (CPU only).

The persistent megakernel holds every task body; if the compiler stops
inlining one of them, the kernel arguments are copied to per-lane scratch
memory and every access to them becomes a memory round trip.  This test
compiles the kernels for gfx950 with the resource-usage remarks and requires
that no kernel uses scratch or spills registers, and that the persistent
kernels keep two workgroups per CU (at most 256 VGPRs).  The big-tile
variant runs one workgroup a CU with the full register file (256 VGPRs and
256 accumulation registers); its G bodies fill it, so the compiler spills a
few of the runner's registers around them: bounded here, and never inside
the MFMA loops (checked in the assembly)."""
import os
import re
import shutil
import subprocess

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "dynamic_moe_task_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_kernels_use_no_scratch(tmp_path):
    asm = tmp_path / "k.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-S", "--cuda-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", CSRC,
           os.path.join(CSRC, "moe_kernels.hip"), "-o", str(asm),
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels = {}
    name = None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[bytes/lane\])?: (\d+)", line)
        if m and name:
            kernels[name][m.group(1).strip()] = int(m.group(2))
    persistent = [k for k in kernels if "moe_persistent" in k and "moe_persistent_big" not in k]
    big = [k for k in kernels if "moe_persistent_big" in k]
    # STATIC, DYNAMIC, BARRIER and ORDERED, each in a small-batch and a large-batch
    # variant, and the decoder layer's STATIC and ORDERED; the four schedules
    # again in the big-tile variant
    assert len(persistent) == 10, sorted(kernels)
    assert len(big) == 4, sorted(kernels)
    text = asm.read_text().split("\n")
    for k in big:
        v = kernels[k]
        assert v["VGPRs"] <= 256 and v.get("AGPRs", 0) <= 256, (k, v)
        assert v.get("ScratchSize", 0) <= 256, (k, v)
        if "moe_persistent_bigILi1E" in k:
            continue  # DYNAMIC (switched off at the ABI; see below)
        # no spill or reload within 50 lines of any MFMA of the G loops
        start = next(i for i, l in enumerate(text) if l.startswith(k + ":"))
        end = next(i for i in range(start, len(text)) if "s_endpgm" in text[i])
        body = text[start:end]
        mfma = [i for i, l in enumerate(body) if "v_mfma_f32_32x32x16" in l]
        spill = [i for i, l in enumerate(body) if "scratch_" in l]
        assert mfma, k
        clusters = []
        for i in mfma:
            if clusters and i - clusters[-1][1] < 400:
                clusters[-1][1] = i
            else:
                clusters.append([i, i])
        for a, b in clusters:
            assert not [i for i in spill if a - 50 <= i <= b + 50], (k, a, b)
    for k, v in kernels.items():
        if "moe_persistent_big" in k:
            continue
        if "moe_persistentILi1E" in k:
            # DYNAMIC holds every task body in one loop over popped
            # descriptors; at the 256-VGPR cap of two workgroups a CU it
            # spills a few registers (the schedule is switched off at the
            # ABI, so its speed is not what this guards)
            assert v.get("ScratchSize", 0) <= 256, (k, v)
            continue
        assert v.get("ScratchSize", 0) == 0, (k, v)
        assert v.get("VGPRs Spill", 0) == 0, (k, v)
    for k in persistent:
        assert kernels[k]["VGPRs"] + kernels[k].get("AGPRs", 0) <= 256, (k, kernels[k])
