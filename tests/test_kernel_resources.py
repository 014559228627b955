"""Register budget of every gfx950 kernel, read from the compiler's own
resource metadata (device assembly of each HIP source, compiled here on the
CPU). A kernel that spills vector registers inside its block loop runs much
slower with the same results, so no parity test notices; this test does.

Budget: no vector-register spills in any kernel.
"""

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_109_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# kernel-name fragment -> allowed vector-register spills (default 0)
SPILL_ALLOWANCE = {}


def compile_to_asm(src):
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           "-o", "-", src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout


def kernel_resources(asm):
    """(name, vgpr_count, vgpr_spill_count, lds_bytes) per kernel from the AMDGPU metadata."""
    out = []
    for block in asm.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        vgpr = int(re.search(r"\.vgpr_count:\s+(\d+)", block).group(1))
        spill = int(re.search(r"\.vgpr_spill_count:\s+(\d+)", block).group(1))
        lds = int(re.search(r"\.group_segment_fixed_size:\s+(\d+)", block).group(1))
        out.append((name, vgpr, spill, lds))
    return out


@pytest.fixture(scope="module")
def resources():
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        asms = list(ex.map(compile_to_asm, srcs))
    return {os.path.basename(s): kernel_resources(a) for s, a in zip(srcs, asms)}


def test_every_source_has_kernels(resources):
    for src, ks in resources.items():
        assert ks, f"{src}: no kernel metadata found"


def test_no_vector_register_spills(resources):
    bad = []
    for src, ks in resources.items():
        for name, vgpr, spill, lds in ks:
            allowed = max([v for frag, v in SPILL_ALLOWANCE.items() if frag in name], default=0)
            if spill > allowed:
                bad.append(f"{src}: {name} spills {spill} VGPRs (allowed {allowed}, {vgpr} in use)")
    assert not bad, "\n".join(bad)


def test_register_and_lds_limits(resources):
    for src, ks in resources.items():
        for name, vgpr, spill, lds in ks:
            assert vgpr <= 512, (src, name, vgpr)
            assert lds <= 160 * 1024, (src, name, lds)
