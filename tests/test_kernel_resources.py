"""Register and scratch budget of the kernels (host-only: compiles the HIP
sources to gfx950 assembly and reads the kernel metadata).

Every attention kernel must fit its registers without spilling to scratch:
a spill puts scratch traffic inside the key loop (it cost the 64-row
kernels about 70 % in time when it happened).  The 8-wave work-groups need
at most 256 VGPRs per lane for two waves per SIMD."""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_attention_diffusion_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _kernel_meta(src):
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "k.s")
        cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        text = open(out).read()
    meta = {}
    for block in re.split(r"\n\s+- \.", text.split("amdhsa.kernels:")[1]):
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        vals = {k: int(v) for k, v in re.findall(r"\.(vgpr_count|vgpr_spill_count|sgpr_spill_count|"
                                                 r"agpr_count|group_segment_fixed_size|"
                                                 r"private_segment_fixed_size):\s+(\d+)", block)}
        meta[name.group(1)] = vals
    return meta


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", ["attn_bf16.hip", "attn.hip"])
def test_attention_kernels_do_not_spill(src):
    meta = _kernel_meta(src)
    split = {k: v for k, v in meta.items() if "attn_split" in k}
    assert split, f"no split kernels found in {src}"
    for name, v in split.items():
        assert v.get("vgpr_spill_count", 0) == 0, (name, v)
        assert v.get("sgpr_spill_count", 0) == 0, (name, v)
        budget = 256 if "bf16" in name else 512
        assert v.get("vgpr_count", 0) + v.get("agpr_count", 0) <= budget, (name, v)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")))
def test_no_kernel_uses_scratch(src):
    meta = _kernel_meta(src)
    if not meta:
        pytest.skip(f"{src} holds host code only")
    for name, v in meta.items():
        assert "private_segment_fixed_size" in v, name
        assert v["private_segment_fixed_size"] == 0, (name, v)
