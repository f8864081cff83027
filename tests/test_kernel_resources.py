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


def _asm(src):
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "k.s")
        cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


def _regs(operand_text):
    regs = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", operand_text):
        if m.group(3):
            regs.add(int(m.group(3)))
        else:
            regs.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return regs


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_in_flight_v_reads_are_left_alone():
    """The D = 128 split kernels issue the V transpose reads of one tile in
    the same asm batch as the K reads of the next and wait for them only
    before the PV MFMAs (kv_issue / tr_wait16).  In the built code nothing
    between the batch and that wait may read or write the registers the V
    reads are landing in, and the batch must be what the code assumes (8 K
    reads, then 16 transpose reads around one wait for 8 outstanding)."""
    text = _asm("attn_bf16.hip")
    funcs = re.findall(r"\n(_ZN5wedlm15attn_split_bf16ILi128ELi\dEEEvNS_8AttnArgsE):[^\n]*\n(.*?)\n\.Lfunc_end",
                       text, re.S)
    assert funcs
    checked = 0
    for name, body in funcs:
        lines = [l.split(";")[0].strip() for l in body.split("\n")]
        lines = [l for l in lines if l and not l.startswith(".")]
        for i, l in enumerate(lines):
            if l != "s_waitcnt lgkmcnt(8)":
                continue
            before = lines[i - 16:i]
            if not (all(x.startswith("ds_read_b128") for x in before[:8])
                    and all(x.startswith("ds_read_b64_tr_b16") for x in before[8:])):
                continue
            after = lines[i + 1:i + 9]
            assert all(x.startswith("ds_read_b64_tr_b16") for x in after), (name, after)
            v_regs = set()
            for x in before[8:] + after:
                v_regs |= _regs(x.split(None, 1)[1].split(",")[0])
            j = i + 9
            while lines[j] != "s_waitcnt lgkmcnt(0)":
                ops = lines[j].split(None, 1)
                assert not (len(ops) > 1 and _regs(ops[1]) & v_regs), (name, lines[j])
                assert not lines[j].startswith("ds_"), (name, lines[j])
                j += 1
            checked += 1
    assert checked >= 1, "no K+V read batch found in the D = 128 split kernels"
