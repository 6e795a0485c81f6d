"""Resource gate of every gfx950 kernel, read from the compiler's own kernel descriptors (the
analogue of the pages' check of thread and threadgroup-memory use against the device limits,
akol1/TensorFold pull request 4, PR body, gate 5).

Each HIP source is compiled to device assembly with the library's own flags. For every kernel:
* no scratch (private segment 0, no dynamic stack): a spill would put registers in memory;
* LDS within the 160 KiB of a CU, times the workgroups per CU its launch plan counts on;
* registers within what the waves per SIMD of its launch allow: the unified register file holds
  512 per lane and SIMD, allocated in granules of 8, and a workgroup of 64 W threads puts W / 4
  waves on each SIMD (more where the launch plan counts on several workgroups per CU).
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from sparse_attention_attn_amd import build as B

HIPCC = B.HIPCC if os.path.exists(B.HIPCC) else shutil.which("hipcc")
pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not found")

SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]
LDS_PER_CU = 160 * 1024
REGS_PER_LANE = 512
# Kernels whose launch plan counts on several workgroups per CU (name fragment: count).
WORKGROUPS_PER_CU = {"topk_rows8_kernel": 4}


def descriptors(asm):
    """{kernel symbol: {field: int}} from the .amdhsa_kernel blocks, plus the flat workgroup
    size from the metadata."""
    out = {}
    for name, body in re.findall(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", asm, re.S):
        out[name] = {k: int(v) for k, v in re.findall(r"\.amdhsa_(\w+) (\d+)", body)}
    for m in re.finditer(r"\.max_flat_workgroup_size:\s+(\d+)\n(?:.*\n)*?\s+\.name:\s+(\S+)", asm):
        if m.group(2) in out:
            out[m.group(2)]["max_flat_workgroup_size"] = int(m.group(1))
    return out


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    d = tmp_path_factory.mktemp("isa_res")

    def compile_one(src):
        out = d / (src + ".s")
        cmd = [HIPCC, *B.HIP_FLAGS, *B.COMMON, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(out)]
        subprocess.run(cmd, check=True, capture_output=True)
        return src, descriptors(out.read_text())

    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        return dict(ex.map(compile_one, SOURCES))


def test_every_source_has_kernels(kernels):
    for src, ks in kernels.items():
        if src == "sa_noalloc.hip":  # the static scratch array only
            continue
        assert ks, f"{src}: no kernel descriptors in the listing"
        for name, f in ks.items():
            assert "max_flat_workgroup_size" in f, f"{src}: {name} has no workgroup size in its metadata"


def test_no_scratch_and_no_dynamic_stack(kernels):
    for src, ks in kernels.items():
        for name, f in ks.items():
            assert f["private_segment_fixed_size"] == 0, f"{src}: {name} spills to scratch"
            assert f.get("uses_dynamic_stack", 0) == 0, f"{src}: {name} uses a dynamic stack"


def test_lds_and_registers_fit_the_launch(kernels):
    seen = 0
    for src, ks in kernels.items():
        for name, f in ks.items():
            wgs = next((n for frag, n in WORKGROUPS_PER_CU.items() if frag in name), 1)
            lds = f["group_segment_fixed_size"]
            assert lds * wgs <= LDS_PER_CU, f"{src}: {name}: {wgs} x {lds} B of LDS per CU"
            waves_per_simd = wgs * f["max_flat_workgroup_size"] // 64 // 4
            regs = -(-f["next_free_vgpr"] // 8) * 8
            assert regs * max(waves_per_simd, 1) <= REGS_PER_LANE, (
                f"{src}: {name}: {regs} registers per lane for {waves_per_simd} waves per SIMD")
            seen += 1
    assert seen >= 20, "fewer kernels than the library has"


def test_attention_kernels_two_waves_per_simd(kernels):
    """The bf16 attention kernels are built for eight waves per workgroup, one workgroup per CU,
    two waves per SIMD (one wave's softmax beside the other's matrix products)."""
    names = [n for ks in kernels.values() for n in ks if "attn_bf16" in n or "attn_split_kernel" in n]
    assert names
    for src, ks in kernels.items():
        for name, f in ks.items():
            if name in names:
                assert f["max_flat_workgroup_size"] == 512, name
                assert -(-f["next_free_vgpr"] // 8) * 8 <= 256, name
