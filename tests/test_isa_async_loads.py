"""The attention kernels load each unit's query and sinks with inline-asm loads (and the split
kernel's consumers add to their group's count with an inline-asm atomic) whose destination
registers fill in asynchronously: the compiler sees a finished value at the
load, so nothing stops it from copying or spilling those registers before the data has
arrived. The kernels are correct only if it never does, i.e. if every instruction that
touches such a destination comes after an `s_waitcnt vmcnt` (the explicit waits that cover
the loads). This compiles csrc/sa_attn.hip, csrc/sa_attn_split.hip, csrc/sa_attn_f32.hip and
csrc/sa_attn_f32_split.hip to gfx950 assembly with the library's own flags and checks that, for every kernel, along the code that follows
each such load.
"""
import os
import re
import shutil
import subprocess

import pytest

from sparse_attention_attn_amd import build as B

HIPCC = B.HIPCC if os.path.exists(B.HIPCC) else shutil.which("hipcc")
pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not found")

LOAD = re.compile(r"^\s*(?:global_load_dword(?:x2|x3|x4)?|global_atomic_\w+)\s+([av](?:\[\d+:\d+\]|\d+)),")
RANGE = re.compile(r"\b([av])\[(\d+):(\d+)\]")
SINGLE = re.compile(r"\b([av])(\d+)\b")


def registers(text):
    regs = {(c, i) for c, lo, hi in RANGE.findall(text) for i in range(int(lo), int(hi) + 1)}
    regs |= {(c, int(i)) for c, i in SINGLE.findall(RANGE.sub(" ", text))}
    return regs


def kernels(asm):
    """{symbol: [instruction lines]} for every kernel in an assembly listing."""
    out, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur = m.group(1)
            out[cur] = []
            continue
        if cur is not None:
            out[cur].append(line)
            if "s_endpgm" in line:
                cur = None
    return out


def early_touches(lines):
    """(load line, offending line) pairs: an async register load whose destination is read
    or written before the next vector-memory wait, in program text order."""
    bad, in_asm, loads = [], False, 0
    for i, line in enumerate(lines):
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        m = LOAD.match(line) if in_asm else None
        if not m or " lds" in line:
            continue
        loads += 1
        dst = registers(m.group(1))
        for later in lines[i + 1:]:
            code = later.split(";")[0]
            if "s_waitcnt" in code and "vmcnt" in code:
                break
            if registers(code) & dst:
                bad.append((line.strip(), later.strip()))
                break
    return bad, loads


def test_parser_finds_an_early_copy():
    listing = "\n".join([
        ";;#ASMSTART", "\tglobal_load_dwordx4 v[156:159], v[154:155], off", ";;#ASMEND",
        "\tv_accvgpr_write_b32 a2, v156",
        "\ts_waitcnt vmcnt(0)",
        ";;#ASMSTART", "\tglobal_load_dwordx4 a[0:3], v[6:7], off", ";;#ASMEND",
        "\ts_waitcnt vmcnt(1)",
        "\tv_mfma_f32_16x16x32_bf16 v[8:11], v[12:15], a[0:3], 0",
    ])
    bad, loads = early_touches(listing.splitlines())
    assert loads == 2 and len(bad) == 1 and "a2, v156" in bad[0][1]


@pytest.mark.parametrize("src,tag", [("sa_attn.hip", "attn_bf16"), ("sa_attn_split.hip", "attn_split"),
                                     ("sa_attn_f32.hip", "attn_f32"), ("sa_attn_f32_split.hip", "attn_f32_split")])
def test_async_query_loads_are_not_touched_before_a_wait(tmp_path, src, tag):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, *B.HIP_FLAGS, *B.COMMON, "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    ks = {k: v for k, v in kernels(out.read_text()).items() if tag in k}
    assert ks, f"no {tag} kernels in the listing"
    total = 0
    for name, lines in ks.items():
        bad, loads = early_touches(lines)
        total += loads
        assert not bad, f"{name}: async load destination touched before its wait: {bad[:3]}"
    assert total > 0, "no asynchronous register loads found"
