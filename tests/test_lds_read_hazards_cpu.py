"""Static check of the kernel's hand-pipelined GEMM loop, on the CPU.

The matrix-product loop issues its LDS fragment reads in inline-asm blocks and
waits for them (s_waitcnt lgkmcnt) inside later blocks.  The compiler sees the
destination registers of those reads as written when the asm statement ends,
so any compiler-generated instruction placed between the issuing block and the
waiting one that reads them would see stale data (a fragment transform hoisted
above the wait did exactly that once).  This test compiles the kernel to gfx950
assembly and follows every asm LDS read: reads issued are pending until an
lgkmcnt(n) wait leaves at most n younger ones outstanding; no instruction may
read a pending register."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "moe_step_megakernel_amd", "csrc", "moe_step.hip")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _regs(tok):
    tok = tok.strip()
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def in_flight_reads(asm_text):
    """(asm LDS reads, [instructions that read a register whose read is pending])."""
    pending = []          # destination registers of the outstanding asm LDS reads, oldest first
    inasm = False
    reads, hits = 0, []
    for i, line in enumerate(asm_text.split("\n")):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            inasm = True
            continue
        if t.startswith(";;#ASMEND"):
            inasm = False
            continue
        if not t or t[0] in ";." or t.endswith(":"):
            continue
        op = t.split()[0]
        if op.startswith("s_waitcnt") and "lgkmcnt" in t:
            n = int(re.search(r"lgkmcnt\((\d+)\)", t).group(1))
            pending = pending[len(pending) - n:] if n > 0 else []
            continue
        if inasm and op.startswith("ds_read"):
            reads += 1
            pending.append(_regs(t.split()[1].rstrip(",")))
            continue
        if not pending or op.startswith(("s_", "ds_read", "global_", "buffer_")):
            continue
        parts = t.split(None, 1)
        if len(parts) < 2:
            continue
        srcs = set()
        for o in parts[1].split(",")[1:]:
            srcs |= _regs(o)
        if srcs & set().union(*pending):
            hits.append((i + 1, t))
    return reads, hits


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_no_instruction_reads_an_lds_fragment_before_its_wait(tmp_path):
    out = tmp_path / "moe_step_gfx950.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--offload-device-only", "-S", SRC, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    reads, hits = in_flight_reads(out.read_text())
    assert reads > 500, "the asm pipeline's LDS reads were not found"
    assert not hits, f"{len(hits)} instructions read a fragment before its wait, e.g. {hits[:5]}"


def test_checker_flags_a_read_before_the_wait():
    # a fragment read issued in one block, converted before the block that waits
    asm = "\n".join([";;#ASMSTART", "ds_read_b128 v[4:7], v1", "v_mfma_f32_32x32x16_bf16 a[0:15], v[8:11], v[12:15], "
                     "a[0:15]", ";;#ASMEND", "v_lshlrev_b32_e32 v20, 16, v5", ";;#ASMSTART", "s_waitcnt lgkmcnt(0)",
                     ";;#ASMEND", "v_lshlrev_b32_e32 v21, 16, v6"])
    reads, hits = in_flight_reads(asm)
    assert reads == 1 and len(hits) == 1 and "v20" in hits[0][1]
