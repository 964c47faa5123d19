"""Wait states around the GEMM's inline-assembly LDS copies (CPU only).

The forward GEMM issues its global -> LDS copies (buffer_load ... lds) as
inline assembly, which the compiler's hazard recognizer does not look into.
gfx9 requires five wait states between a VALU write of an SGPR (such as
v_readfirstlane, which the compiler uses to rematerialise descriptors) and a
VMEM instruction reading it, and one between an SALU write of M0 and an LDS
DMA.  The copies carry their own s_nop for that; this test compiles
csrc/gemm.hip for gfx950 to assembly and checks every such copy in every
kernel (inline-asm and compiler-generated alike): no VALU instruction
writing one of its SGPR operands (descriptor, soffset) within the preceding
five wait states, and at least one wait state after the M0 write."""

import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "scaled_quantize_fp8_amd", "csrc", "gemm.hip")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def _sgprs(tok):
    out = set()
    for m in re.finditer(r"s\[(\d+):(\d+)\]", tok):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"(?<![\w\[])s(\d+)\b", tok):
        out.add(int(m.group(1)))
    return out


def scan(lines):
    """Return (hazards, copies): hazards lists (function, wait states, VALU
    line, copy line); copies counts the LDS DMAs seen."""
    hazards, copies, func, recent = [], 0, None, []
    for line in lines:
        if re.match(r"^_Z\w+:", line):
            func, recent = line.split(":")[0], []
            continue
        s = line.strip()
        if not s or s.startswith(";") or s.startswith(".") or s.endswith(":"):
            continue
        op = s.split()[0]
        if op.startswith("buffer_load") and s.endswith(" lds"):
            copies += 1
            need = set()
            for o in s[len(op):].split(",")[1:]:
                need |= _sgprs(o)
            ws = 0
            # M0 must not be written by the instruction right before the copy
            m0_ok = not (recent and recent[-1][0].startswith("s_") and recent[-1][1].split()[1:2] == ["m0,"])
            for i, (pop, ptxt) in enumerate(reversed(recent)):
                if ws >= 5:
                    break
                if pop == "s_nop":
                    ws += int(ptxt.split()[1], 0) + 1
                    continue
                if pop.startswith("v_") and _sgprs(ptxt[len(pop):].split(",")[0]) & need:
                    hazards.append((func, ws, ptxt, s))
                    break
                ws += 1
            if not m0_ok:
                hazards.append((func, 0, "M0 written by the instruction right before the LDS DMA", s))
        recent.append((op, s))
        if len(recent) > 16:
            recent.pop(0)
    return hazards, copies


def test_scan_flags_a_planted_hazard():
    """The scanner itself: a readfirstlane two slots before a copy reading
    that SGPR is a hazard; five wait states of s_nop clear it."""
    bad = ["_Zk:", "v_readfirstlane_b32 s29, v44", "s_mov_b32 m0, s7", "s_nop 0",
           "buffer_load_dwordx4 v10, s[28:31], s46 offen lds"]
    good = ["_Zk:", "v_readfirstlane_b32 s29, v44", "s_mov_b32 m0, s7", "s_nop 4",
            "buffer_load_dwordx4 v10, s[28:31], s46 offen lds"]
    no_nop = ["_Zk:", "s_mov_b32 m0, s7", "buffer_load_dwordx4 v10, s[28:31], s46 offen lds"]
    assert len(scan(bad)[0]) == 1
    assert scan(good) == ([], 1)
    assert len(scan(no_nop)[0]) == 1


@pytest.mark.timeout(600)
def test_gemm_lds_copies_keep_their_wait_states():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "gemm.s")
        cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "--cuda-device-only", "-S", SRC, "-o", out, "-w"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        hazards, copies = scan(open(out).read().split("\n"))
    assert copies > 100, "no inline-asm LDS copies found: the scan no longer matches the code"
    assert not hazards, hazards[:5]
