"""The routing kernel's DPP fma chains, checked in the generated gfx950 code.

The bf16 routing path multiplies through `v_fmac_f32_dpp ... row_newbcast`
written as inline asm.  On gfx9 a DPP instruction must not read a VGPR that a
VALU instruction wrote in the two wait states before it, and the compiler's
hazard check does not look inside inline asm, so the kernel places the wait
states itself.  This test compiles route.hip for gfx950 and walks back from
every `v_fmac_f32_dpp` in every route_kernel instantiation: no VALU write of
any of its VGPR operands (accumulator, broadcast source, centroid value) may
sit within two wait states (an instruction counts one, `s_nop N` counts N+1).
A label within that distance counts as a violation (another path may enter
there).  No GPU needed.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fine_grained_mixture_moe_amd", "csrc")

VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def vregs(text: str) -> set:
    out = set()
    for m in VREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def valu_dest(ins: str):
    """VGPRs written by a VALU instruction (None if it writes none)."""
    op = ins.split()[0]
    if not op.startswith("v_") or op.startswith(("v_readlane", "v_readfirstlane", "v_cmp")):
        return None
    operands = ins[len(op):].split(",")
    return vregs(operands[0]) if operands else None


def check(asm: str):
    lines = [l.split(";")[0].strip() for l in asm.split("\n")]
    fn = None
    n_dpp, bad = 0, []
    for k, line in enumerate(lines):
        if re.match(r"^_Z\S*:$", line):
            fn = line[:-1]
            continue
        if fn is None or "route_kernel" not in fn or not line.startswith("v_fmac_f32_dpp"):
            continue
        n_dpp += 1
        regs = vregs(line.split("row_newbcast")[0][len("v_fmac_f32_dpp"):])
        ws, j = 0, k - 1
        while ws < 2 and j >= 0:
            prev = lines[j]
            j -= 1
            if not prev or prev.startswith((".", "#")):
                continue
            if prev.endswith(":"):
                bad.append((fn, k, line, "label within two wait states"))
                break
            if prev.startswith("s_nop"):
                ws += int(prev.split()[1], 0) + 1
                continue
            dest = valu_dest(prev)
            if dest and dest & regs:
                bad.append((fn, k, line, prev))
                break
            ws += 1
    return n_dpp, bad


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_dpp_fma_operands_have_their_wait_states(tmp_path):
    out = tmp_path / "route.s"
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-S", "--cuda-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "route.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    n_dpp, bad = check(out.read_text())
    assert n_dpp > 0, "no DPP fma in the routing kernels"
    assert not bad, "\n".join(f"{f} line {k}: {l}  <- {why}" for f, k, l, why in bad[:20])


def test_checker_flags_a_planted_hazard():
    """The checker itself: a VALU write right before the DPP read is caught, two nops clear it."""
    base = """_ZN3moe12route_kernelE:
\tv_and_b32_e32 v70, 0xffff0000, v18
{nops}\tv_fmac_f32_dpp v25, v70, v39 row_newbcast:0 row_mask:0xf bank_mask:0xf
"""
    n, bad = check(base.format(nops=""))
    assert n == 1 and len(bad) == 1
    n, bad = check(base.format(nops="\ts_nop 0\n"))
    assert len(bad) == 1
    n, bad = check(base.format(nops="\ts_nop 1\n"))
    assert not bad
    # the accumulator counts too
    acc = """_ZN3moe12route_kernelE:
\ts_nop 1
\tv_fmac_f32_dpp v25, v1, v39 row_newbcast:0 row_mask:0xf bank_mask:0xf
\tv_fmac_f32_dpp v26, v1, v39 row_newbcast:0 row_mask:0xf bank_mask:0xf
\tv_fmac_f32_dpp v25, v2, v40 row_newbcast:1 row_mask:0xf bank_mask:0xf
"""
    n, bad = check(acc)
    assert n == 3 and len(bad) == 1
