"""The routing kernels' load pipelines, checked in the generated gfx950 code.

With one token per wave in 4-wave blocks, the route kernel keeps three
centroid/token chunks in flight in four register sets.  That only works while
the compiler's wait counts before the LDS stores stay partial: a branch around
a load, or a loop left from inside the unrolled group, made it fall back to
waiting for every load (vmcnt(0)) at each chunk, which costs a full memory
latency per chunk.  This test compiles route.hip for gfx950 and checks, in
every 1-token 4-wave route_kernel instantiation, the loop that stores the
chunks to LDS: every vmcnt wait in its body must leave at least one register
set (five loads) in flight.  The decode kernel's k loop (direct-to-LDS loads, S
stages per wave) is checked the same way: one partial wait per step, the loads
of S - 3 chunks left in flight.  No GPU needed.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fine_grained_mixture_moe_amd", "csrc")
RING = re.compile(r"^(_Z\S*route_kernelILi1ELi\d+ELi4ELb[01]E\S*):$")


def ring_loops(asm: str):
    """(kernel, [vmcnt values]) of each backward-branch loop that stores to LDS."""
    out = []
    lines = [l.split(";")[0].strip() for l in asm.split("\n")]
    fn, labels, start = None, {}, 0
    for k, line in enumerate(lines):
        m = RING.match(line)
        if m:
            fn, labels, start = m.group(1), {}, k
            continue
        if re.match(r"^_Z\S*:$", line):
            fn = None
            continue
        if fn is None:
            continue
        lm = re.match(r"^(\.LBB\S+):$", line)
        if lm:
            labels[lm.group(1)] = k
            continue
        bm = re.search(r"s_(?:cbranch_\w+|branch)\s+(\.LBB\S+)", line)
        if bm and bm.group(1) in labels and labels[bm.group(1)] < k:
            body = lines[labels[bm.group(1)]:k + 1]
            if any(b.startswith("ds_write_b128") for b in body) and any(b.startswith("s_barrier") for b in body):
                waits = [int(w) for b in body for w in re.findall(r"vmcnt\((\d+)\)", b)]
                out.append((fn, waits))
    return out


@pytest.fixture(scope="module")
def route_asm(tmp_path_factory):
    """route.hip compiled for gfx950 (device code, assembly), once for the tests of this file."""
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("route") / "route.s"
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-S", "--cuda-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "route.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def test_ring_loop_keeps_loads_in_flight(route_asm):
    loops = ring_loops(route_asm)
    kernels = {fn for fn, _ in loops}
    assert len(kernels) >= 6, f"expected the 1-token 4-wave instantiations, found {sorted(kernels)}"
    bad = [(fn, w) for fn, w in loops if not w or min(w) < 5]
    assert not bad, "\n".join(f"{fn}: vmcnt waits {w}" for fn, w in bad)


def test_checker_flags_a_full_wait():
    """The checker itself: a vmcnt(0) in an LDS-storing loop is reported, partial waits are not."""
    asm = """_ZN3moe12_GLOBAL__N_112route_kernelILi1ELi1ELi4ELb1EEEviiiiiPKvPKfS5_PiPfS7_S6_Pd:
.LBB0_1:
\tglobal_load_dwordx4 v[2:5], v[6:7], off
\ts_waitcnt vmcnt({n})
\tds_write_b128 v8, v[10:13]
\ts_barrier
\ts_cbranch_scc1 .LBB0_1
\ts_endpgm
"""
    (fn, waits), = ring_loops(asm.format(n=0))
    assert waits == [0]
    (fn, waits), = ring_loops(asm.format(n=15))
    assert min(waits) >= 5


# The decode routing kernel (one workgroup per token): each wave streams its centroid chunks
# straight into LDS, S stages deep, and waits for one chunk at a time.
DECODE = re.compile(r"^(_Z\S*route_decode_kernelILi(\d+)ELi(\d+)ELb[01]E\S*):$")


def decode_k_loops(asm: str):
    """(kernel, S, vmcnt waits, lgkmcnt waits, fmas) of each decode instantiation's innermost loop
    that issues direct-to-LDS loads (its k loop)."""
    best = {}
    lines = [l.split(";")[0].strip() for l in asm.split("\n")]
    fn, labels, S = None, {}, 0
    for k, line in enumerate(lines):
        m = DECODE.match(line)
        if m:
            fn, labels, S = m.group(1), {}, int(m.group(3))
            continue
        if re.match(r"^_Z\S*:$", line):
            fn = None
            continue
        if fn is None:
            continue
        lm = re.match(r"^(\.LBB\S+):$", line)
        if lm:
            labels[lm.group(1)] = k
            continue
        bm = re.search(r"s_(?:cbranch_\w+|branch)\s+(\.LBB\S+)", line)
        if bm and bm.group(1) in labels and labels[bm.group(1)] < k:
            body = lines[labels[bm.group(1)]:k + 1]
            if not any(b.startswith("buffer_load_dwordx4") and b.endswith(" lds") for b in body):
                continue
            if fn in best and len(best[fn][-1]) <= len(body):
                continue
            vm = [int(w) for b in body for w in re.findall(r"vmcnt\((\d+)\)", b)]
            lg = [int(w) for b in body for w in re.findall(r"lgkmcnt\((\d+)\)", b)]
            fm = sum(1 for b in body if b.startswith("v_fmac_f32"))
            best[fn] = (S, vm, lg, fm, body)
    return [(fn, S, vm, lg, fm) for fn, (S, vm, lg, fm, _) in best.items()]


def test_decode_k_loop_keeps_chunks_in_flight(route_asm):
    """In every decode instantiation the k loop runs its S steps without a branch (32 fmas each),
    waits for one chunk per step and leaves the loads of the next S - 3 chunks in flight (vmcnt
    8 (S - 3), never 0), and waits for LDS reads at most twice per step."""
    loops = decode_k_loops(route_asm)
    assert len(loops) >= 14, f"expected the 7 forms x 2 token types, found {len(loops)}"
    bad = []
    for fn, S, vm, lg, fm in loops:
        if fm != 32 * S or not vm or set(vm) != {8 * (S - 3)} or len(vm) != S or len(lg) > 2 * S:
            bad.append(f"{fn}: S={S} fmas={fm} vmcnt={vm} lgkmcnt={len(lg)} waits")
    assert not bad, "\n".join(bad)


def test_decode_checker_sees_a_full_wait():
    """The decode checker itself: a k loop waiting for every load is reported as vmcnt [0]."""
    asm = """_ZN3moe12_GLOBAL__N_119route_decode_kernelILi1ELi8ELb1EEEviiiiiPKvPKfS5_PiPfS7_S6_Pd:
.LBB5_19:
\ts_waitcnt vmcnt(0)
\tv_fmac_f32_e32 v81, v54, v62
\tbuffer_load_dwordx4 v66, s[16:19], s12 offen lds
\ts_cbranch_scc0 .LBB5_19
\ts_endpgm
"""
    (fn, S, vm, lg, fm), = decode_k_loops(asm)
    assert (S, vm, fm) == (8, [0], 1)
