"""Wait states that the compiler does not insert inside inline assembly, checked on the gfx950
assembly generated from the prefill source (no GPU needed; skipped without hipcc).

The prefill kernels issue their LDS-direct tile loads (buffer_load_dwordx4 ... lds) from inline
assembly, and the compiler's hazard recognizer does not look inside assembly blocks.  Two
hazards of the CDNA instruction set apply to such a load (AMD Instinct MI300/CDNA3 ISA reference,
"Manually Inserted Wait States"; gfx950 keeps them): a vector memory instruction that reads an
SGPR written by a VALU instruction (v_readlane, v_readfirstlane, ...) needs five wait states after
that write, and an LDS-direct load needs one after M0 is written.  The source is compiled with
the build's flags under the default machine scheduler and under iterative-ilp, a schedule that
reloads the loads' buffer-resource words from spill lanes right before them.  The test then
counts wait states back from every LDS-direct load (s_nop N gives N + 1, any other instruction
one).
"""

import importlib.util
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "heterogeneous_sliding_windows_amd")


def _build_module():
    spec = importlib.util.spec_from_file_location("moa_build", os.path.join(PKG, "build.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _sgprs(tok):
    """SGPR numbers an operand names: s5 -> {5}, s[4:7] -> {4, 5, 6, 7}; m0 -> {'m0'}."""
    tok = tok.strip()
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m[1]), int(m[2]) + 1))
    m = re.fullmatch(r"s(\d+)", tok)
    if m:
        return {int(m[1])}
    return {"m0"} if tok == "m0" else set()


def _instructions(asm_text):
    out = []
    for line in asm_text.splitlines():
        line = line.split(";")[0].strip()
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        out.append(line)
    return out


def _dest(ins):
    parts = ins.split(None, 1)
    return parts[1].split(",")[0] if len(parts) > 1 else ""


def lds_direct_violations(asm_text):
    """[(load, writer, wait states)] for every LDS-direct load that reads an SGPR a VALU
    instruction wrote fewer than 5 wait states earlier, or M0 fewer than 1 after its write,
    and the number of LDS-direct loads.  A later scalar write of the SGPR ends the hazard."""
    ins = _instructions(asm_text)
    bad, loads = [], 0
    for i, load in enumerate(ins):
        if not (load.startswith("buffer_load") and load.endswith(" lds")):
            continue
        loads += 1
        ops = load.split(None, 1)[1].split(",")
        valu_watch = _sgprs(ops[1]) | _sgprs(ops[2].split()[0])
        m0_pending = True
        waits, j = 0, i - 1
        while j >= 0 and waits < 5 and (valu_watch or m0_pending):
            prev = ins[j]
            j -= 1
            op = prev.split()[0]
            dst = _sgprs(_dest(prev))
            if m0_pending and "m0" in dst:
                if waits < 1:
                    bad.append((load, prev, waits))
                m0_pending = False
            if op.startswith("v_") and dst & valu_watch:
                bad.append((load, prev, waits))
                valu_watch -= dst
            elif op.startswith("s_"):
                valu_watch -= dst
            waits += int(prev.split()[1], 0) + 1 if op == "s_nop" else 1
    return bad, loads


def _compile_asm(extra, out):
    b = _build_module()
    cmd = [b.hipcc(), *b.COMMON, *extra, "-x", "hip", "--cuda-device-only", "-S",
           os.path.join(b.CSRC, "prefill.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


def test_checker_flags_the_hazards():
    """The scan itself: a VALU write of a resource word or the soffset too close to the load,
    and an M0 write right before it, are caught; enough wait states or a scalar rewrite clear it."""
    close = "v_readlane_b32 s7, v204, 12\ns_nop 0\nbuffer_load_dwordx4 v1, s[4:7], s9 offen lds\n"
    assert len(lds_direct_violations(close)[0]) == 1
    soff = "v_readfirstlane_b32 s9, v3\ns_nop 2\nbuffer_load_dwordx4 v1, s[4:7], s9 offen lds\n"
    assert len(lds_direct_violations(soff)[0]) == 1
    far = "v_readlane_b32 s7, v204, 12\ns_nop 4\nbuffer_load_dwordx4 v1, s[4:7], s9 offen lds\n"
    assert lds_direct_violations(far) == ([], 1)
    rewritten = ("v_readlane_b32 s7, v204, 12\ns_mov_b32 s7, s2\n"
                 "buffer_load_dwordx4 v1, s[4:7], s9 offen lds\n")
    assert lds_direct_violations(rewritten) == ([], 1)
    m0 = "s_mov_b32 m0, s1\nbuffer_load_dwordx4 v1, s[4:7], s9 offen lds\n"
    assert len(lds_direct_violations(m0)[0]) == 1
    m0_ok = "s_mov_b32 m0, s1\ns_nop 0\nbuffer_load_dwordx4 v1, s[4:7], s9 offen lds\n"
    assert lds_direct_violations(m0_ok) == ([], 1)


@pytest.mark.parametrize("sched", ["default", "iterative-ilp"])
def test_lds_direct_loads_wait_for_their_operands(tmp_path, sched):
    b = _build_module()
    try:
        b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    extra = [] if sched == "default" else ["-mllvm", "-amdgpu-sched-strategy=" + sched]
    asm = _compile_asm(extra, str(tmp_path / "prefill.s"))
    bad, loads = lds_direct_violations(asm)
    # two D instantiations x (plain, handoff) x (prologue + loop) tiles of K and V loads
    assert loads >= 16, loads
    assert not bad, "\n".join(f"{w} ({n} wait states) before {l}" for l, w, n in bad[:8])
