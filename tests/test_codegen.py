"""Wait states that the compiler does not insert inside inline assembly, checked on the gfx950
assembly generated from the kernel sources (no GPU needed; skipped without hipcc).

The compiler's hazard recognizer does not look inside assembly blocks, and it does not know
what an assembly block is: a block's own instruction gets no wait states from it, and neither
does a compiled instruction that follows a block.  The kernels have two kinds of block:

* LDS-direct tile loads (buffer_load_dwordx4 ... lds).  A vector memory instruction that reads
  an SGPR written by a VALU instruction (v_readlane, v_readfirstlane, ...) needs five wait states
  after that write, and an LDS-direct load needs one after M0 is written (AMD Instinct
  MI300/CDNA3 ISA reference, "Manually Inserted Wait States"; gfx950 keeps them).  The block
  carries the one wait state for M0; the kernels compute every SGPR operand with scalar
  instructions, and the scan checks that no VALU write of one precedes a load, under the
  default machine scheduler (the build's) and under iterative-ilp.  A reload of resource words
  from spill lanes (v_readlane) right before a load would need the five.
* v_permlane32_swap / v_permlane16_swap row exchanges (written as assembly because the builtin's
  two results were merged): 2 wait states after a VALU write of either operand, the wait this
  compiler inserts before the builtin.

The matrix products (v_mfma_*) are compiler builtins, so the compiler places their waits; the
scan holds them to the rules of the CDNA3 ISA reference's table of independent instructions
required between matrix (MAI) instructions and their dependents ("Dependency Resolution:
Required Independent Instructions") all the same, which guards against a product or an
accumulator move written as assembly later: a VALU write of a register (v_accvgpr_write and
v_accvgpr_mov included) needs 2 wait states before a matrix product reads it as a source, and a
matrix product's result needs 12 after a 32x32x16 product (8 after a 16x16 one) before a
vector instruction touches it (the numbers this compiler inserts for the same dependences on
gfx950; a dependent product that reads the result as its accumulator issues back to back, as
the same table allows).

The sources are compiled with the build's flags under the default machine scheduler and under
iterative-ilp; the scan counts wait states as s_nop N = N + 1 and any other instruction 1, along
the instruction order (the blocks that matter sit within one basic block of their dependents).
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


def _vregs(tok):
    """Vector registers an operand names, as ('v', n) / ('a', n): v5, v[4:7], a3, a[0:15]."""
    tok = tok.strip()
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m[1], n) for n in range(int(m[2]), int(m[3]) + 1)}
    m = re.fullmatch(r"([va])(\d+)", tok)
    return {(m[1], int(m[2]))} if m else set()


def _operands(ins):
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return []
    return [o.strip().split()[0] for o in parts[1].split(",") if o.strip()]


def _waits(ins):
    op = ins.split()[0]
    return int(ins.split()[1], 0) + 1 if op == "s_nop" else 1


def _is_valu(op):
    return op.startswith("v_") and not op.startswith("v_mfma")


MAI_SRC_WAIT = 2        # VALU write -> matrix product source read
SWAP_SRC_WAIT = 2       # VALU write -> v_permlane*_swap operand


def mai_result_wait(op):
    """Wait states after a matrix product before a vector instruction touches its result: 12 for
    the 32x32x16 shape, 8 for the 16x16 ones (16x16x32 bf16, 16x16x4 f32): the compiler's own
    waits for each on gfx950."""
    return 12 if "32x32" in op else 8


def source_read_violations(asm_text):
    """[(consumer, writer, wait states)]: a VALU instruction writing a register that a matrix
    product reads as a source (A, B or accumulator) fewer than MAI_SRC_WAIT wait states before
    it, or an operand of a permlane swap fewer than SWAP_SRC_WAIT before it; and the number of
    consumers seen."""
    ins = _instructions(asm_text)
    bad, seen = [], 0
    for i, cons in enumerate(ins):
        op = cons.split()[0]
        if op.startswith("v_mfma"):
            need, srcs = MAI_SRC_WAIT, set().union(*[_vregs(o) for o in _operands(cons)[1:]])
        elif op.startswith("v_permlane16_swap") or op.startswith("v_permlane32_swap"):
            need, srcs = SWAP_SRC_WAIT, set().union(*[_vregs(o) for o in _operands(cons)])
        else:
            continue
        seen += 1
        waits, j = 0, i - 1
        while j >= 0 and waits < need and srcs:
            prev = ins[j]
            j -= 1
            pop = prev.split()[0]
            ops = _operands(prev)
            dst = _vregs(ops[0]) if ops else set()
            if _is_valu(pop) and dst & srcs:
                bad.append((cons, prev, waits))
                srcs -= dst
            waits += _waits(prev)
    return bad, seen


def result_use_violations(asm_text):
    """[(product, user, wait states)]: a vector instruction other than a matrix product that
    reads or writes a register of a matrix product's result fewer than mai_result_wait wait
    states after it; and the number of products seen.  A later matrix product that takes the
    result as its accumulator (the back-to-back case) or rewrites it leaves the watch as is."""
    ins = _instructions(asm_text)
    bad, seen = [], 0
    for i, prod in enumerate(ins):
        if not prod.split()[0].startswith("v_mfma"):
            continue
        seen += 1
        dst = _vregs(_operands(prod)[0])
        need = mai_result_wait(prod.split()[0])
        waits, j = 0, i + 1
        while j < len(ins) and waits < need and dst:
            nxt = ins[j]
            j += 1
            op = nxt.split()[0]
            if _is_valu(op):
                used = set().union(*[_vregs(o) for o in _operands(nxt)])
                if used & dst:
                    bad.append((prod, nxt, waits))
                    dst -= used
            waits += _waits(nxt)
    return bad, seen


def _compile_asm(extra, out, source="prefill.hip"):
    b = _build_module()
    cmd = [b.hipcc(), *b.COMMON, *b.EXTRA.get(source, []), *extra, "-x", "hip",
           "--cuda-device-only", "-S", os.path.join(b.CSRC, source), "-o", out]
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


def test_lds_direct_loads_wait_for_their_operands(tmp_path):
    b = _build_module()
    try:
        b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    asm = _compile_asm([], str(tmp_path / "prefill.s"))
    bad, loads = lds_direct_violations(asm)
    # two D instantiations x (plain, handoff) x (prologue + loop) tiles of K and V loads
    assert loads >= 16, loads
    assert not bad, "\n".join(f"{w} ({n} wait states) before {l}" for l, w, n in bad[:8])


def test_lds_direct_loads_clean_under_iterative_ilp(tmp_path):
    """Under the iterative-ilp scheduler too, no VALU write of an SGPR operand precedes a load.
    An earlier kernel with 64-key tiles at 190 VGPRs did not pass this: that schedule reloaded
    resource words from spill lanes (v_readlane) right before the loads, which the scan reported
    (test_checker_flags_the_hazards plants the same pattern)."""
    b = _build_module()
    try:
        b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    asm = _compile_asm(["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
                       str(tmp_path / "prefill_ilp.s"))
    bad, loads = lds_direct_violations(asm)
    assert loads >= 16, loads
    assert not bad, "\n".join(f"{w} ({n} wait states) before {l}" for l, w, n in bad[:8])


def test_checker_flags_matrix_and_swap_hazards():
    """The scans themselves, on planted sequences: a register written by a VALU instruction
    (v_accvgpr_mov included) too close to a matrix product or a permlane swap that reads it,
    and a product's result touched too soon, are caught; enough wait states clear each."""
    close = ("v_accvgpr_mov_b32 a2, a66\n"
             "v_mfma_f32_32x32x16_bf16 v[34:49], v[2:5], a[0:3], 0\n")
    assert len(source_read_violations(close)[0]) == 1
    one = "v_cvt_pk_bf16_f32 v3, v8, v9\ns_nop 0\nv_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]\n"
    assert len(source_read_violations(one)[0]) == 1
    ok = "v_cvt_pk_bf16_f32 v3, v8, v9\ns_nop 1\nv_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]\n"
    assert source_read_violations(ok) == ([], 1)
    acc = "v_accvgpr_write_b32 a7, v1\nv_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]\n"
    assert len(source_read_violations(acc)[0]) == 1
    swap = "v_max_f32_e32 v7, v1, v2\nv_permlane32_swap_b32 v8, v7\n"
    assert len(source_read_violations(swap)[0]) == 1
    swap_ok = "v_max_f32_e32 v7, v1, v2\ns_nop 1\nv_permlane32_swap_b32 v8, v7\n"
    assert source_read_violations(swap_ok) == ([], 1)
    short = ("v_mfma_f32_32x32x16_bf16 v[34:49], v[2:5], a[0:3], 0\ns_nop 7\ns_nop 2\n"
             "v_max_f32_e32 v1, v34, v35\n")
    assert len(result_use_violations(short)[0]) == 1
    fenced = ("v_mfma_f32_32x32x16_bf16 v[34:49], v[2:5], a[0:3], 0\ns_nop 7\ns_nop 7\n"
              "v_max_f32_e32 v1, v34, v35\n")
    assert result_use_violations(fenced) == ([], 1)
    chained = ("v_mfma_f32_32x32x16_bf16 v[34:49], v[2:5], a[0:3], 0\n"
               "v_mfma_f32_32x32x16_bf16 v[34:49], v[6:9], a[4:7], v[34:49]\n"
               "s_nop 7\ns_nop 7\nv_max_f32_e32 v1, v34, v35\n")
    assert result_use_violations(chained) == ([], 2)
    read_acc = "v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]\ns_nop 3\nv_accvgpr_read_b32 v1, a4\n"
    assert len(result_use_violations(read_acc)[0]) == 1


@pytest.mark.parametrize("sched", ["default", "iterative-ilp"])
@pytest.mark.parametrize("source", ["prefill.hip", "decode.hip"])
def test_matrix_products_and_swaps_wait_for_their_operands(tmp_path, sched, source):
    b = _build_module()
    try:
        b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    extra = [] if sched == "default" else ["-mllvm", "-amdgpu-sched-strategy=" + sched]
    asm = _compile_asm(extra, str(tmp_path / "k.s"), source)
    # matrix products in all instantiations: prefill 64 32x32x16 (Q.K and P.V of both head
    # dims, plain and fused), decode 48 16x16x32; swaps add to the first count
    least = 64 if source == "prefill.hip" else 48
    bad, seen = source_read_violations(asm)
    assert seen >= least, seen
    assert not bad, "\n".join(f"{w} ({n} wait states) before {c}" for c, w, n in bad[:8])
    bad, seen = result_use_violations(asm)
    assert seen >= least, seen
    assert not bad, "\n".join(f"{u} ({n} wait states) after {p}" for p, u, n in bad[:8])
