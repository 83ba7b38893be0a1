"""Occupancies the design relies on, checked against what the compiler reaches.

The decode planner's dispatch model assumes a number of resident decode workgroups per CU
for each head dimension (kDecodeResidentD64, kDecodeResidentD128 in csrc/moa_internal.h).
They must equal the occupancy the compiled decode kernels reach: the compiler reports it for
each kernel, in waves per SIMD, and a 256-thread workgroup puts one wave on each SIMD of a CU.
The bf16 prefill kernel is laid out for three workgroups per CU. Checked on the gfx950
assembly of the sources built with the build's flags (no GPU needed; skipped without hipcc)."""

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


def test_decode_residency_matches_compiled_occupancy(tmp_path):
    b = _build_module()
    try:
        b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = str(tmp_path / "decode.s")
    cmd = [b.hipcc(), *b.COMMON, *b.EXTRA.get("decode.hip", []), "-x", "hip",
           "--cuda-device-only", "-S", os.path.join(b.CSRC, "decode.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = open(out).read()
    with open(os.path.join(b.CSRC, "moa_internal.h")) as f:
        header = f.read()
    want = {d: int(re.search(rf"kDecodeResidentD{d} = (\d+);", header).group(1))
            for d in (64, 128)}
    # each kernel's label, then its "; Occupancy: N" summary line
    found = {}
    for m in re.finditer(r"^(_Z\S*decode_kernelILi(\d+)ELb([01])E\S*):", asm, re.M):
        occ = re.compile(r"^; Occupancy: (\d+)", re.M).search(asm, m.end())
        found[(int(m.group(2)), m.group(3))] = int(occ.group(1))
    assert set(found) == {(64, "0"), (64, "1"), (128, "0"), (128, "1")}, found
    for (d, _), occ in found.items():
        assert occ == want[d], (d, occ, want[d])


def test_prefill_runs_three_workgroups_per_cu(tmp_path):
    """The bf16 prefill kernel is laid out for three 256-thread workgroups per CU (32 KB of LDS
    and at most 168 VGPRs each: three waves on every SIMD), and its launch bounds ask for that.
    The plain and the fused-handoff kernels of both head dims must reach it: a source change
    that pushes the register count past 168 would silently drop it from three waves per SIMD
    to two."""
    b = _build_module()
    try:
        b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = str(tmp_path / "prefill.s")
    cmd = [b.hipcc(), *b.COMMON, *b.EXTRA.get("prefill.hip", []), "-x", "hip",
           "--cuda-device-only", "-S", os.path.join(b.CSRC, "prefill.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = open(out).read()
    found = {}
    for m in re.finditer(r"^(_Z\S*prefill_bf16_kernelILi(\d+)ELb([01])E\S*):", asm, re.M):
        occ = re.compile(r"^; Occupancy: (\d+)", re.M).search(asm, m.end())
        found[(int(m.group(2)), m.group(3))] = int(occ.group(1))
    assert set(found) == {(64, "0"), (64, "1"), (128, "0"), (128, "1")}, found
    for key, occ in found.items():
        assert occ >= 3, (key, occ)
