"""Build libmoa.so (gfx950) in the package directory with hipcc.

    python heterogeneous_sliding_windows_amd/build.py [-v] [--sanitize]

Run by file path (not as a module): the package itself refuses to import
until the library exists.
Every call recompiles all sources.  Objects go to _build/ at the repository
root; the shared library lands next to this file, where the binding loads it.

--sanitize builds a separate copy of the package under _build/sanitize/ whose
host code (the C ABI and the planner) carries AddressSanitizer and
UndefinedBehaviorSanitizer checks (device code is unchanged).  Load it into a
process with the ASan runtime preloaded (sanitizer_runtime() names it), e.g.
tests/test_sanitize.py.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoa.so")
ARCH = "gfx950"

SOURCES = ["moa_abi.cpp", "prefill.hip", "kv_append.hip", "decode.hip"]

COMMON = [
    "--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
    # no packed fp32 instructions: they are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# per-source extra flags: the span table needs IEEE double with no contraction
EXTRA = {"moa_abi.cpp": ["-ffp-contract=off"]}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoa)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # the host pass does not know the packed-fp32 feature; that note is harmless
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))


# host-side sanitizers only (each flag after -Xarch_host: the device code is not instrumented)
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer", "-g"]
SANITIZE_PKG = os.path.join(BUILD, "sanitize", "heterogeneous_sliding_windows_amd")


def sanitizer_runtime():
    """The ASan runtime (with the UBSan handlers) of this toolchain, to preload."""
    import glob
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not cands:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return cands[-1]


def build(verbose=False, sanitize=False):
    """Compile every source and link libmoa.so; with sanitize, the instrumented copy of the
    package (_build/sanitize/heterogeneous_sliding_windows_amd/).  Returns the library path."""
    cc = hipcc()
    bdir = os.path.join(BUILD, "sanitize") if sanitize else BUILD
    os.makedirs(bdir, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(bdir, src + ".o")
        cmd = [cc, *COMMON, *EXTRA.get(src, []), *(SANITIZE if sanitize else []), "-x", "hip",
               "-c", os.path.join(CSRC, src), "-o", obj]
        jobs.append((cmd, obj))
    with ThreadPoolExecutor(max_workers=min(len(jobs), 4)) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs))
    lib = LIB
    if sanitize:
        os.makedirs(SANITIZE_PKG, exist_ok=True)
        for f in ("__init__.py", "rules.py"):
            shutil.copy(os.path.join(PKG, f), os.path.join(SANITIZE_PKG, f))
        lib = os.path.join(SANITIZE_PKG, "libmoa.so")
    tmp = lib + ".tmp"
    _run([cc, "--offload-arch=" + ARCH, "-shared", "-fPIC",
          *(["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
            if sanitize else []),
          "-o", tmp, *[o for _, o in jobs]], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
