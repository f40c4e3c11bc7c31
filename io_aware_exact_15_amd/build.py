"""Builds libfa.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: python -m io_aware_exact_15_amd.build   (or __graft_entry__.build()).
Every call recompiles: objects go to _build/ at the repository root, the
shared library next to this file.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libfa.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["fa_fwd.hip", "fa_fwd_ws.hip", "fa_fwd_fp8.hip", "fa_bwd.hip", "fa_bwd_dq.hip", "fa_decode.hip", "fa_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    # The packed fp32 forms are kept out of the generated code on purpose.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]

# The dK/dV kernel is scheduled with the compiler's iterative ILP strategy
# (5 % faster than the default on the persistent kernel at N=16384, d=128);
# the dQ kernel, in a source of its own, keeps the default, under which it
# does not spill inside its loop.
PER_SOURCE = {"fa_bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


# The host compilation pass does not know the packed-fp32 feature named in
# FLAGS and says so once per translation unit; that notice is the only
# compiler output a clean build has.
_HOST_FEATURE_NOTICE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines() if line.strip() != _HOST_FEATURE_NOTICE)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False):
    """Compiles every source, links libfa.so, returns its path. `verbose` is
    kept for callers; diagnostics are always printed."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        # Kernel sources never rely on NaN propagation (masking uses -inf), so
        # fmaxf can map to v_max3_f32 without quieting each operand first. The
        # ABI file keeps full IEEE semantics for its argument checks.
        lang = ["-x", "hip", "-fno-honor-nans"] if src.endswith(".hip") else []
        out = _run([HIPCC, *FLAGS, *lang, *PER_SOURCE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        return obj, out.strip()

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(compile_one, srcs))
    objs = [obj for obj, _ in results]
    # Compiler diagnostics are printed, and any warning fails the build.
    noisy = [(src, out) for src, (_, out) in zip(srcs, results) if out]
    for src, out in noisy:
        print(f"--- {src}\n{out}", file=sys.stderr)
    if any("warning" in out for _, out in noisy):
        raise RuntimeError("the kernels compiled with warnings (printed above); fix them or state why they stay")
    tmp = OUT + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
