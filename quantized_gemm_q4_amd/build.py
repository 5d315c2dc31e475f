"""Build step for the HIP library: hipcc for gfx950 into
quantized_gemm_q4_amd/libq4amd.so (in-tree, so the built library travels
with the source tree)."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libq4amd.so")
ARCH = "gfx950"

# Kernels that turn floating point into integer codes (and the W8A8
# epilogue) are built without FMA contraction; every TU keeps IEEE-correct
# fp32 division and square root and no fast-math. Packed fp32 VALU forms are
# disabled on the device. Kernel arguments are preloaded into scalar
# registers (as many as fit the user SGPRs; the code object keeps a fallback
# that loads them itself), so a wavefront issues its first memory loads
# without waiting for a kernel-argument load: decode GEMV N = 11008 6.75 ->
# 6.23 us, batched decode 2-5% faster.
COMMON = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden",
          "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-kernarg-preload-count=16",
          "-Wall", "-Wno-unused-command-line-argument"]
SOURCES = {
    "abi.hip": [],
    "quantize.hip": ["-ffp-contract=off"],
    "w4a16.hip": ["-ffp-contract=off"],
    "w4a16_gemv.hip": ["-ffp-contract=off"],
    "w8a8.hip": ["-ffp-contract=off"],
    "mxfp4.hip": ["-ffp-contract=off"],
    "nf4.hip": ["-ffp-contract=off"],
    "nvfp4.hip": ["-ffp-contract=off"],
    "awq.hip": ["-ffp-contract=off"],
    "layernorm.hip": ["-ffp-contract=off"],
}


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every HIP source for gfx950 and link libq4amd.so."""
    hipcc = os.environ.get("HIPCC", "hipcc")
    with tempfile.TemporaryDirectory(prefix="q4build_") as tmp:
        procs, objs = [], []
        for src, extra in SOURCES.items():
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [hipcc, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
            if len([p for _, p in procs if p.poll() is None]) >= jobs:
                procs[0][1].wait()
        failed = False
        for src, p in procs:
            out, _ = p.communicate()
            lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
            if lines and (verbose or p.returncode):
                print("\n".join(lines), file=sys.stderr)
            if p.returncode:
                print(f"hipcc failed on {src}", file=sys.stderr)
                failed = True
        if failed:
            raise RuntimeError("HIP build failed")
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp_lib, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        # a kernel whose host launch stub went missing shows up as an undefined
        # library-internal symbol; fail here rather than at load time
        try:
            und = subprocess.run(["nm", "-D", "--undefined-only", tmp_lib], check=True,
                                 capture_output=True, text=True).stdout
        except (OSError, subprocess.CalledProcessError):
            und = ""
        missing = [ln.split()[-1] for ln in und.splitlines() if "q4k" in ln]
        if missing:
            os.remove(tmp_lib)
            raise RuntimeError("HIP build left undefined internal symbols: " + ", ".join(missing))
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
