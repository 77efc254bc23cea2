"""Build libbdattn.so (the C ABI plus its gfx950 kernels) in-tree with hipcc.

Run ``python -m block_masked_attention_amd.build`` (or call ``build()``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbdattn.so")
SOURCES = ["api.cpp", "plan.cpp", "kernels.hip", "kernels_dq_docs.hip", "kernels_dkdv.hip",
           "kernels_bwd_fused.hip", "lce.hip"]
HEADERS = ["bdattn_mask.h", "plan.h", "launch.h", "device.h"]
ROCM_LIB = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")

# Packed fp32 ops are disabled for all device code (hipcc -O3 would otherwise
# form them from plain float code).
HIP_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]
# Per-file machine-scheduler strategies, the fastest measured for each file's
# kernels: instruction-level parallelism for the key-tile backward kernels and
# the dQ kernel's packed-document variants (which the register-minimising
# schedule makes spill), the iterative register-minimising schedule for the
# other forward and dQ kernels (dQ 2.4% faster than with max-ilp at 256K).
_ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
_MINREG = ["-mllvm", "-amdgpu-sched-strategy=iterative-minreg"]
FILE_FLAGS = {"kernels.hip": _MINREG, "kernels_dq_docs.hip": _ILP, "kernels_dkdv.hip": _ILP,
              "kernels_bwd_fused.hip": _ILP}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the bdattn library needs ROCm's hipcc")


def _clean(out: str) -> str:
    return "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link libbdattn.so next to this
    file; return its path."""
    inc = ["-I", os.path.join(HERE, "..", "include")]
    with tempfile.TemporaryDirectory(prefix="bdattn_build_") as tmpdir:
        jobs = []
        for s in SOURCES:
            src = os.path.join(CSRC, s)
            obj = os.path.join(tmpdir, s + ".o")
            # hipcc treats .cpp as host C++ unless told otherwise; api.cpp and
            # plan.cpp only launch kernels through launch.h, so compile them as
            # HIP too.
            lang = ["-x", "hip"] if s.endswith(".cpp") else []
            cmd = [hipcc()] + HIP_FLAGS + FILE_FLAGS.get(s, []) + inc + ["-c"] + lang + [src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            jobs.append((s, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                  stderr=subprocess.STDOUT, text=True)))
        errors = []
        for s, obj, proc in jobs:
            out = _clean(proc.communicate()[0])
            if proc.returncode != 0:
                errors.append(f"{s}:\n{out}")
            elif verbose and out.strip():
                print(out)
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        tmp = LIB + ".tmp"
        # rocBLAS carries the linear cross-entropy's projections
        link = ([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + [o for _, o, _ in jobs] +
                ["-L", ROCM_LIB, "-Wl,-rpath," + ROCM_LIB, "-lrocblas", "-o", tmp])
        if verbose:
            print(" ".join(link), flush=True)
        res = subprocess.run(link, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + _clean(res.stdout + res.stderr))
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
