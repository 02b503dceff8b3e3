"""Build libdg.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Usage: ``python -m block_scaled_fp8_amd.build`` or ``build()`` from Python.
The generic GEMM kernel file is compiled once per tile shape (``-DDG_TILE_ID=i``)
and the pipelined one once per part (``-DDG_PIPE_PART=i``) so the template
instantiations build in parallel, then everything is linked into
``block_scaled_fp8_amd/libdg.so``.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libdg.so")
NUM_TILES = 9
PIPE_PARTS = 4   # dg_gemm_pipe.hip: dense, contiguous, masked, FP4 weights

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed FP32 instructions are switched off for all device code.
FLAGS = ["-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError("build step failed: " + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def build(verbose=False, jobs=None):
    """Compile every HIP source for gfx950 and link libdg.so.  Always rebuilds."""
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    steps = []
    for t in range(NUM_TILES):
        steps.append([HIPCC, *FLAGS, f"-DDG_TILE_ID={t}", "-c", os.path.join(CSRC, "dg_gemm.hip"),
                      "-o", os.path.join(bdir, f"dg_gemm_t{t}.o")])
    steps.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, "dg_gemm.hip"),
                  "-o", os.path.join(bdir, "dg_gemm_dispatch.o")])
    # MFMA results in VGPRs: the block partials feed VALU promotion FMAs directly instead of
    # being copied out of accumulation registers (matters for the 4-wave tiles, whose
    # operands spill into AGPRs)
    for part in range(PIPE_PARTS):
        steps.append([HIPCC, *FLAGS, "-mllvm", "-amdgpu-mfma-vgpr-form", f"-DDG_PIPE_PART={part}", "-c",
                      os.path.join(CSRC, "dg_gemm_pipe.hip"), "-o", os.path.join(bdir, f"dg_gemm_pipe_p{part}.o")])
    steps.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, "dg_gemm_pipe.hip"),
                  "-o", os.path.join(bdir, "dg_gemm_pipe_dispatch.o")])
    steps.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, "dg_transform.hip"),
                  "-o", os.path.join(bdir, "dg_transform.o")])
    steps.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, "dg_quant.hip"),
                  "-o", os.path.join(bdir, "dg_quant.o")])
    steps.append([HIPCC, "-O2", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}", "-c", os.path.join(CSRC, "dg_api.cpp"),
                  "-o", os.path.join(bdir, "dg_api.o")])
    jobs = jobs or min(16, os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, steps):
            if verbose and out:
                print(out)
    objs = [s[-1] for s in steps]   # (stale objects left in _build are not linked)
    tmp = OUT + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


def clean():
    shutil.rmtree(os.path.join(HERE, "_build"), ignore_errors=True)
    if os.path.exists(OUT):
        os.remove(OUT)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
