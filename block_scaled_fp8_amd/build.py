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
PIPE_PARTS = 7   # dg_gemm_pipe.hip: dense, contiguous, masked, FP4 weights, MN-major A, B, both

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


# Pipelined instantiations that only a forced tile reaches (the planner never picks them):
# the 256-row tiles with FP32 + C output, which spill to scratch.
FORCED_ONLY = ("pipe_kernelILi256ELi224ELi4ELi2ELi0ELi2ELi0ELi2E", "pipe_kernelILi256ELi192ELi4ELi2ELi0ELi2ELi0ELi2E")


def parse_resource_usage(text):
    """Per-kernel figures from hipcc's -Rpass-analysis=kernel-resource-usage remarks."""
    import re
    rows, cur = [], None
    keys = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch", "SGPRs Spill": "sgpr_spill",
            "VGPRs Spill": "vgpr_spill", "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds"}
    for line in text.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            rows.append(cur)
            continue
        if cur is None:
            continue
        for k, short in keys.items():
            m = re.search(re.escape(k) + r": (\d+)", line)
            if m and short not in cur:
                cur[short] = int(m.group(1))
    return rows


def _check_scratch(reports):
    bad = [r["name"] for r in reports if r.get("scratch", 0) > 0 and not any(f in r["name"] for f in FORCED_ONLY)]
    if bad:
        raise RuntimeError("kernels the planner can pick use scratch memory (register spills): " + ", ".join(bad))


def build(verbose=False, jobs=None):
    """Compile every HIP source for gfx950 and link libdg.so.  Always rebuilds.  Fails if a
    GEMM kernel the planner can pick spills registers to scratch."""
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    steps = []
    for t in range(NUM_TILES):
        steps.append([HIPCC, *FLAGS, f"-DDG_TILE_ID={t}", "-Rpass-analysis=kernel-resource-usage", "-c",
                      os.path.join(CSRC, "dg_gemm.hip"), "-o", os.path.join(bdir, f"dg_gemm_t{t}.o")])
    steps.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, "dg_gemm.hip"),
                  "-o", os.path.join(bdir, "dg_gemm_dispatch.o")])
    # MFMA results in VGPRs: the block partials feed VALU promotion FMAs directly instead of
    # being copied out of accumulation registers (matters for the 4-wave tiles, whose
    # operands spill into AGPRs)
    for part in range(PIPE_PARTS):
        steps.append([HIPCC, *FLAGS, "-mllvm", "-amdgpu-mfma-vgpr-form", f"-DDG_PIPE_PART={part}",
                      "-Rpass-analysis=kernel-resource-usage", "-c",
                      os.path.join(CSRC, "dg_gemm_pipe.hip"), "-o", os.path.join(bdir, f"dg_gemm_pipe_p{part}.o")])
    steps.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, "dg_gemm_pipe.hip"),
                  "-o", os.path.join(bdir, "dg_gemm_pipe_dispatch.o")])
    steps.append([HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, "dg_gemm_skinny.hip"),
                  "-o", os.path.join(bdir, "dg_gemm_skinny.o")])
    steps.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, "dg_transform.hip"),
                  "-o", os.path.join(bdir, "dg_transform.o")])
    steps.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, "dg_quant.hip"),
                  "-o", os.path.join(bdir, "dg_quant.o")])
    steps.append([HIPCC, "-O2", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}", "-c", os.path.join(CSRC, "dg_api.cpp"),
                  "-o", os.path.join(bdir, "dg_api.o")])
    jobs = jobs or min(16, os.cpu_count() or 4)
    reports = []
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for step, out in zip(steps, ex.map(_run, steps)):
            if "-Rpass-analysis=kernel-resource-usage" in step:
                reports += parse_resource_usage(out)
            elif verbose and out:
                print(out)
    _check_scratch(reports)
    global LAST_RESOURCE_USAGE
    LAST_RESOURCE_USAGE = reports
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


LAST_RESOURCE_USAGE = []

_SF = {0: "1d2d FP32", 1: "1d1d FP32", 2: "UE8M0", 3: "FP4 weights"}
_OUT = {0: "BF16", 1: "FP32", 2: "FP32+C"}
_GRP = {0: "dense", 1: "contiguous", 2: "masked"}


_LAY = {0: "nt", 1: "A [K,M]", 2: "B [K,N]", 3: "A [K,M], B [K,N]"}


def resource_table(reports):
    """One line per GEMM instantiation: kernel, tile, waves, scales, output, operand storage,
    registers, scratch, occupancy and LDS."""
    import re
    lines = []
    for r in reports:
        regs = (f"VGPR {r.get('vgpr', 0):3d} AGPR {r.get('agpr', 0):3d} scratch {r.get('scratch', 0):3d} B/lane "
                f"SGPR spills {r.get('sgpr_spill', 0):2d} waves/SIMD {r.get('occupancy', 0)} LDS {r.get('lds', 0)}")
        m = re.search(r"pipe_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E", r["name"])
        if m:
            bm, bn, wm, wn, sf, out, grp, nb, lay = map(int, m.groups())
            forced = any(f in r["name"] for f in FORCED_ONLY)
            lines.append(f"pipelined {_GRP[grp]:10s} {bm}x{bn} {wm * wn} waves {_SF[sf]:11s} {_OUT[out]:6s} "
                         f"{_LAY[lay]:16s} B stages {nb}: {regs}" + ("   (forced tiles only)" if forced else ""))
            continue
        m = re.search(r"gemm_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E", r["name"])
        if m:
            bm, bn, wm, wn, sf, grp, out, lay = map(int, m.groups())
            sfn = {0: "1d2d FP32", 1: "1d1d FP32", 2: "UE8M0"}[sf]
            grn = {0: "dense", 1: "contiguous", 2: "masked", 3: "K-grouped"}[grp]
            lines.append(f"generic   {grn:10s} {bm}x{bn} {wm * wn} waves {sfn:11s} {_OUT[out]:6s} {_LAY[lay]:16s}"
                         f"           : {regs}")
            continue
        m = re.search(r"skinny_kernelILi(\d+)ELi(\d+)ELi(\d+)E", r["name"])
        if m:
            bn, nw, out = map(int, m.groups())
            lines.append(f"skinny    dense      <=64x{bn} {nw} waves 1d2d FP32   {_OUT[out]:6s} nt"
                         f"                          : {regs}")
    return lines


if __name__ == "__main__":
    build(verbose="--resource-report" not in sys.argv)
    if "--resource-report" in sys.argv:
        print("# Register, scratch, occupancy and LDS figures of every GEMM instantiation in libdg.so, from")
        print("# hipcc's -Rpass-analysis=kernel-resource-usage remarks (gfx950).  Made by:")
        print("#   python -m block_scaled_fp8_amd.build --resource-report")
        print("# The build fails if a kernel the planner can pick uses scratch (register spills).")
        print("\n".join(sorted(resource_table(LAST_RESOURCE_USAGE))))
    sys.exit(0)
