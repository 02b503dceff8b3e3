"""rocprofv3 summaries of one bench.py workload, written to profiles/.

    python profile_counters.py <workload> [--outdir DIR] [--passes trace,pmc1,pmc2,l2,fetch,write]

Runs bench.py under rocprofv3 once per pass (this script never touches the GPU itself; each
pass is a child process with python3 right after rocprofv3's "--"):
  trace : --kernel-trace --stats                    -> duration of every kernel
  pmc1  : MFMA busy, busy CU cycles, wave cycles, wait cycles, active VALU/LDS, MFMA count
  pmc2  : instruction counts by kind, LDS bank conflicts and LDS active cycles
  l2    : L2 (TCC) hits and misses
  fetch : FETCH_SIZE, write : WRITE_SIZE (HBM traffic, calibrated by a plain 512 MiB copy
          that bench.py runs in the same process)
and writes profiles/<workload>_<pass group>.txt: the commands, the raw per-dispatch means
of the dominant kernel, and the derived figures.  Raw profiler output stays in --outdir.
"""
import argparse
import csv
import glob
import hashlib
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
NUM_CU = 256
SIMDS_PER_CU = 4
XCDS = 8

PASSES = {
    "pmc1": "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_WAVE_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_ANY "
            "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_INSTS_MFMA GRBM_GUI_ACTIVE",
    "pmc2": "SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_SALU SQ_INSTS_VMEM SQ_INSTS_SMEM SQ_LDS_BANK_CONFLICT "
            "SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS GRBM_GUI_ACTIVE",
    "l2": "TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE",
    "fetch": "FETCH_SIZE",
    "write": "WRITE_SIZE",
}
# the dominant kernel of each workload (a substring of its name)
KERNEL = {
    "dense_4096x7168x2048": "pipe_kernel", "dense_c_4096x1536x7168": "pipe_kernel",
    "dense_64x7168x2048": "skinny_kernel", "masked_32x256x7168x2048": "pipe_kernel",
    "contiguous_32x4096x7168": "pipe_kernel", "fp8_fp4_dense_4096x7168x2048": "pipe_kernel",
    "fp8_fp4_masked_32x256x7168x2048": "pipe_kernel", "cast_4096x7168_bf16": "cast_kernel",
    "cast_ue8m0_4096x7168_bf16": "cast_kernel", "k_grouped_8x7168x2048_k16384": "gemm_kernel",
    "dense_nn_4096x7168x2048": "pipe_kernel", "dense_tn_4096x7168x2048": "pipe_kernel",
    "dense_tt_4096x7168x2048": "pipe_kernel", "k_grouped_tn_8x7168x2048_k16384": "gemm_kernel",
    "contiguous_nn_32x4096x7168": "pipe_kernel", "fp8_fp4_contiguous_32x4096x7168": "pipe_kernel",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
TRAFFIC_HEADER = """# HBM traffic of the timed kernel launch from rocprofv3 counters, one MI355X.
# Per workload, two runs of one counter each (written by profile_counters.py):
#   rocprofv3 --pmc FETCH_SIZE -f csv -d <out> -o run -- python3 bench.py --workload <w> --steps 5 --warmup 2 --settle-ms 0 --no-cpu-baseline --no-extras --copy-calibration-mb 512
#   rocprofv3 --pmc WRITE_SIZE -f csv -d <out> -o run -- python3 bench.py --workload <w> --steps 5 --warmup 2 --settle-ms 0 --no-cpu-baseline --no-extras --copy-calibration-mb 512
# Calibration: the same runs copy 512 MiB device-to-device once (a kernel of known traffic,
#   512 MiB read and 512 MiB written); its counter reading gives the bytes per counter KiB.
# Bytes = counter KiB x 1024 x factor.  <w>.source_sha1 ties a workload's figures to the kernel
# sources they were taken from (bench.py's kernel_source_hash); bench.py reports traffic as null
# when the current sources differ.
"""


def source_hash(workload):
    sys.path.insert(0, ROOT)
    from bench import kernel_source_hash, sources_for
    return kernel_source_hash(sources_for(workload))


def run_source_hash(workload, outdir, no_run):
    """The kernel-source hash of the run whose output is summarised: recorded in --outdir when
    the passes run, read back from there by --no-run (the sources may have changed since)."""
    f = os.path.join(outdir, f"{workload}_source_sha1.txt")
    if no_run and os.path.exists(f):
        return open(f).read().strip()
    sha = source_hash(workload)
    if not no_run:
        with open(f, "w") as fh:
            fh.write(sha + "\n")
    return sha


def update_traffic_file(workload, res, sha):
    """Replace the workload's lines in profiles/hbm_traffic.txt (other workloads are kept)."""
    keep = []
    if os.path.exists(TRAFFIC_FILE):
        for line in open(TRAFFIC_FILE):
            t = line.strip()
            if t and not t.startswith("#") and "=" in t and not t.startswith(workload + "."):
                keep.append(t)
    keep.append(f"{workload}.source_sha1 = {sha}")
    for k, name in (("FETCH_SIZE", "fetch_kib_per_launch"), ("WRITE_SIZE", "write_kib_per_launch")):
        if k in res:
            keep.append(f"{workload}.{name} = {res[k]:.0f}")
    for k, name in (("fetch_factor", "fetch_factor"), ("write_factor", "write_factor")):
        if k in res:
            keep.append(f"{workload}.{name} = {res[k]:.4f}")
    keep.append(f"{workload}.read_bytes_per_launch = {res.get('FETCH_SIZE_bytes', 0.0):.0f}")
    keep.append(f"{workload}.write_bytes_per_launch = {res.get('WRITE_SIZE_bytes', 0.0):.0f}")
    keep.append(f"{workload}.bytes_per_launch = {res['bytes_per_launch']:.0f}")
    with open(TRAFFIC_FILE, "w") as f:
        f.write(TRAFFIC_HEADER + "\n".join(sorted(keep, key=lambda x: x.split(".")[0])) + "\n")


def bench_args(workload):
    return ["python3", os.path.join(ROOT, "bench.py"), "--workload", workload, "--steps", "5", "--warmup", "2",
            "--settle-ms", "0", "--no-cpu-baseline", "--no-extras", "--copy-calibration-mb", "512"]


def pass_command(name, d, workload):
    if name == "trace":
        prof = ["rocprofv3", "--kernel-trace", "--stats", "-f", "csv", "-d", d, "-o", "run"]
    else:
        prof = ["rocprofv3", "--pmc", *PASSES[name].split(), "-f", "csv", "-d", d, "-o", "run"]
    return prof + ["--"] + bench_args(workload)


def run_pass(name, workload, outdir):
    d = os.path.join(outdir, f"{workload}_{name}")
    cmd = pass_command(name, d, workload)
    t0 = time.time()
    env = dict(os.environ, TMPDIR="/tmp")
    with open(d + ".log", "w") as log:
        r = subprocess.run(["timeout", "-k", "10", "240", *cmd], stdout=log, stderr=subprocess.STDOUT, cwd="/tmp",
                           env=env)
    print(f"[profile] {workload} {name}: rc {r.returncode} in {time.time() - t0:.0f} s", flush=True)
    # (rocprofv3 can end with a segmentation fault after the program finished: use the files if complete)
    return " ".join(cmd).replace(ROOT + "/", ""), d


def read_counters(d, kernel):
    """Per-dispatch counter values of the dispatches whose name contains ``kernel``, averaged."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        return None, 0
    per = {}
    for row in csv.DictReader(open(files[0])):
        if kernel not in row.get("Kernel_Name", ""):
            continue
        per.setdefault(row["Dispatch_Id"], {})[row["Counter_Name"]] = float(row["Counter_Value"])
    if not per:
        return None, 0
    names = set().union(*[set(v) for v in per.values()])
    means = {n: sum(v.get(n, 0.0) for v in per.values()) / len(per) for n in names}
    return means, len(per)


def read_copy_calibration(d):
    """Counter reading of the 512 MiB calibration copy in the same pass: bench.py runs it right
    after the warm-up steps, so it is the last copy dispatch (the input uploads come earlier)."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    last, val = -1, None
    for row in csv.DictReader(open(files[0])) if files else []:
        if "copy" in row.get("Kernel_Name", "").lower():
            i = int(row["Dispatch_Id"])
            if i > last:
                last, val = i, float(row["Counter_Value"])
    return val


def read_trace(d):
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    return list(csv.DictReader(open(files[0]))) if files else []


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workload")
    ap.add_argument("--outdir", default=os.path.join(ROOT, "gpurun_out", "profile"))
    ap.add_argument("--passes", default="trace,pmc1,pmc2,l2,fetch,write")
    ap.add_argument("--no-run", action="store_true", help="only summarise the output of an earlier run in --outdir")
    args = ap.parse_args()
    os.makedirs(args.outdir, exist_ok=True)
    kernel = KERNEL[args.workload]
    passes = args.passes.split(",")
    sha = run_source_hash(args.workload, args.outdir, args.no_run)
    out = [f"# rocprofv3 summary: bench.py --workload {args.workload}, one MI355X ({NUM_CU} CUs)",
           f"# kernel source sha1 (bench.py's kernel_source_hash for this workload) = {sha}",
           f"# made by: python profile_counters.py {args.workload} --passes {args.passes}", ""]
    res = {}
    for name in passes:
        if args.no_run:
            d = os.path.join(args.outdir, f"{args.workload}_{name}")
            cmd = " ".join(pass_command(name, d, args.workload)).replace(ROOT + "/", "")
        else:
            cmd, d = run_pass(name, args.workload, args.outdir)
        out.append(f"## {name}: {cmd}")
        if name == "trace":
            rows = read_trace(d)
            out.append(f"{'kernel':70s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} {'max us':>9s}")
            for r in rows[:8]:
                out.append(f"{r['Name'][:70]:70s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                           f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f}")
            out.append("")
            continue
        vals, nd = read_counters(d, kernel)
        if vals is None:
            out.append("(no dispatches of the kernel found)\n")
            continue
        res.update(vals)
        out.append(f"dispatches of *{kernel}*: {nd}; mean per dispatch:")
        for k in sorted(vals):
            out.append(f"  {k} = {vals[k]:.6g}")
        if name in ("fetch", "write"):
            cal = read_copy_calibration(d)
            if cal:
                factor = (512 * 1024 if name == "fetch" else 512 * 1024) / cal
                key = "FETCH_SIZE" if name == "fetch" else "WRITE_SIZE"
                res[key + "_bytes"] = vals.get(key, 0.0) * 1024 * factor
                res[name + "_factor"] = factor
                out.append(f"  calibration copy of 512 MiB read {cal:.6g} KiB -> {factor:.4f} bytes per counter byte; "
                           f"{key} = {res[key + '_bytes'] / 1e6:.2f} MB per dispatch")
        out.append("")
    # derived figures
    g = res.get("GRBM_GUI_ACTIVE")
    der = []
    if g and "SQ_VALU_MFMA_BUSY_CYCLES" in res:
        # GRBM_GUI_ACTIVE is summed over the XCDs: GRBM_GUI_ACTIVE / XCDS is the kernel's cycles
        der.append(f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {XCDS} * {NUM_CU} CUs * "
                   f"{SIMDS_PER_CU} SIMDs) = {res['SQ_VALU_MFMA_BUSY_CYCLES'] / (g / XCDS * NUM_CU * SIMDS_PER_CU):.3f}")
        if res.get("SQ_INSTS_MFMA"):
            der.append(f"  (SQ_VALU_MFMA_BUSY_CYCLES / SQ_INSTS_MFMA = "
                       f"{res['SQ_VALU_MFMA_BUSY_CYCLES'] / res['SQ_INSTS_MFMA']:.1f} busy cycles per MFMA)")
    if "SQ_WAVE_CYCLES" in res and res["SQ_WAVE_CYCLES"]:
        for k in ("SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS"):
            if k in res:
                der.append(f"{k} / SQ_WAVE_CYCLES = {res[k] / res['SQ_WAVE_CYCLES']:.3f}")
    if "SQ_LDS_BANK_CONFLICT" in res and res.get("SQ_LDS_IDX_ACTIVE"):
        der.append(f"LDS bank conflict cycles / LDS active cycles = "
                   f"{res['SQ_LDS_BANK_CONFLICT'] / res['SQ_LDS_IDX_ACTIVE']:.4f}")
    if "SQ_INSTS_MFMA" in res and res["SQ_INSTS_MFMA"]:
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM"):
            if k in res:
                der.append(f"{k} per MFMA = {res[k] / res['SQ_INSTS_MFMA']:.3f}"
                           + ("  (SQ_INSTS_VALU counts the MFMAs too)" if k == "SQ_INSTS_VALU" else ""))
    h, m = res.get("TCC_HIT_sum"), res.get("TCC_MISS_sum")
    if h is not None and m is not None and h + m > 0:
        der.append(f"L2 hit rate = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum) = {h / (h + m):.3f}")
    if "FETCH_SIZE_bytes" in res or "WRITE_SIZE_bytes" in res:
        fb, wb = res.get("FETCH_SIZE_bytes", 0.0), res.get("WRITE_SIZE_bytes", 0.0)
        der.append(f"HBM bytes per dispatch: read {fb / 1e6:.2f} MB + written {wb / 1e6:.2f} MB = {(fb + wb) / 1e6:.2f} MB")
        res["bytes_per_launch"] = fb + wb
    if der:
        out.append("## derived (per dispatch of the dominant kernel)")
        out += ["  " + x for x in der]
    tag = "kernel_trace" if passes == ["trace"] else "counters"
    for base in (os.path.join(ROOT, "profiles"), args.outdir):   # (the copy in outdir travels back)
        os.makedirs(base, exist_ok=True)
        path = os.path.join(base, f"{args.workload}_{tag}.txt")
        with open(path, "w") as f:
            f.write("\n".join(out) + "\n")
        print(f"[profile] wrote {path}", flush=True)
    if "FETCH_SIZE_bytes" in res and "WRITE_SIZE_bytes" in res:
        update_traffic_file(args.workload, res, sha)
        print(f"[profile] {args.workload}.bytes_per_launch = {res['bytes_per_launch']:.0f} -> {TRAFFIC_FILE}", flush=True)


if __name__ == "__main__":
    sys.exit(main())
