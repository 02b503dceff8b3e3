"""Benchmark: block-scaled FP8 GEMM on one MI355X.

Default workload: dense NT, M=4096, N=7168, K=2048, V3-shaped synthetic data
(A ~ N(0,1) with 0.1% outliers x50, B ~ N(0,0.02)), E4M3 with FP32 scales per
1x128 activation group and per 128x128 weight block, BF16 output.

One step = the whole hot path on one batch: the activation-scale transform
(dg_transform_sf: FP32 K-major -> MN-major) followed by the GEMM (persistent
tile scheduling, LDS staging, FP8 MFMA, per-128-K promotion, BF16 epilogue).
Inputs are resident in HBM before timing starts; each step uses the next of
several input/output buffer sets (together larger than the 256 MB MALL) so no
step reads data the previous step left in cache.

Prints one JSON line (see the "roofline" and "cpu_baseline" objects).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published

WORKLOADS = {
    "dense_4096x7168x2048": dict(kind="dense", M=4096, N=7168, K=2048),
    "dense_64x7168x2048": dict(kind="dense", M=64, N=7168, K=2048),
    "dense_c_4096x1536x7168": dict(kind="dense_c", M=4096, N=1536, K=7168),
    "masked_32x256x7168x2048": dict(kind="masked"),
    "contiguous_32x4096x7168": dict(kind="contig"),
    "cast_4096x7168_bf16": dict(kind="cast", M=4096, K=7168),
    "cast_ue8m0_4096x7168_bf16": dict(kind="cast", M=4096, K=7168, ue8m0=True),
    # MoE weight gradient: 8 experts' token counts (multiples of 128, 16384 in all) split K
    "k_grouped_8x7168x2048_k16384": dict(kind="k_grouped", M=7168, N=2048,
                                         ks=[1792, 2304, 2048, 1536, 2560, 2048, 1920, 2176]),
}
DEFAULT = "dense_4096x7168x2048"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


GEMM_SOURCES = ("dg_gemm.hip", "dg_gemm_pipe.hip", "dg_internal.h")
CAST_SOURCES = ("dg_quant.hip", "dg_internal.h")


def read_traffic(workload, hash_key="kernel_source_sha1", sources=GEMM_SOURCES):
    """HBM bytes per launch of the timed kernel from the committed rocprofv3 counter summary,
    or None if absent or taken from an older kernel build."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        line = line.strip()
        if line and not line.startswith("#") and "=" in line:
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    key = f"{workload}.bytes_per_launch"
    src_hash = vals.get(hash_key)
    if key not in vals or src_hash != kernel_source_hash(sources):
        return None
    return float(vals[key])


def kernel_source_hash(sources=GEMM_SOURCES):
    import hashlib
    h = hashlib.sha1()
    for f in sources:
        with open(os.path.join(ROOT, "block_scaled_fp8_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def make_dense(spec, nsets, dev):
    from tests import gen
    M, N, K = spec["M"], spec["N"], spec["K"]
    p = gen.dense(M, N, K, seed=0, with_c=spec["kind"] == "dense_c")
    out_dtype = torch.float32 if spec["kind"] == "dense_c" else torch.bfloat16
    sets = []
    for _ in range(nsets):
        s = dict(a=torch.from_numpy(p["a"]).to(dev), b=torch.from_numpy(p["b"]).to(dev),
                 sa_raw=torch.from_numpy(p["sa"]).to(dev), sb=torch.from_numpy(p["sb"]).to(dev),
                 d=torch.empty((M, N), dtype=out_dtype, device=dev))
        if p["c"] is not None:
            s["c"] = torch.from_numpy(p["c"]).to(dev)
        sets.append(s)
    flops = 2.0 * M * N * K
    esz = 2 if out_dtype == torch.bfloat16 else 4
    sf_k = K // 128
    alg_bytes = M * K + N * K + 4 * M * sf_k + 4 * ((N + 127) // 128) * sf_k + esz * M * N
    if p["c"] is not None:
        alg_bytes += 4 * M * N
    return p, sets, flops, alg_bytes


def copy_calibration(args, dev):
    """One plain device copy of a known size: the reference that scales the FETCH_SIZE and
    WRITE_SIZE counters of the GEMM launches taken in the same profiler run."""
    if not args.copy_calibration_mb:
        return
    src = torch.empty(args.copy_calibration_mb << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size kernel that "
                         "calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the dense GEMM "
              "would shard along M or N with no exchange, the grouped forms by expert).", file=sys.stderr)
        sys.exit(2)

    import block_scaled_fp8_amd as dg
    dev = "cuda:0"
    torch.cuda.init()
    spec = WORKLOADS[args.workload]
    if spec["kind"] == "cast":
        return bench_cast(args, spec, dg, dev)
    if spec["kind"] == "k_grouped":
        return bench_k_grouped(args, spec, dg, dev)
    if spec["kind"] not in ("dense", "dense_c"):
        return bench_grouped(args, spec, dg, dev)

    p, sets, flops, alg_bytes = make_dense(spec, 8, dev)
    stream = torch.cuda.current_stream()
    M, N, K = spec["M"], spec["N"], spec["K"]

    def step(i, ev=None):
        s = sets[i % len(sets)]
        sa = dg.get_mn_major_tma_aligned_tensor(s["sa_raw"])
        if ev is not None:
            ev[0].record(stream)
        dg.fp8_gemm_nt((s["a"], sa), (s["b"], s["sb"]), s["d"], c=s.get("c"))
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    copy_calibration(args, dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    gemm_ms = [a.elapsed_time(b) for a, b in evs]
    gemm_avg_ms = float(np.mean(gemm_ms))
    ms_per_step = elapsed * 1e3 / args.steps
    value = flops * args.steps / elapsed / 1e12
    achieved = flops / (gemm_avg_ms * 1e-3) / 1e12
    traffic = read_traffic(args.workload)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_dense(p, args.cpu_seconds)

    out = {
        "metric": "TFLOP/s + % FP8 MFMA peak, block-scaled FP8 GEMM M=4096 N=7168 K=2048"
        if args.workload == DEFAULT else f"TFLOP/s, block-scaled FP8 GEMM {args.workload}",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic",
        "pct_fp8_peak": round(100.0 * value / PEAK_FP8_TFLOPS, 2),
        "config": {"workload": args.workload, "M": M, "N": N, "K": K,
                   "out": "fp32+C" if spec["kind"] == "dense_c" else "bf16",
                   "scales": "fp32 1x128 act, 128x128 weight",
                   "step": "transform_sf(act scales) + gemm", "buffer_sets": len(sets)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "traffic": traffic, "kernel": "dg::pipe::pipe_kernel (GEMM launch alone)",
                     "gemm_avg_ms": round(gemm_avg_ms, 5), "gemm_min_ms": round(float(np.min(gemm_ms)), 5),
                     "alg_bytes": alg_bytes, "alg_flops": flops},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_k_grouped(args, spec, dg, dev):
    """The K-grouped GEMM of the MoE weight gradient, accumulating in place (C = D).  Both
    operands are N(0, 1) activations cast per 1x128 group by the library's cast, whose scale
    output is already the [sum ks / 128, mn] layout this GEMM takes."""
    M, N, ks = spec["M"], spec["N"], spec["ks"]
    K, G = sum(ks), len(ks)
    g = torch.Generator(device=dev).manual_seed(0)
    sets = []
    for _ in range(2):
        qa, sa = dg.per_token_group_cast_fp8(torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16))
        qb, sb = dg.per_token_group_cast_fp8(torch.randn((N, K), generator=g, device=dev).to(torch.bfloat16))
        sets.append(dict(a=qa, sa=sa.t(), b=qb, sb=sb.t(), d=torch.zeros((G, M, N), device=dev)))
    flops = 2.0 * M * N * K
    alg_bytes = M * K + N * K + 4 * (M + N) * (K // 128) + 2 * 4 * G * M * N
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        s = sets[i % len(sets)]
        if ev is not None:
            ev[0].record(stream)
        dg.k_grouped_fp8_gemm_nt_contiguous((s["a"], s["sa"]), (s["b"], s["sb"]), s["d"], ks, s["d"])
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    copy_calibration(args, dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    avg = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        rows = 512
        s = sets[0]
        a = s["a"][:rows].cpu().numpy()
        sa = s["sa"][:, :rows].t().cpu().numpy()
        b, sb = s["b"].cpu().numpy(), s["sb"].t().cpu().numpy()
        c = np.zeros((G, rows, N), dtype=np.float32)
        t = time.perf_counter()
        oracle.k_grouped(a, sa, b, sb, ks, c)
        dt = time.perf_counter() - t
        cpu = {"value": round(2.0 * rows * N * K / dt / 1e12, 6), "unit": "TFLOP/s", "cores": os.cpu_count(),
               "kind": "oracle", "seconds": round(dt, 2),
               "sample": f"rows 0..{rows - 1} of A (all {G} groups, all of B), float64 numpy"}
    out = {
        "metric": f"TFLOP/s, K-grouped FP8 GEMM {args.workload}",
        "value": round(flops * args.steps / elapsed / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "N": N, "ks": ks, "out": "fp32, C = D in place",
                   "scales": "fp32 1x128 on both operands", "buffer_sets": len(sets)},
        "roofline": {"bound": "mfma", "achieved": round(flops / (avg * 1e-3) / 1e12, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(flops / (avg * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                     "traffic": read_traffic(args.workload),   # per step, like alg_bytes
                     "kernel": f"dg::gemm_kernel, {G} launches per step (one per group)",
                     "step_gpu_ms": round(avg, 5), "alg_bytes": alg_bytes, "alg_flops": flops},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_cast(args, spec, dg, dev):
    """The per-token-group FP8 cast of a BF16 activation matrix (the A operand of the dense
    workload before quantization); HBM-bound."""
    M, K = spec["M"], spec["K"]
    ue8m0 = spec.get("ue8m0", False)
    g = torch.Generator(device=dev).manual_seed(0)
    sets = [torch.randn((M, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16) for _ in range(8)]
    sf_bytes = 4 * (K // 512) if ue8m0 else 4 * (K // 128)   # per row: packed codes or FP32 scales
    alg_bytes = M * K * 2 + M * K + M * sf_bytes
    copy_calibration(args, dev)
    stream = torch.cuda.current_stream()
    # two output sets, allocated once and overwritten in turn
    outs = [dg.per_token_group_cast_fp8(sets[i], pack_ue8m0=ue8m0) for i in range(2)]
    for i in range(args.warmup):
        dg.per_token_group_cast_fp8(sets[i % len(sets)], pack_ue8m0=ue8m0, out=outs[i % 2])
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        dg.per_token_group_cast_fp8(sets[i % len(sets)], pack_ue8m0=ue8m0, out=outs[i % 2])
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = [a.elapsed_time(b) for a, b in evs]
    avg = float(np.mean(ms))
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        x = sets[0][:256].float().cpu().numpy()
        t = time.perf_counter()
        oracle.per_token_group_cast(x, ue8m0=ue8m0)
        dt = time.perf_counter() - t
        cpu = {"value": round(256 * (K * 3 + sf_bytes) / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "seconds": round(dt, 2), "sample": "rows 0..255 of the 4096x7168 BF16 input, numpy"}
    out = {
        "metric": f"GB/s, per-token-group FP8 cast {args.workload}",
        "value": round(alg_bytes * args.steps / elapsed / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16 -> fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "K": K, "buffer_sets": len(sets),
                   "scales": "ue8m0x4" if ue8m0 else "f32"},
        "roofline": {"bound": "hbm", "achieved": round(alg_bytes / (avg * 1e-3) / 1e9, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(alg_bytes / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": read_traffic(args.workload, "cast_source_sha1", CAST_SOURCES),
                     "kernel": f"dg::cast_kernel<true, {'true' if ue8m0 else 'false'}>", "avg_ms": round(avg, 5), "alg_bytes": alg_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_dense(p, seconds):
    """The float64 oracle, as it stands, on a bounded row sample of the same problem."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    M, N, K = p["M"], p["N"], p["K"]
    rows = min(64, M)
    t0 = time.perf_counter()
    oracle.gemm_nt(p["a"][:rows], p["sa"][:rows], p["b"], p["sb"], 128, c=None if p["c"] is None else p["c"][:rows])
    t = time.perf_counter() - t0
    if t < seconds / 4 and rows < M:
        rows = int(min(M, max(rows, rows * (seconds / max(t, 1e-3)))))
        rows = max(1, rows - rows % 8) if rows >= 8 else rows
        t0 = time.perf_counter()
        oracle.gemm_nt(p["a"][:rows], p["sa"][:rows], p["b"], p["sb"], 128,
                       c=None if p["c"] is None else p["c"][:rows])
        t = time.perf_counter() - t0
    fl = 2.0 * rows * N * K
    return {"value": round(fl / t / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(t, 2),
            "sample": f"rows 0..{rows - 1} of the {M}x{N}x{K} problem (all N columns, full K), float64 numpy"}


def bench_grouped(args, spec, dg, dev):
    from tests import gen
    stream = torch.cuda.current_stream()
    if spec["kind"] == "masked":
        p = gen.config5()
        G, Mmax, N, K = p["G"], p["M_max"], p["N"], p["K"]
        a = torch.from_numpy(p["a"]).to(dev)
        b = torch.from_numpy(p["b"]).to(dev)
        sa = dg.get_mn_major_tma_aligned_packed_ue8m0_tensor(torch.from_numpy(p["sa"]).to(dev))
        sb = dg.get_mn_major_tma_aligned_packed_ue8m0_tensor(torch.from_numpy(p["sb"]).to(dev), gran_mn=128, mn=N)
        mm = torch.from_numpy(p["masked_m"]).to(dev)
        d = torch.empty((G, Mmax, N), dtype=torch.bfloat16, device=dev)
        valid = int(np.clip(p["masked_m"], 0, Mmax).sum())
        pk = (K // 128 + 3) // 4
        active = int((p["masked_m"] > 0).sum())
        alg_bytes = active * (N * K + 4 * N * pk) + valid * (K + 4 * pk + 2 * N) + 4 * G
        flops = 2.0 * valid * N * K

        def launch():
            dg.m_grouped_fp8_gemm_nt_masked((a, sa), (b, sb), d, mm, expected_m=128)
        bound, peak, unit = "hbm", PEAK_HBM_GBS, "GB/s"
    else:
        p = gen.config4()
        G, N, K = p["G"], p["N"], p["K"]
        a = torch.from_numpy(p["a"]).to(dev)
        b = torch.from_numpy(p["b"]).to(dev)
        sa = dg.get_mn_major_tma_aligned_tensor(torch.from_numpy(p["sa"]).to(dev))
        sb = torch.from_numpy(p["sb"]).to(dev)
        lay = torch.from_numpy(p["layout"]).to(dev)
        d = torch.empty((p["M"], N), dtype=torch.bfloat16, device=dev)
        flops = 2.0 * p["M"] * N * K
        alg_bytes = G * N * K + p["M"] * K + 2 * p["M"] * N

        def launch():
            dg.m_grouped_fp8_gemm_nt_contiguous((a, sa), (b, sb), d, lay)
        bound, peak, unit = "mfma", PEAK_FP8_TFLOPS, "TFLOP/s"
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    copy_calibration(args, dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    avg_ms = e0.elapsed_time(e1) / args.steps
    if bound == "hbm":
        achieved = alg_bytes / (avg_ms * 1e-3) / 1e9
        value = alg_bytes * args.steps / elapsed / 1e9
    else:
        achieved = flops / (avg_ms * 1e-3) / 1e12
        value = flops * args.steps / elapsed / 1e12
    out = {"metric": f"{unit}, block-scaled FP8 GEMM {args.workload}", "value": round(value, 2), "unit": unit,
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(elapsed * 1e3 / args.steps, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "fp8_e4m3 (fp32 accumulate)", "data": "synthetic",
           "config": {"workload": args.workload, "tflops": round(flops / (avg_ms * 1e-3) / 1e12, 2)},
           "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                        "frac": round(achieved / peak, 4), "traffic": read_traffic(args.workload),
                        "avg_ms": round(avg_ms, 5), "alg_bytes": alg_bytes, "alg_flops": flops},
           "cpu_baseline": None}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
