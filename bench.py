"""Benchmark: block-scaled FP8 GEMM on one MI355X.

Default workload: dense NT, M=4096, N=7168, K=2048, V3-shaped synthetic data
(A ~ N(0,1) with 0.1% outliers x50, B ~ N(0,0.02)), E4M3 with FP32 scales per
1x128 activation group and per 128x128 weight block, BF16 output.

One step = the whole hot path on one batch: the activation-scale transform
(dg_transform_sf: FP32 K-major -> MN-major) followed by the GEMM (persistent
tile scheduling, LDS staging, FP8 MFMA, per-128-K promotion, BF16 epilogue).
Inputs are resident in HBM before timing starts; each step uses the next of
several input/output buffer sets so no step reads data the previous step left
in the caches.  --workload picks the other workloads (grouped, decode, FP8 x FP4,
K-grouped, the activation cast).

Timing: W untimed warm-up steps, then exactly K timed steps between two device
synchronisations and nothing else on the stream (wall clock -> "value"; a timing
event between two kernels would make the queue drain first).  The dominant
kernel's launch duration comes from HIP events on the stream it is launched on,
right after the timed region: 5 runs of K back-to-back launches between two
events (mean, median and min of the runs' launch periods), or, for kernels
shorter than the binding's host time per call (decode, cast), a captured graph
of K launches replayed between two events.  After that a sustained run samples
the GPU clock and socket power with amd-smi, and a device-to-device copy of
1 GiB measures the practical HBM ceiling.

Prints one JSON line (see the "roofline" and "cpu_baseline" objects).
"""
import argparse
import json
import os
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
NOMINAL_SCLK_MHZ = 2400.0     # the clock the published peaks assume

WORKLOADS = {
    "dense_4096x7168x2048": dict(kind="dense", M=4096, N=7168, K=2048),
    "dense_64x7168x2048": dict(kind="dense", M=64, N=7168, K=2048, graph=True),
    "dense_c_4096x1536x7168": dict(kind="dense_c", M=4096, N=1536, K=7168),
    # the other operand layouts (A stored [K, M] for "t", B stored [K, N] for "n")
    "dense_nn_4096x7168x2048": dict(kind="dense", M=4096, N=7168, K=2048, layout="nn"),
    "dense_tn_4096x7168x2048": dict(kind="dense", M=4096, N=7168, K=2048, layout="tn"),
    "dense_tt_4096x7168x2048": dict(kind="dense", M=4096, N=7168, K=2048, layout="tt"),
    "masked_32x256x7168x2048": dict(kind="masked"),
    "contiguous_32x4096x7168": dict(kind="contig"),
    # the same with every group's weights stored [K, N] (m_grouped_fp8_gemm_nn_contiguous)
    "contiguous_nn_32x4096x7168": dict(kind="contig", layout="nn"),
    # FP8 activations x FP4 weights, contiguous groups (m_grouped_fp8_fp4_gemm_nt_contiguous)
    "fp8_fp4_contiguous_32x4096x7168": dict(kind="contig", fp4=True),
    "fp8_fp4_dense_4096x7168x2048": dict(kind="fp4_dense", M=4096, N=7168, K=2048),
    "fp8_fp4_masked_32x256x7168x2048": dict(kind="fp4_masked"),
    "cast_4096x7168_bf16": dict(kind="cast", M=4096, K=7168, graph=True),
    "cast_ue8m0_4096x7168_bf16": dict(kind="cast", M=4096, K=7168, ue8m0=True, graph=True),
    # MoE weight gradient: 8 experts' token counts (multiples of 128, 16384 in all) split K
    "k_grouped_8x7168x2048_k16384": dict(kind="k_grouped", M=7168, N=2048,
                                         ks=[1792, 2304, 2048, 1536, 2560, 2048, 1920, 2176]),
    # the same with token-major operands (A stored [sum ks, M], B stored [sum ks, N])
    "k_grouped_tn_8x7168x2048_k16384": dict(kind="k_grouped", M=7168, N=2048, layout="tn",
                                            ks=[1792, 2304, 2048, 1536, 2560, 2048, 1920, 2176]),
}
DEFAULT = "dense_4096x7168x2048"
HEADLINE_METRIC = "TFLOP/s + % FP8 MFMA peak, block-scaled FP8 GEMM M=4096 N=7168 K=2048"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
GEMM_SOURCES = ("dg_gemm.hip", "dg_gemm_pipe.hip", "dg_gemm_skinny.hip", "dg_internal.h")
CAST_SOURCES = ("dg_quant.hip", "dg_internal.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(sources=GEMM_SOURCES):
    """sha1 of the kernel sources with comments and whitespace removed (so an edit of a comment
    does not orphan the traffic figures taken from the same code)."""
    import hashlib
    import re
    h = hashlib.sha1()
    for f in sources:
        with open(os.path.join(ROOT, "block_scaled_fp8_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def sources_for(workload):
    """The kernel sources whose traffic a workload measures: the file of its dominant kernel
    (the cast, the decode kernel, the generic kernel for the K-grouped GEMM, the pipelined
    kernel for every other GEMM) and the shared header."""
    if workload.startswith("cast"):
        return CAST_SOURCES
    if workload.startswith("dense_64x"):
        return ("dg_gemm_skinny.hip", "dg_internal.h")
    if workload.startswith("k_grouped"):
        return ("dg_gemm.hip", "dg_internal.h")
    return ("dg_gemm_pipe.hip", "dg_internal.h")


def read_traffic(workload):
    """HBM bytes per launch of the timed kernel from the committed rocprofv3 counter summary
    (profiles/hbm_traffic.txt, written by profile_counters.py), or None if absent or taken from
    another kernel source than the current one."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        line = line.strip()
        if line and not line.startswith("#") and "=" in line:
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    key = f"{workload}.bytes_per_launch"
    if key not in vals or vals.get(f"{workload}.source_sha1") != kernel_source_hash(sources_for(workload)):
        return None
    return float(vals[key])


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return os.cpu_count()


class Workload:
    """What one benchmark line measures: step i is ``pre(i)`` (work queued before the dominant
    kernel, if any) then ``launch(i)`` (the dominant kernel) on the current stream; ``work``
    is the metric's numerator per step (FLOPs or bytes)."""

    def __init__(self, **kw):
        self.pre = None
        self.__dict__.update(kw)

    def step(self, i):
        if self.pre is not None:
            self.pre(i)
        self.launch(i)


# ---------------------------------------------------------------- workloads
def w_dense(spec, dg, dev):
    from tests import gen
    M, N, K = spec["M"], spec["N"], spec["K"]
    with_c = spec["kind"] == "dense_c"
    p = gen.dense(M, N, K, seed=0, with_c=with_c)
    out_dtype = torch.float32 if with_c else torch.bfloat16
    # buffer sets rotated through the steps: enough that one rotation moves at least 512 MiB, so
    # no step finds its operands in the 8 x 4 MB of L2 or the 256 MB of last-level cache (the
    # decode's 15.7 MB per set takes 35 sets); two for operands of 256 MiB and more
    set_bytes = M * K + N * K + (4 if with_c else 2) * M * N + (4 * M * N if with_c else 0)
    nsets = 2 if M * K + N * K >= 256 << 20 else max(8, min(64, -(-(512 << 20) // set_bytes)))
    layout = spec.get("layout", "nt")
    # operands as the layout stores them: A [K, M] for "t", B [K, N] for "n"
    a_st = p["a"] if layout[0] == "n" else np.ascontiguousarray(p["a"].T)
    b_st = p["b"] if layout[1] == "t" else np.ascontiguousarray(p["b"].T)
    gemm = getattr(dg, "fp8_gemm_" + layout)
    sets = []
    for _ in range(nsets):
        s = dict(a=torch.from_numpy(a_st).to(dev), b=torch.from_numpy(b_st).to(dev),
                 sa_raw=torch.from_numpy(p["sa"]).to(dev), sb=torch.from_numpy(p["sb"]).to(dev),
                 d=torch.empty((M, N), dtype=out_dtype, device=dev))
        s["sa"] = dg.get_mn_major_tma_aligned_tensor(s["sa_raw"])
        if with_c:
            s["c"] = torch.from_numpy(p["c"]).to(dev)
        sets.append(s)
    esz = 2 if out_dtype == torch.bfloat16 else 4
    sf_k = K // 128
    alg_bytes = M * K + N * K + 4 * M * sf_k + 4 * ((N + 127) // 128) * sf_k + esz * M * N + (4 * M * N if with_c else 0)
    flops = 2.0 * M * N * K

    def pre(i):
        # path A: the activation scales are transformed on every call, and the GEMM reads them
        s = sets[i % nsets]
        s["sa_step"] = dg.get_mn_major_tma_aligned_tensor(s["sa_raw"])

    def launch(i):
        s = sets[i % nsets]
        gemm((s["a"], s.get("sa_step", s["sa"])), (s["b"], s["sb"]), s["d"], c=s.get("c"))

    def cpu(seconds):
        import oracle
        rows = max(1, min(M, 64))

        def run_oracle(r):
            # the oracle on the operands as stored (rows 0..r-1 of D)
            a_rows = a_st[:r] if layout[0] == "n" else a_st[:, :r]
            t0 = time.perf_counter()
            oracle.gemm_layout(layout, a_rows, p["sa"][:r], b_st, p["sb"], 128, c=None if p["c"] is None else p["c"][:r])
            return time.perf_counter() - t0

        t = run_oracle(rows)
        if t < seconds / 4 and rows < M:
            rows = int(min(M, max(rows, rows * seconds / max(t, 1e-3))))
            rows = max(8, rows - rows % 8)
            t = run_oracle(rows)
        bound_work = 2.0 * rows * N * K if not spec.get("graph") else alg_bytes * rows / M
        return bound_work / t, t, f"rows 0..{rows - 1} of the {M}x{N}x{K} problem (all N columns, full K), float64 numpy"

    skinny = M <= 64
    kernel = "dg::skinny::skinny_kernel" if skinny else "dg::pipe::pipe_kernel"
    hbm = skinny
    return Workload(pre=pre, launch=launch, work=alg_bytes if hbm else flops, flops=flops, alg_bytes=alg_bytes,
                    bound="hbm" if hbm else "mfma", kernel=kernel, cpu=cpu,
                    config={"workload": None, "M": M, "N": N, "K": K, "out": "fp32+C" if with_c else "bf16",
                            "layout": layout, "scales": "fp32 1x128 act, 128x128 weight",
                            "step": "transform_sf(act scales) + gemm", "buffer_sets": nsets})


def w_masked(spec, dg, dev, fp4=False):
    from tests import gen
    import oracle
    if fp4:
        p = gen.fp8_fp4_grouped_masked(32, 256, 7168, 2048, seed=0)
    else:
        p = gen.config5()
    G, Mmax, N, K = 32, 256, 7168, 2048
    mm = torch.from_numpy(p["masked_m"]).to(dev)
    pk = (K // 128 + 3) // 4
    valid = int(np.clip(p["masked_m"], 0, Mmax).sum())
    active = int((p["masked_m"] > 0).sum())
    w_set = (N * K // 2 + 4 * N * (K // 128)) if fp4 else (N * K + 4 * N * pk)
    step_bytes = active * w_set + valid * (K + 4 * pk + 2 * N)
    # buffer sets rotated through the steps: one rotation moves at least 1 GiB, so a step's
    # weights (313 MB with FP4, 542 MB with FP8) are not found in the 256 MB last-level cache
    nsets = max(2, -(-(1 << 30) // step_bytes))
    sets = [dict(a=torch.from_numpy(p["a"]).to(dev), b=torch.from_numpy(p["b"]).to(dev),
                 d=torch.empty((G, Mmax, N), dtype=torch.bfloat16, device=dev)) for _ in range(nsets)]
    if fp4:
        sa = dg.transform_sf(torch.from_numpy(p["sa"]).to(dev), Mmax, 1, True)
        sb = dg.transform_sf(torch.from_numpy(p["sb"]).to(dev), N, 1, True)
        w_bytes = N * K // 2 + 4 * N * (K // 128)

        def launch(i):
            s = sets[i % nsets]
            dg.m_grouped_fp8_fp4_gemm_nt_masked((s["a"], sa), (s["b"], sb), s["d"], mm, expected_m=128)
    else:
        sa = dg.get_mn_major_tma_aligned_packed_ue8m0_tensor(torch.from_numpy(p["sa"]).to(dev))
        sb = dg.get_mn_major_tma_aligned_packed_ue8m0_tensor(torch.from_numpy(p["sb"]).to(dev), gran_mn=128, mn=N)
        w_bytes = N * K + 4 * N * pk

        def launch(i):
            s = sets[i % nsets]
            dg.m_grouped_fp8_gemm_nt_masked((s["a"], sa), (s["b"], sb), s["d"], mm, expected_m=128)
    alg_bytes = active * w_bytes + valid * (K + 4 * pk + 2 * N) + 4 * G
    flops = 2.0 * valid * N * K

    def cpu(seconds):
        gs = [g for g in range(G) if p["masked_m"][g] > 0][:4]
        t0 = time.perf_counter()
        for g in gs:
            m = int(p["masked_m"][g])
            if fp4:
                oracle.gemm_fp8_fp4_nt(p["a"][g, :m], p["sa"][g, :m], p["b"][g], p["sb"][g])
            else:
                oracle.gemm_nt(p["a"][g, :m], p["sa"][g, :m], p["b"][g], p["sb"][g], 128)
        t = time.perf_counter() - t0
        rows = int(sum(p["masked_m"][g] for g in gs))
        by = len(gs) * w_bytes + rows * (K + 4 * pk + 2 * N)
        return by / t, t, f"groups {gs} of the seed-0 draw ({rows} valid rows, their whole weights), float64 numpy"

    return Workload(launch=launch, work=alg_bytes, flops=flops, alg_bytes=alg_bytes, bound="hbm",
                    kernel="dg::pipe::pipe_kernel (masked)", cpu=cpu,
                    config={"workload": None, "groups": G, "m_max": Mmax, "N": N, "K": K, "valid_rows": valid,
                            "weights": "fp4 e2m1, ue8m0 per 1x32" if fp4 else "fp8 e4m3, ue8m0 per 128x128",
                            "scales": "ue8m0 packed x4, mn-major", "out": "bf16",
                            "step": "gemm (scales pre-packed, as the cast emits them)", "buffer_sets": nsets})


def w_contig(spec, dg, dev):
    from tests import gen
    import oracle
    fp4 = spec.get("fp4", False)
    p = gen.fp8_fp4_grouped_contiguous(32, 4096, 7168, seed=0) if fp4 else gen.config4()
    G, N, K = p["G"], p["N"], p["K"]
    a = torch.from_numpy(p["a"]).to(dev)
    b = torch.from_numpy(p["b"]).to(dev)
    if fp4:   # scales packed once (UE8M0), as the FP4 benchmark lines do
        sa = dg.transform_sf(torch.from_numpy(p["sa"]).to(dev), p["M"], 1, True)
        sb = dg.transform_sf(torch.from_numpy(p["sb"]).to(dev), N, 1, True)
    else:
        sa = dg.get_mn_major_tma_aligned_tensor(torch.from_numpy(p["sa"]).to(dev))
        sb = torch.from_numpy(p["sb"]).to(dev)
    lay = torch.from_numpy(p["layout"]).to(dev)
    flops = 2.0 * p["M"] * N * K
    if fp4:
        alg_bytes = G * N * K // 2 + p["M"] * K + 4 * p["M"] * ((K // 128 + 3) // 4) + 4 * G * N * (K // 128) \
            + 2 * p["M"] * N
    else:
        alg_bytes = G * N * K + p["M"] * K + 2 * p["M"] * N
    form = spec.get("layout", "nt")
    if form == "nn":
        b = b.transpose(1, 2).contiguous()   # [G, K, N]
    gemm = dg.m_grouped_fp8_fp4_gemm_nt_contiguous if fp4 else getattr(dg, f"m_grouped_fp8_gemm_{form}_contiguous")
    # buffer sets rotated through the steps: one rotation moves at least 1 GiB (FP8 weights: one
    # set, 1.24 GB per step; FP4 weights: two sets of 0.80 GB), past the 256 MB last-level cache
    nsets = max(1, -(-(1 << 30) // alg_bytes))
    sets = [dict(a=a, b=b, d=torch.empty((p["M"], N), dtype=torch.bfloat16, device=dev))]
    for _ in range(nsets - 1):
        sets.append(dict(a=a.clone(), b=b.clone(), d=torch.empty((p["M"], N), dtype=torch.bfloat16, device=dev)))

    def launch(i):
        s = sets[i % nsets]
        gemm((s["a"], sa), (s["b"], sb), s["d"], lay)

    def cpu(seconds):
        rows = np.arange(0, p["M"], max(1, p["M"] // 96))
        t0 = time.perf_counter()
        if fp4:
            oracle.grouped_contiguous_fp8_fp4(p["a"][rows], p["sa"][rows], p["b"], p["sb"], p["layout"][rows])
        elif form == "nn":
            oracle.grouped_contiguous_nn(p["a"][rows], p["sa"][rows], np.swapaxes(p["b"], 1, 2), p["sb"],
                                         p["layout"][rows])
        else:
            oracle.grouped_contiguous(p["a"][rows], p["sa"][rows], p["b"], p["sb"], p["layout"][rows])
        t = time.perf_counter() - t0
        return 2.0 * len(rows) * N * K / t, t, f"{len(rows)} evenly spaced rows (every group's weights), float64 numpy"

    return Workload(launch=launch, work=flops, flops=flops, alg_bytes=alg_bytes, bound="mfma",
                    kernel="dg::pipe::pipe_kernel (contiguous)", cpu=cpu,
                    config={"workload": None, "groups": G, "rows": p["M"], "N": N, "K": K, "out": "bf16",
                            "layout": form, "buffer_sets": nsets,
                            "scales": ("ue8m0 packed x4 (act per 1x128), fp4 e2m1 weights with ue8m0 per 1x32" if fp4
                                       else "fp32 1x128 act, 128x128 weight")})


def w_fp4_dense(spec, dg, dev):
    from tests import gen
    import oracle
    M, N, K = spec["M"], spec["N"], spec["K"]
    p = gen.fp8_fp4(M, N, K, seed=0)
    sets = []
    for _ in range(8):
        sets.append(dict(a=torch.from_numpy(p["a"]).to(dev), b=torch.from_numpy(p["b"]).to(dev),
                         sa=dg.transform_sf(torch.from_numpy(p["sa"]).to(dev), M, 1, True),
                         sb=dg.transform_sf(torch.from_numpy(p["sb"]).to(dev), N, 1, True),
                         d=torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
    flops = 2.0 * M * N * K
    alg_bytes = M * K + N * K // 2 + 4 * M * ((K // 128 + 3) // 4) + 4 * N * (K // 128) + 2 * M * N

    def launch(i):
        s = sets[i % len(sets)]
        dg.fp8_fp4_gemm_nt((s["a"], s["sa"]), (s["b"], s["sb"]), s["d"])

    def cpu(seconds):
        rows = 48
        t0 = time.perf_counter()
        oracle.gemm_fp8_fp4_nt(p["a"][:rows], p["sa"][:rows], p["b"], p["sb"])
        t = time.perf_counter() - t0
        return 2.0 * rows * N * K / t, t, f"rows 0..{rows - 1} of the {M}x{N}x{K} problem, float64 numpy"

    return Workload(launch=launch, work=flops, flops=flops, alg_bytes=alg_bytes, bound="mfma",
                    kernel="dg::pipe::pipe_kernel (fp4 weights)", cpu=cpu,
                    config={"workload": None, "M": M, "N": N, "K": K, "out": "bf16",
                            "weights": "fp4 e2m1, ue8m0 per 1x32", "scales": "ue8m0 packed x4 (act per 1x128)",
                            "step": "gemm (scales pre-packed)", "buffer_sets": len(sets)})


def w_k_grouped(spec, dg, dev):
    """The K-grouped GEMM of the MoE weight gradient, accumulating in place (C = D).  Both
    operands are N(0, 1) activations cast per 1x128 group by the library's cast, whose scale
    output is already the [sum ks / 128, mn] layout this GEMM takes."""
    import oracle
    M, N, ks = spec["M"], spec["N"], spec["ks"]
    K, G = sum(ks), len(ks)
    layout = spec.get("layout", "nt")
    gemm = getattr(dg, f"k_grouped_fp8_gemm_{layout}_contiguous")
    g = torch.Generator(device=dev).manual_seed(0)
    sets = []
    for _ in range(2):
        qa, sa = dg.per_token_group_cast_fp8(torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16))
        qb, sb = dg.per_token_group_cast_fp8(torch.randn((N, K), generator=g, device=dev).to(torch.bfloat16))
        if layout == "tn":   # token-major storage: [sum ks, M] and [sum ks, N]
            qa, qb = qa.t().contiguous(), qb.t().contiguous()
        sets.append(dict(a=qa, sa=sa.t(), b=qb, sb=sb.t(), d=torch.zeros((G, M, N), device=dev)))
    flops = 2.0 * M * N * K
    alg_bytes = M * K + N * K + 4 * (M + N) * (K // 128) + 2 * 4 * G * M * N

    def launch(i):
        s = sets[i % len(sets)]
        gemm((s["a"], s["sa"]), (s["b"], s["sb"]), s["d"], ks, s["d"])

    def cpu(seconds):
        rows = 256
        s = sets[0]
        sa = s["sa"][:, :rows].t().cpu().numpy()
        b, sb = s["b"].cpu().numpy(), s["sb"].t().cpu().numpy()
        c = np.zeros((G, rows, N), dtype=np.float32)
        if layout == "tn":   # the oracle on the operands as stored
            a = s["a"][:, :rows].cpu().numpy()
            t0 = time.perf_counter()
            oracle.k_grouped_tn(a, sa, b, sb, ks, c)
        else:
            a = s["a"][:rows].cpu().numpy()
            t0 = time.perf_counter()
            oracle.k_grouped(a, sa, b, sb, ks, c)
        t = time.perf_counter() - t0
        return 2.0 * rows * N * K / t, t, f"rows 0..{rows - 1} of A (all {G} groups, all of B), float64 numpy"

    return Workload(launch=launch, work=flops, flops=flops, alg_bytes=alg_bytes, bound="mfma",
                    kernel="K-grouped GEMM (one step = every group)", cpu=cpu,
                    config={"workload": None, "M": M, "N": N, "ks": ks, "layout": layout, "out": "fp32, C = D in place",
                            "scales": "fp32 1x128 on both operands", "buffer_sets": len(sets)})


def w_cast(spec, dg, dev):
    """The per-token-group FP8 cast of a BF16 activation matrix (the A operand of the dense
    workload before quantization); HBM-bound."""
    import oracle
    M, K = spec["M"], spec["K"]
    ue8m0 = spec.get("ue8m0", False)
    g = torch.Generator(device=dev).manual_seed(0)
    sf_bytes = 4 * (K // 512) if ue8m0 else 4 * (K // 128)
    alg_bytes = M * K * 2 + M * K + M * sf_bytes
    # input and output sets rotated through the steps: one rotation moves at least 1 GiB, so no
    # step finds its input in the 256 MB last-level cache
    nsets = max(8, -(-(1 << 30) // alg_bytes))
    xs = [torch.randn((M, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16) for _ in range(nsets)]
    outs = [dg.per_token_group_cast_fp8(xs[i], pack_ue8m0=ue8m0) for i in range(nsets)]

    def launch(i):
        dg.per_token_group_cast_fp8(xs[i % nsets], pack_ue8m0=ue8m0, out=outs[i % nsets])

    def cpu(seconds):
        x = xs[0][:256].float().cpu().numpy()
        t0 = time.perf_counter()
        oracle.per_token_group_cast(x, ue8m0=ue8m0)
        t = time.perf_counter() - t0
        return 256 * (K * 3 + sf_bytes) / t, t, "rows 0..255 of the BF16 input, numpy"

    return Workload(launch=launch, work=alg_bytes, flops=0.0, alg_bytes=alg_bytes, bound="hbm",
                    kernel=f"dg::cast_kernel<true, {'true' if ue8m0 else 'false'}>", cpu=cpu,
                    config={"workload": None, "M": M, "K": K, "scales": "ue8m0x4" if ue8m0 else "f32",
                            "buffer_sets": len(xs)})


BUILDERS = {"dense": w_dense, "dense_c": w_dense, "masked": w_masked, "contig": w_contig,
            "fp4_dense": w_fp4_dense, "fp4_masked": lambda s, dg, dev: w_masked(s, dg, dev, fp4=True),
            "k_grouped": w_k_grouped, "cast": w_cast}


# ---------------------------------------------------------------- measurement
def capture(fn, count):
    """A graph of ``count`` calls fn(0..count-1), captured on a side stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)                                          # (the first call outside the graph)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(count):
            fn(i)
    torch.cuda.synchronize()
    return g


def sample_clock_power():
    """(mean gfx clock over the XCDs in MHz, socket power in W) from amd-smi, or (None, None)."""
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-p", "--json"], capture_output=True, text=True,
                           timeout=20)
        j = json.loads(r.stdout[r.stdout.index("{"):])
        gd = j["gpu_data"][0] if "gpu_data" in j else j[0]
        clocks = [v["clk"]["value"] for k, v in gd["clock"].items() if k.startswith("gfx_") and isinstance(v, dict)
                  and isinstance(v.get("clk"), dict) and isinstance(v["clk"].get("value"), (int, float))]
        pw = gd["power"]["socket_power"]["value"]
        return (float(np.mean(clocks)) if clocks else None), (float(pw) if isinstance(pw, (int, float)) else None)
    except Exception as e:  # the tool is missing or its output differs: report nothing
        log("amd-smi sample failed:", repr(e)[:200])
        return None, None


def sustained_clock_power(run_some, seconds=2.0):
    """Keep the GPU busy with ``run_some()`` for about ``seconds`` while amd-smi samples it;
    the median of the samples taken while the work ran."""
    samples, stop = [], threading.Event()

    def sampler():
        time.sleep(0.3)
        while not stop.is_set():
            samples.append(sample_clock_power())

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds or (not samples and time.perf_counter() - t0 < 4 * seconds):
        run_some()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=30)
    clk = [c for c, _ in samples if c]
    pw = [p for _, p in samples if p]
    return (float(np.median(clk)) if clk else None), (float(np.median(pw)) if pw else None), len(samples)


def copy_ceiling_gbs(dev, mib=1024):
    """Read + write bytes per second of a plain 1 GiB device-to-device copy (best of 5)."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, 2.0 * src.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    torch.cuda.empty_cache()
    return best


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
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="after the warm-up steps, keep running untimed steps for this long so that the "
                         "timed region starts at the GPU's sustained clock (0: no settling)")
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the sustained clock/power sampling and the copy ceiling (profiler runs)")
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
    wl = BUILDERS[spec["kind"]](spec, dg, dev)
    wl.config["workload"] = args.workload
    K, W = args.steps, args.warmup
    stream = torch.cuda.current_stream()
    graph_mode = bool(spec.get("graph"))

    for i in range(W):
        wl.step(i)
    torch.cuda.synchronize()
    # Under sustained load the board's power control first pulls the shader clock well below
    # its steady value and settles within some 20 ms (a kernel trace of this benchmark shows
    # the GEMM at 62 us, then 74-77 us for a few ms, then back to 61-62 us): untimed steps
    # carry the GPU through that transient before the timed region starts.
    settled, t_settle = 0, time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(8):
            wl.step(W + settled)
            settled += 1
        torch.cuda.synchronize()
    copy_calibration(args, dev)

    if graph_mode:
        # the host needs longer per call than these kernels run: time captured graphs
        steps_graph = capture(wl.step, K)
        steps_graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        steps_graph.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        launch_graph = capture(wl.launch, K)
        periods = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch_graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            periods.append(e0.elapsed_time(e1) / K)
        kern_ms = dict(mean=float(np.mean(periods)), median=float(np.median(periods)), min=float(np.min(periods)),
                       how=f"graph of {K} launches replayed between two events, 5 replays")

        def run_some():
            launch_graph.replay()
    else:
        # the timed region holds the K steps and nothing else: a timing event between two
        # kernels makes the queue drain before the next one starts (about 6 us per event on
        # this GPU), which is instrumentation, not part of the job
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            wl.step(i)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        # the dominant kernel's own duration, live: HIP events on its stream around runs of K
        # back-to-back launches (the same buffer rotation as the steps), 5 runs
        periods = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(K):
                wl.launch(i)
            e1.record(stream)
            torch.cuda.synchronize()
            periods.append(e0.elapsed_time(e1) / K)
        kern_ms = dict(mean=float(np.mean(periods)), median=float(np.median(periods)), min=float(np.min(periods)),
                       how=f"HIP events around {K} back-to-back launches, 5 runs")

        def run_some():
            for i in range(20):
                wl.launch(i)

    ms_per_step = elapsed * 1e3 / K
    unit = "GB/s" if wl.bound == "hbm" else "TFLOP/s"
    scale = 1e9 if unit == "GB/s" else 1e12
    value = wl.work * K / elapsed / scale
    peak = PEAK_HBM_GBS if wl.bound == "hbm" else PEAK_FP8_TFLOPS
    achieved = wl.work / (kern_ms["mean"] * 1e-3) / scale

    extras = {}
    if not args.no_extras:
        sclk, power, nsamp = sustained_clock_power(run_some)
        extras["sclk_mhz"] = None if sclk is None else round(sclk, 1)
        extras["socket_power_w"] = power
        extras["clock_samples"] = nsamp
        extras["copy_ceiling_gbs"] = round(copy_ceiling_gbs(dev), 1)
    cpu = None
    if not args.no_cpu_baseline:
        v, secs, sample = wl.cpu(args.cpu_seconds)
        cpu = {"value": round(v / scale, 6), "unit": unit, "cores": blas_threads(), "kind": "oracle",
               "seconds": round(secs, 2), "sample": sample}

    roof = {"bound": wl.bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": read_traffic(args.workload),
            "kernel": wl.kernel, "kernel_ms_mean": round(kern_ms["mean"], 5),
            "kernel_ms_median": round(kern_ms["median"], 5), "kernel_ms_min": round(kern_ms["min"], 5),
            "frac_median": round(wl.work / (kern_ms["median"] * 1e-3) / scale / peak, 4),
            "timing": kern_ms["how"], "alg_bytes": wl.alg_bytes, "alg_flops": wl.flops}
    if extras.get("sclk_mhz"):
        roof["frac_at_observed_clock"] = round(achieved / (peak * extras["sclk_mhz"] / NOMINAL_SCLK_MHZ), 4) \
            if wl.bound != "hbm" else None
    if wl.bound == "hbm" and extras.get("copy_ceiling_gbs"):
        roof["frac_of_copy_ceiling"] = round(achieved / extras["copy_ceiling_gbs"], 4)
    out = {
        "metric": HEADLINE_METRIC if args.workload == DEFAULT else f"{unit}, {args.workload}",
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 x fp4_e2m1 (fp32 accumulate)" if "fp4" in spec["kind"] else
                 ("bf16 -> fp8_e4m3" if spec["kind"] == "cast" else "fp8_e4m3 (fp32 accumulate)"),
        "data": "synthetic",
        "config": wl.config,
        "roofline": roof,
        "cpu_baseline": cpu,
        "gpu": extras,
    }
    out["gpu"]["settle"] = {"ms": args.settle_ms, "untimed_steps": settled}
    if args.workload == DEFAULT:
        out["pct_fp8_peak"] = round(100.0 * value / PEAK_FP8_TFLOPS, 2)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
