"""Benchmark of the fp8 a8w8 GEMM on one MI355X.

Headline: ptpc fp8 e4m3 GEMM, M=32768 N=7168 K=1792, bf16 out (the mori PR 785
gemm-only table's ptpc row, section Cost).  A step is one GEMM launch over
operands already resident in HBM: A quantised per token on the GPU
(quantize_per_token), B quantised per output channel and preshuffled once.
Inputs are seeded synthetic N(0,1) fp32 (A seed 31, B seed 32).

Prints ONE JSON line.  The roofline object reports the GEMM kernel's
algorithmic FLOPs per launch over its average launch time (HIP events on the
launch stream) against the fp8 dense MFMA peak; traffic comes from the
rocprofv3 FETCH_SIZE / WRITE_SIZE summaries under profiles/ when they were
taken for the current kernel, else null.  Two context objects follow the
timed run: mfma_ceiling, what the part sustains issuing nothing but the
GEMM's matrix instruction (one and two waves per SIMD, dmm_mfma_ceiling_fp8),
and vendor_baseline, the vendor library (hipBLASLt through torch._scaled_mm)
on the same codes and scales.  cpu_baseline is the CPU oracle
timed on a bounded row sample of the same workload; its result is also
compared with the GPU output of the timed run (the acceptance rule of
oracle.tolerance) and the statistics reported as cpu_baseline.parity.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--extra]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    # the part needs ~50-60 ms of load to climb from its idle clock to the
    # steady one: 500 headline launches (~155 ms) warm it up fully
    p.add_argument("--warmup", type=int, default=500)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--extra", action="store_true", help="also time the other modes and shapes")
    p.add_argument("--cpu-rows", type=int, default=32768,
                   help="rows of the headline the oracle computes (default: all of them)")
    p.add_argument("--calibrate", action="store_true",
                   help="also time every variant of the matrix-op calibration kernel (what each kind of "
                        "instruction interleaved with the matrix ops costs)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run a plain 1 GiB HBM copy kernel 3 times (the reference dispatch for "
                        "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return p.parse_args()


def timed(fn, steps, warmup, min_warm_s=0.0):
    """Average ms per call over ``steps`` back-to-back launches on the current
    stream (HIP events), after ``warmup`` launches -- and, with min_warm_s,
    after at least that much wall time of launches, so that the part has left
    its idle clock; synchronised both sides."""
    import torch

    t0 = time.perf_counter()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_warm_s:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def headline_operands(dmm, torch, m, n, k, seed_a, seed_b, mode="ptpc", keep_b=False):
    """Quantised operands on the GPU: (a codes, preshuffled b codes, a scale,
    b scale[, b codes in plain order when keep_b])."""
    from dense_matmul_amd import inputs

    a32 = torch.from_numpy(inputs.operand_a(m, k, seed_a)).to("cuda:0")
    b32 = torch.from_numpy(inputs.normal((n, k), seed_b)).to("cuda:0")
    if mode == "ptpc":
        qa, sa = dmm.quantize_per_token(a32)
        qb, sb = dmm.quantize_per_token(b32)
    elif mode == "blockscale":
        qa, sa = dmm.quantize_blockscale_a(a32)
        qb, sb = dmm.quantize_blockscale_b(b32)
    else:
        qa, sa = dmm.quantize_mxfp8(a32)
        qb, sb = dmm.quantize_mxfp8(b32)
    bs = dmm.preshuffle_b(qb)
    del a32, b32
    torch.cuda.synchronize()
    return (qa, bs, sa, sb, qb) if keep_b else (qa, bs, sa, sb)


COPY_BYTES = 1 << 30


def copy_calibration(torch):
    """A plain elementwise copy (negation) of COPY_BYTES of fp32, read once
    and written once, far larger than the last-level cache: its counters
    give bytes-per-counted-byte for FETCH_SIZE and WRITE_SIZE."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


KERNEL_SOURCES = ("gemm_a8w8.hip", "common.h", "kpipe.h", "lds_layout.h", "tile_order.h")


def kernel_source_hash():
    """sha256 over the fp8 GEMM kernel's source files, to tell whether a
    counter summary was taken for the kernel as it is now."""
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "dense_matmul_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_from_profiles(kernel_tag):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    profiles/<tag>_traffic.json, or None when there is none or it was taken
    for other kernel sources than the current ones."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("source_sha256") != kernel_source_hash():
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(m, n, k, rows_n, gpu_c=None):
    """The oracle, untouched, on ``rows_n`` evenly spaced rows of the headline
    workload (all of it by default) with every thread of this process's CPU
    share; returns TFLOP/s and the sample used.  With gpu_c (the GPU's bf16
    bits of the same workload), the oracle's rows are checked against it
    after the timing."""
    import numpy as np

    import oracle
    from dense_matmul_amd import inputs

    a = inputs.normal((m, k), 31)
    b = inputs.normal((n, k), 32)
    qa, sa = oracle.quantize_per_token(a)
    qb, sb = oracle.quantize_per_token(b)
    rows_n = min(rows_n, m)
    rows = np.linspace(0, m - 1, rows_n).astype(np.int64) if rows_n < m else None
    # every host thread of this process's CPU share (OMP_NUM_THREADS caps it
    # where the machine's count is larger than the share)
    threads = min(len(os.sched_getaffinity(0)), int(os.environ.get("OMP_NUM_THREADS", "0")) or 1 << 30)
    t0 = time.perf_counter()
    ref = oracle.gemm_ptpc(qa, qb, sa, sb, rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows_n * n * k
    res = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": (f"{rows_n} evenly spaced rows of {m}" if rows_n < m else f"all {m} rows") +
                     f" (all {n} columns, K={k}), GEMM only, {dt:.1f} s"}
    if gpu_c is not None:
        from oracle import tolerance

        got = gpu_c if rows is None else gpu_c[rows]
        try:
            st = tolerance.check(got, ref, "bench headline vs oracle", mode="ptpc", operands=(qa, qb, sa, sb),
                                 rows=rows)
            res["parity"] = {"rel_l2": st["rel_l2"], "elements": st["elements"], "max_err": st["max_err"],
                             "secondary": st["primary_fail"], "ok": True}
        except AssertionError as e:
            res["parity"] = {"ok": False, "error": str(e)[:200]}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import dense_matmul_amd as dmm

    dmm.lib()
    if args.copy_calibration:
        copy_calibration(torch)
    m, n, k = 32768, 7168, 1792
    qa, bs, sa, sb, qb = headline_operands(dmm, torch, m, n, k, 31, 32, keep_b=True)
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    ms = timed(lambda: dmm.gemm_a8w8_ptpc(qa, bs, sa, sb, out=out), args.steps, args.warmup)
    # context, measured right after the timed run (the part as warm as it was)
    ceiling = mfma_ceiling(dmm, torch, qa, all_variants=args.calibrate)
    vendor = vendor_baseline(torch, qa, qb, sa, sb, out, args.steps, args.warmup)
    gpu_c = None if args.no_cpu else out.view(torch.int16).cpu().numpy().view("uint16")
    flops = 2.0 * m * n * k
    tflops = flops / (ms * 1e-3) / 1e12
    rec = {
        "metric": "fp8 GEMM TFLOP/s + % of fp8 MFMA peak, ptpc 32768x7168x1792 (1 MI355X)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic N(0,1), seeds 31/32, quantised per token / per channel on the GPU",
        "config": {"workload": "ptpc fp8 GEMM M=32768 N=7168 K=1792", "mode": "ptpc", "m": m, "n": n, "k": k,
                   "pct_of_fp8_peak": round(100.0 * tflops / PEAK_FP8_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_FP8_TFLOPS, 4), "traffic": traffic_from_profiles("gemm_a8w8_ptpc")},
        "mfma_ceiling": dict(ceiling, value_over_one_wave_ceiling=round(
            tflops / ceiling["one_wave_per_simd_TFLOP/s"], 4)),
        "vendor_baseline": vendor,
    }
    del out, qb
    if args.extra:
        rec["extra"] = extra_shapes(dmm, torch, args)
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(m, n, k, args.cpu_rows, gpu_c)
    print(json.dumps(rec), flush=True)


def mfma_ceiling(dmm, torch, frag, all_variants=False, iters=1200, launches=100):
    """What the part sustains issuing nothing but the GEMM's matrix op:
    back-to-back independent fp8 16x16x128 ops on every SIMD, one and two
    waves per SIMD, operands taken from the headline's own A codes
    (dmm_mfma_ceiling_fp8).  With all_variants, also the mxfp8 form and the
    same stream with one kind of instruction interleaved after each op, one
    wave per SIMD.  TFLOP/s over HIP events on the launch stream."""
    out = torch.empty(1 << 20, dtype=torch.float32, device="cuda:0")

    def rate(wps, variant):
        flops = dmm.mfma_ceiling_fp8(frag, iters, wps, variant, out=out)[1]
        ms = timed(lambda: dmm.mfma_ceiling_fp8(frag, iters, wps, variant, out=out), launches, 10)
        return round(flops / (ms * 1e-3) / 1e12, 1)

    # the part's clock settles to a new load within a fraction of a second:
    # run the plain stream ~0.3 s before the first figure
    timed(lambda: dmm.mfma_ceiling_fp8(frag, iters, 1, "plain", out=out), 1000, 0)

    res = {"kind": "back-to-back independent fp8 16x16x128 matrix ops (calibration kernel)",
           "one_wave_per_simd_TFLOP/s": rate(1, "plain"), "two_waves_per_simd_TFLOP/s": rate(2, "plain")}
    if all_variants:
        res["one_wave_per_simd_variants_TFLOP/s"] = {
            v: rate(1, v) for v in ("plain", "scaled", "lds_read", "valu2", "acc_read", "acc_read16", "vmem_load",
                                    "lds_dma")}
        res["two_waves_per_simd_variants_TFLOP/s"] = {
            v: rate(2, v) for v in ("plain", "lds_read", "valu2", "acc_read", "acc_read16", "vmem_load", "lds_dma")}
    del out
    return res


def vendor_baseline(torch, qa, qb, sa, sb, ours, steps, warmup, min_warm_s=0.0):
    """The vendor library on the same codes and scales: torch._scaled_mm
    (hipBLASLt on ROCm) with per-row A and per-column B fp32 scales, bf16
    out, timed like the headline; its output is compared with this
    library's (relative L2 distance)."""
    lib = "hipBLASLt via torch._scaled_mm (per-row A / per-column B fp32 scales)"
    try:
        a8, b8 = qa.view(torch.float8_e4m3fn), qb.view(torch.float8_e4m3fn)
        sa2, sb2 = sa.view(-1, 1), sb.view(1, -1)

        def f():
            return torch._scaled_mm(a8, b8.t(), scale_a=sa2, scale_b=sb2, out_dtype=torch.bfloat16)

        ms = timed(f, steps, warmup, min_warm_s)
        c = f()
        m, k = qa.shape
        n = qb.shape[0]
        rel = ((c.float() - ours.float()).norm() / ours.float().norm()).item()
        del c
        return {"library": lib, "us": round(ms * 1e3, 1), "TFLOP/s": round(2.0 * m * n * k / (ms * 1e-3) / 1e12, 1),
                "rel_l2_vs_this_library": rel}
    except Exception as e:  # an unsupported _scaled_mm form leaves only the error in the line
        return {"library": lib, "error": f"{type(e).__name__}: {str(e)[:160]}"}


def extra_shapes(dmm, torch, args):
    """Secondary lines: the other scaling modes, the tail-only and gathered
    shapes, and the bf16 GEMM (fewer steps each)."""
    res = {}
    # short shapes: at least 150 ms of launches before timing (the clock ramp)
    steps, warm, warm_s = max(5, args.steps // 4), 20, 0.15
    for name, mode, m, n, k, sa_seed, sb_seed in [
        ("blockscale_16384x7168x2048", "blockscale", 16384, 7168, 2048, 41, 42),
        ("mxfp8_32768x7168x1792", "mxfp8", 32768, 7168, 1792, 31, 32),
        ("mxfp8_16384x7168x2048", "mxfp8", 16384, 7168, 2048, 41, 42),
        ("ptpc_4096x7168x256", "ptpc", 4096, 7168, 256, 11, 12),
        ("ptpc_16384x7168x512", "ptpc", 16384, 7168, 512, 21, 22),
        ("ptpc_gathered_32768x6288x7168", "ptpc", 32768, 6288, 7168, tuple(range(500, 508)), 510),
        ("ptpc_gathered_32768x3648x7168", "ptpc", 32768, 3648, 7168, tuple(range(500, 508)), 511),
        ("ptpc_2048x1168x1792", "ptpc", 2048, 1168, 1792, 61, 62),
    ]:
        qa, bs, sa, sb, qb = headline_operands(dmm, torch, m, n, k, sa_seed, sb_seed, mode, keep_b=True)
        out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
        fn = {"ptpc": dmm.gemm_a8w8_ptpc, "blockscale": dmm.gemm_a8w8_blockscale, "mxfp8": dmm.gemm_a8w8_mxfp8}[mode]
        ms = timed(lambda: fn(qa, bs, sa, sb, out=out), steps, warm, warm_s)
        tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        hbm = (m * k + n * k + 2 * m * n) / (ms * 1e-3) / 1e9
        res[name] = {"us": round(ms * 1e3, 1), "TFLOP/s": round(tf, 1), "pct_fp8_peak": round(100 * tf / PEAK_FP8_TFLOPS, 1),
                     "alg_GB/s": round(hbm, 0)}
        if mode == "ptpc":  # the vendor library has the per-row / per-column form only
            v = vendor_baseline(torch, qa, qb, sa, sb, out, steps, warm, warm_s)
            res[name]["vendor_us"] = v.get("us")
        del qa, bs, sa, sb, qb, out
        torch.cuda.empty_cache()
    from dense_matmul_amd import inputs

    # the quantisers (run before the GEMM, not in its time), on the configured
    # shapes' operands: algorithmic bytes = fp32 in + codes + scales
    for name, fn, rows, cols, extra_bytes in [
            ("quantize_per_token_32768x1792", dmm.quantize_per_token, 32768, 1792, lambda r, c: 4 * r),
            ("quantize_per_token_32768x7168", dmm.quantize_per_token, 32768, 7168, lambda r, c: 4 * r),
            ("quantize_per_token_7168x1792", dmm.quantize_per_token, 7168, 1792, lambda r, c: 4 * r),
            ("quantize_blockscale_a_16384x2048", dmm.quantize_blockscale_a, 16384, 2048, lambda r, c: 4 * r * c // 128),
            ("quantize_blockscale_b_7168x2048", dmm.quantize_blockscale_b, 7168, 2048,
             lambda r, c: 4 * ((r + 127) // 128) * (c // 128)),
            ("quantize_mxfp8_32768x1792", dmm.quantize_mxfp8, 32768, 1792, lambda r, c: r * c // 32),
            ("quantize_mxfp8_7168x1792", dmm.quantize_mxfp8, 7168, 1792, lambda r, c: r * c // 32)]:
        x = torch.from_numpy(inputs.normal((rows, cols), 3)).to("cuda:0")
        ms = timed(lambda: fn(x), 100, 20, warm_s)
        gbs = (5 * rows * cols + extra_bytes(rows, cols)) / (ms * 1e-3) / 1e9
        res[name] = {"us": round(ms * 1e3, 1), "alg_GB/s": round(gbs), "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 1)}
        del x
        torch.cuda.empty_cache()

    m, k, n = 4096, 1024, 896
    a32, b_kn = inputs.bf16_operands(m, k, n, 233)
    a = torch.from_numpy(a32).to(torch.bfloat16).to("cuda:0")
    b = torch.from_numpy(b_kn.T.copy()).to(torch.bfloat16).to("cuda:0")
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    ms = timed(lambda: dmm.gemm_bf16(a, b, out=out), 200, 20, warm_s)
    tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
    res["bf16_4096x1024x896"] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1),
                                 "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 1)}
    return res


if __name__ == "__main__":
    main()
