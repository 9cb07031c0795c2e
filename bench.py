"""Benchmark of the fp8 a8w8 GEMM on one MI355X.

Headline: ptpc fp8 e4m3 GEMM, M=32768 N=7168 K=1792, bf16 out (the mori PR 785
gemm-only table's ptpc row, section Cost).  A step is one GEMM launch over
operands already resident in HBM: A quantised per token on the GPU
(quantize_per_token), B quantised per output channel and preshuffled once.
Inputs are seeded synthetic N(0,1) fp32 (A seed 31, B seed 32).

Timing protocol (DeepGEMM PR 453, Performance Overhead: the median per-call
time over 9 batches; mori PR 785, Cost: an idle box, the arms alternating,
the minimum over 3 passes):
  * the device and its activity before the run are recorded (an idle check);
  * warm-up: --warmup launches and at least WARM_S seconds of launches, so the
    part has left its idle clock whatever the launch count;
  * `steps` back-to-back launches are captured once in a HIP graph and the
    graph is replayed 9 times, in 3 passes of 3 replays, each pass followed by
    the vendor library's 3 batches of `steps` launches (the arms alternate);
    each batch is bracketed by a device synchronisation and timed with HIP
    events on the launch stream;
  * ms_per_step is the median per-call time of the 9 batches (min and max
    beside it, and the minimum of the 3 per-pass medians);
  * a secondary cold figure: one launch right after a 1 GiB scrub write, the
    median of 9.

Prints ONE JSON line.  The roofline object reports the GEMM kernel's
algorithmic FLOPs per launch over that per-call time against the fp8 dense
MFMA peak; traffic comes from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary
under profiles/ when it was taken for the current kernel sources, else null.
Context objects follow the timed run: mfma_ceiling, what the part sustains
issuing nothing but the GEMM's matrix instruction (the calibration library
libdmm_calib.so, not part of libdmm), and vendor_baseline (hipBLASLt through
torch._scaled_mm) on the same codes and scales.  cpu_baseline is the CPU
oracle timed on the headline (all rows by default); its result is also
compared with the GPU output of the timed run under the acceptance rule of
oracle.tolerance and the statistics are reported as cpu_baseline.parity.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--extra] [--calibrate]
       python bench.py --workload NAME [--steps K] [--warmup W]   (one workload, eager
           launches, for profilers; NAME from dense_matmul_amd.inputs.WORKLOADS)
"""
import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
# the part needs ~50-60 ms of load to climb from its idle clock to the
# steady one; every timed workload first gets at least this much
WARM_S = 0.3
BATCHES, PASSES = 9, 3
SCRUB_BYTES = 1 << 30


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200, help="launches per timed batch (graph)")
    p.add_argument("--warmup", type=int, default=20,
                   help="untimed launches before timing (at least WARM_S seconds of launches run regardless)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--extra", action="store_true", help="also time the other modes and shapes")
    p.add_argument("--cpu-rows", type=int, default=32768,
                   help="rows of the headline the oracle computes (default: all of them)")
    p.add_argument("--calibrate", action="store_true",
                   help="also time every variant of the matrix-op calibration kernel (what each kind of "
                        "instruction interleaved with the matrix ops costs) and the per-CU load and store rates")
    p.add_argument("--no-ceiling", action="store_true", help="skip the calibration-kernel context")
    p.add_argument("--workload", default=None,
                   help="run only this workload (a key of dense_matmul_amd.inputs.WORKLOADS, or a quantiser of "
                        "QUANTISERS, PRESHUFFLES): --warmup then --steps eager launches, one short JSON line; for rocprofv3")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run a plain 1 GiB HBM copy kernel 3 times (the reference dispatch for "
                        "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return p.parse_args()


# ------------------------------------------------------------------ timing
def warm(fn, launches, min_s):
    """``launches`` launches, then more until at least ``min_s`` seconds of
    launches have run; synchronised.  Returns the wall seconds spent."""
    import torch

    t0 = time.perf_counter()
    for _ in range(launches):
        fn()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_s:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    return time.perf_counter() - t0


def event_ms(run, calls):
    """Per-call ms of one batch: ``run()`` issues ``calls`` launches on the
    current stream, bracketed by device synchronisations and HIP events."""
    import torch

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    run()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / calls


def capture(fn, steps):
    """A HIP graph of ``steps`` back-to-back launches of fn (fn allocates
    nothing: it writes a caller buffer)."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager call on the side stream before capture
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            fn()
    torch.cuda.synchronize()
    return g


def repeat(fn, n):
    for _ in range(n):
        fn()


def summary(vals):
    return {"median": statistics.median(vals), "min": min(vals), "max": max(vals)}


def timed_arms(arms, steps, warmup, min_s, batches=BATCHES, passes=PASSES):
    """Time several arms (name -> fn) with the protocol of the module
    docstring: each arm warmed, captured as a graph of ``steps`` launches
    (or, with ``eager`` in the name, issued eagerly), then ``passes`` passes
    in which each arm in turn runs batches/passes batches.  Returns name ->
    {median, min, max, pass_min (the least per-pass median), batches_ms,
    warm_s} in ms per call."""
    runs, res = {}, {}
    for name, fn in arms.items():
        res[name] = {"warm_s": round(warm(fn, warmup, min_s), 3)}
        if name.endswith("eager"):
            runs[name] = lambda fn=fn: repeat(fn, steps)
        else:
            g = capture(fn, steps)
            runs[name] = g.replay
    per = {name: [[] for _ in range(passes)] for name in arms}
    for p in range(passes):
        for name in arms:
            for _ in range(batches // passes):
                per[name][p].append(event_ms(runs[name], steps))
    for name in arms:
        flat = [v for pv in per[name] for v in pv]
        res[name].update(summary(flat))
        res[name]["pass_min"] = min(statistics.median(pv) for pv in per[name])
        res[name]["batches_ms"] = [round(v, 5) for v in flat]
    return res


def cold_ms(fn, reps=BATCHES):
    """One launch right after a 1 GiB scrub write (the operands leave the
    caches, the clock stays up): median, min, max per-call ms over reps."""
    import torch

    scrub = torch.empty(SCRUB_BYTES // 4, dtype=torch.float32, device="cuda:0")
    vals = []
    for i in range(reps):
        scrub.fill_(float(i))
        vals.append(event_ms(fn, 1))
    del scrub
    torch.cuda.empty_cache()
    return summary(vals)


# ----------------------------------------------------------------- context
def device_record():
    """The device, the software stack and the GPU's activity before the run
    (amdsmi when importable)."""
    import torch

    p = torch.cuda.get_device_properties(0)
    rec = {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
           "hbm_GiB": round(p.total_memory / 2**30, 1), "torch": torch.__version__, "hip": torch.version.hip}
    try:
        import amdsmi

        amdsmi.amdsmi_init()
        try:
            h = amdsmi.amdsmi_get_processor_handles()[0]
            act = amdsmi.amdsmi_get_gpu_activity(h)
            rec["idle_check"] = {"gfx_activity_pct": act.get("gfx_activity"),
                                 "umm_activity_pct": act.get("umc_activity")}
            try:
                rec["idle_check"]["processes"] = len(amdsmi.amdsmi_get_gpu_process_list(h))
            except Exception:
                pass
            try:
                clk = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
                rec["max_sclk_MHz"] = clk.get("max_clk")
            except Exception:
                pass
        finally:
            amdsmi.amdsmi_shut_down()
    except Exception as e:  # no management library: record why
        rec["idle_check"] = {"error": f"{type(e).__name__}: {str(e)[:100]}"}
    return rec


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


KERNEL_SOURCES = ("gemm_a8w8.hip", "common.h", "kpipe.h", "lds_layout.h", "tile_order.h", "b_layout.h")


def code_text(src):
    """C++ source text without its comments and blank space: what a compiler
    sees, so that editing a comment does not make a profile stale."""
    import re

    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash():
    """sha256 over the fp8 GEMM kernel's source files (code_text of each),
    to tell whether a counter summary was taken for the kernel as it is
    now."""
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "dense_matmul_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
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


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


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
    tq = time.perf_counter()
    qa, sa = oracle.quantize_per_token(a)
    qb, sb = oracle.quantize_per_token(b)
    tq = time.perf_counter() - tq
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
                     f" (all {n} columns, K={k}), GEMM only, {dt:.1f} s",
           "cpu_model": cpu_model(),
           # the quantisation of both operands, timed apart from the GEMM (one thread)
           "quantize": {"s": round(tq, 3), "GB/s": round((m + n) * k * 5 / tq / 1e9, 2), "threads": 1}}
    if gpu_c is not None:
        from oracle import tolerance

        got = gpu_c if rows is None else gpu_c[rows]
        try:
            st = tolerance.check(got, ref, "bench headline vs oracle", mode="ptpc", operands=(qa, qb, sa, sb),
                                 rows=rows)
            res["parity"] = {"rel_l2": st["rel_l2"], "elements": st["elements"], "max_err": st["max_err"],
                             "primary_fail": st["primary_fail"], "secondary_cap": st["secondary_cap"], "ok": True}
        except AssertionError as e:
            res["parity"] = {"ok": False, "error": str(e)[:200]}
    return res


# ------------------------------------------------------------ calibration
CALIB_LIB = os.path.join(ROOT, "dense_matmul_amd", "calib", "libdmm_calib.so")
CALIB_VARIANTS = {"plain": 0, "scaled": 1, "lds_read": 2, "valu2": 3, "acc_read": 4, "acc_read16": 5,
                  "vmem_load": 6, "lds_dma": 7, "w32_plain": 8, "w32_lds_read": 9, "w32_vmem_load": 10,
                  "w32_lds_dma": 11}
_calib = None


def calib_lib():
    """libdmm_calib.so (the benchmark's matrix-op calibration kernel)."""
    global _calib
    if _calib is None:
        if not os.path.exists(CALIB_LIB):
            raise ImportError(f"{CALIB_LIB} is not built")
        # torch first: the library must bind to the HIP runtime torch loads
        # (the same soname), not bring in a second copy that finds no device
        import torch  # noqa: F401

        L = ctypes.CDLL(CALIB_LIB)
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        L.calib_mfma_ceiling_fp8.argtypes = [P, I64, P, I64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.POINTER(ctypes.c_int), P]
        L.calib_mfma_ceiling_fp8.restype = ctypes.c_int
        L.calib_memory_rate.argtypes = [P, I64, I64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
        L.calib_memory_rate.restype = ctypes.c_int
        L.calib_last_error.argtypes = []
        L.calib_last_error.restype = ctypes.c_char_p
        _calib = L
    return _calib


def mfma_ceiling_fp8(frag, iters, waves_per_simd=1, variant="plain", out=None):
    """One launch of the calibration kernel on e4m3 codes ``frag`` (at least
    2 MiB); returns (out, FLOPs of the launch)."""
    import torch

    fb = frag.view(torch.uint8)
    if out is None:
        out = torch.empty(1 << 20, dtype=torch.float32, device=frag.device)
    wg = ctypes.c_int(0)
    L = calib_lib()
    st = L.calib_mfma_ceiling_fp8(ctypes.c_void_p(fb.data_ptr()), fb.numel(), ctypes.c_void_p(out.data_ptr()),
                                  out.numel(), int(iters), int(waves_per_simd), CALIB_VARIANTS[variant],
                                  ctypes.byref(wg), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        raise (ValueError if st == 1 else RuntimeError)(L.calib_last_error().decode())
    return out, 2.0 * 16 * 16 * 128 * 16 * int(iters) * wg.value * 4 * int(waves_per_simd)


def mfma_ceiling(torch, frag, all_variants=False, iters=1200, launches=50):
    """What the part sustains issuing nothing but the GEMM's matrix op:
    back-to-back independent fp8 16x16x128 ops on every SIMD, one and two
    waves per SIMD, operands taken from the headline's own A codes.  With
    all_variants, also the mxfp8 form, the 32x32x64 op, and each with one
    kind of instruction interleaved.  TFLOP/s over HIP events on the launch
    stream (eager launches, each batch after a short warm-up)."""
    out = torch.empty(1 << 20, dtype=torch.float32, device="cuda:0")

    def rate(wps, variant):
        flops = mfma_ceiling_fp8(frag, iters, wps, variant, out=out)[1]
        fn = lambda: mfma_ceiling_fp8(frag, iters, wps, variant, out=out)
        warm(fn, 5, 0.02)
        ms = event_ms(lambda: repeat(fn, launches), launches)
        return round(flops / (ms * 1e-3) / 1e12, 1)

    warm(lambda: mfma_ceiling_fp8(frag, iters, 1, "plain", out=out), 0, WARM_S)
    res = {"kind": "back-to-back independent fp8 16x16x128 matrix ops (calibration kernel)",
           "one_wave_per_simd_TFLOP/s": rate(1, "plain"), "two_waves_per_simd_TFLOP/s": rate(2, "plain")}
    if all_variants:
        res["one_wave_per_simd_variants_TFLOP/s"] = {v: rate(1, v) for v in CALIB_VARIANTS}
        res["two_waves_per_simd_variants_TFLOP/s"] = {v: rate(2, v) for v in CALIB_VARIANTS if v != "scaled"}
    del out
    return res


MEMORY_KINDS = {"loads_vgpr": 0, "loads_lds": 1, "stores_lines": 2, "stores_epilogue": 3}


def memory_rate(torch, buf, region, kind, nt_sc1=False, grid=None, iters=256, launches=5):
    """Per-CU rate of one kind of 1 KiB vector-memory instruction (the
    calibration library's memory-rate kernel): each of ``grid`` workgroups
    (default: one per CU) streams through its own ``region`` bytes of
    ``buf``.  Returns (bytes per shader cycle per CU from the workgroups'
    s_memtime, aggregate TB/s from HIP events), from the last of
    ``launches`` launches after one warm-up."""
    L = calib_lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = cus if grid is None else grid
    cyc = torch.zeros(2 * grid, dtype=torch.int64, device=buf.device)
    st = torch.cuda.current_stream().cuda_stream

    def run():
        e = L.calib_memory_rate(ctypes.c_void_p(buf.data_ptr()), buf.numel(), int(region), int(iters),
                                MEMORY_KINDS[kind], int(nt_sc1), int(grid), ctypes.c_void_p(cyc.data_ptr()),
                                ctypes.c_void_p(st))
        if e != 0:
            raise (ValueError if e == 1 else RuntimeError)(L.calib_last_error().decode())

    run()
    ms = event_ms(lambda: repeat(run, launches), launches)
    c = cyc.view(grid, 2).cpu()
    cycles = float((c[:, 1] - c[:, 0]).double().mean())
    per_cu = 4.0 * iters * 16 * 1024
    return round(per_cu / cycles, 1), round(per_cu * grid / (ms * 1e-3) / 1e12, 2)


def memory_calibration(torch):
    """Loads and stores per CU and in aggregate (1 KiB instructions, sixteen
    in flight per wave): loads from a region per CU that the L2 holds
    (64 KiB), one that only the last-level cache holds (256 KiB: 8 MiB per
    XCD), and one streamed from HBM (4 MiB); stores of whole lines and in the
    fp8 GEMM's epilogue pattern, default and non-temporal device-scope
    policy, on every CU and on one CU per XCD."""
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    buf.fill_(1)
    res = {"unit": "[bytes per shader cycle per CU, aggregate TB/s]",
           "kind": "calibration kernel: 4 waves per CU, 1 KiB per instruction, 16 in flight per wave"}
    for kind in ("loads_vgpr", "loads_lds"):
        for name, region in (("L2_64KiB_per_CU", 64 << 10), ("MALL_256KiB_per_CU", 256 << 10), ("HBM_4MiB_per_CU", 4 << 20)):
            res[f"{kind}_{name}"] = memory_rate(torch, buf, region, kind)
    for kind in ("stores_lines", "stores_epilogue"):
        for nt in (False, True):
            pol = "nt_sc1" if nt else "default"
            res[f"{kind}_{pol}_all_CUs"] = memory_rate(torch, buf, 4 << 20, kind, nt_sc1=nt)
            res[f"{kind}_{pol}_8_CUs"] = memory_rate(torch, buf, 4 << 20, kind, nt_sc1=nt, grid=8)
    del buf
    torch.cuda.empty_cache()
    return res


def vendor_fn(torch, qa, qb, sa, sb):
    """torch._scaled_mm (hipBLASLt on ROCm) on the same codes, per-row A and
    per-column B fp32 scales, bf16 out."""
    a8, b8 = qa.view(torch.float8_e4m3fn), qb.view(torch.float8_e4m3fn)
    sa2, sb2 = sa.view(-1, 1), sb.view(1, -1)
    return lambda: torch._scaled_mm(a8, b8.t(), scale_a=sa2, scale_b=sb2, out_dtype=torch.bfloat16)


VENDOR = "hipBLASLt via torch._scaled_mm (per-row A / per-column B fp32 scales)"


# -------------------------------------------------------------------- main
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
    if args.workload:
        run_workload(dmm, torch, args.workload, args.steps, args.warmup)
        return
    device = device_record()
    m, n, k = 32768, 7168, 1792
    flops = 2.0 * m * n * k
    qa, bs, sa, sb, qb = headline_operands(dmm, torch, m, n, k, 31, 32, keep_b=True)
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    ours = lambda: dmm.gemm_a8w8_ptpc(qa, bs, sa, sb, out=out)
    arms = {"ours": ours}
    vendor = {"library": VENDOR}
    try:
        vf = vendor_fn(torch, qa, qb, sa, sb)
        vf()
        arms["vendor_eager"] = vf
    except Exception as e:  # an unsupported _scaled_mm form leaves only the error in the line
        vendor["error"] = f"{type(e).__name__}: {str(e)[:160]}"
    t = timed_arms(arms, args.steps, args.warmup, WARM_S)
    ms = t["ours"]["median"]
    tflops = flops / (ms * 1e-3) / 1e12
    timing = {"protocol": f"HIP graph of {args.steps} launches replayed {BATCHES} times in {PASSES} passes "
                          f"alternating with the vendor arm; per-call median of the batches",
              "warm_s": t["ours"]["warm_s"], "batches": BATCHES, "launches_per_batch": args.steps,
              "min_ms": round(t["ours"]["min"], 5), "max_ms": round(t["ours"]["max"], 5),
              "min_of_pass_medians_ms": round(t["ours"]["pass_min"], 5), "batches_ms": t["ours"]["batches_ms"]}
    cold = cold_ms(ours)
    timing["cold_ms_after_1GiB_scrub"] = {kk: round(v, 5) for kk, v in cold.items()}
    if "vendor_eager" in t:
        c = vf()
        vms = t["vendor_eager"]["median"]
        vendor.update({"us": round(vms * 1e3, 1), "TFLOP/s": round(flops / (vms * 1e-3) / 1e12, 1),
                       "min_of_pass_medians_us": round(t["vendor_eager"]["pass_min"] * 1e3, 1),
                       "rel_l2_vs_this_library": ((c.float() - out.float()).norm() / out.float().norm()).item()})
        del c
    gpu_c = None if args.no_cpu else out.view(torch.int16).cpu().numpy().view("uint16")
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
        "timing": timing,
        "device": device,
        "vendor_baseline": vendor,
    }
    del out, qb
    torch.cuda.empty_cache()
    if not args.no_ceiling:
        try:
            ceiling = mfma_ceiling(torch, qa, all_variants=args.calibrate)
            rec["mfma_ceiling"] = dict(ceiling, value_over_one_wave_ceiling=round(
                tflops / ceiling["one_wave_per_simd_TFLOP/s"], 4))
        except ImportError as e:
            rec["mfma_ceiling"] = {"error": str(e)}
    if args.calibrate:
        rec["memory_calibration"] = memory_calibration(torch)
    if args.extra:
        rec["extra"] = extra_shapes(dmm, torch, args)
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(m, n, k, args.cpu_rows, gpu_c)
    print(json.dumps(rec), flush=True)


# The quantisers on the configured shapes' operands: name -> (binding
# function, rows, cols, scale bytes).  Algorithmic bytes = fp32 in + codes +
# scales.
QUANTISERS = {
    "quantize_per_token_32768x1792": ("quantize_per_token", 32768, 1792, lambda r, c: 4 * r),
    "quantize_per_token_32768x7168": ("quantize_per_token", 32768, 7168, lambda r, c: 4 * r),
    "quantize_per_token_7168x1792": ("quantize_per_token", 7168, 1792, lambda r, c: 4 * r),
    "quantize_blockscale_a_16384x2048": ("quantize_blockscale_a", 16384, 2048, lambda r, c: 4 * r * c // 128),
    "quantize_blockscale_b_7168x2048": ("quantize_blockscale_b", 7168, 2048,
                                        lambda r, c: 4 * ((r + 127) // 128) * (c // 128)),
    "quantize_mxfp8_32768x1792": ("quantize_mxfp8", 32768, 1792, lambda r, c: r * c // 32),
    "quantize_mxfp8_7168x1792": ("quantize_mxfp8", 7168, 1792, lambda r, c: r * c // 32),
}


# The one-time B preshuffle on the headline's B: name -> (N, K); it reads
# and writes N K bytes.
PRESHUFFLES = {"preshuffle_b_7168x1792": (7168, 1792)}


def quantiser_bytes(name):
    if name in PRESHUFFLES:
        n, k = PRESHUFFLES[name]
        return 2 * n * k
    _, rows, cols, scale_bytes = QUANTISERS[name]
    return 5 * rows * cols + scale_bytes(rows, cols)


def prep_fn(dmm, torch, name):
    """A launch of quantiser or preshuffle ``name`` on its synthetic input."""
    from dense_matmul_amd import inputs

    if name in PRESHUFFLES:
        n, k = PRESHUFFLES[name]
        b = torch.from_numpy(inputs.normal((n, k), 4)).to("cuda:0").to(torch.float8_e4m3fn)
        out = torch.empty_like(b)
        return lambda: dmm.preshuffle_b(b, out=out)
    fname, rows, cols, _ = QUANTISERS[name]
    x = torch.from_numpy(inputs.normal((rows, cols), 3)).to("cuda:0")
    return lambda: getattr(dmm, fname)(x)


def run_workload(dmm, torch, name, steps, warmup):
    """One named workload (a GEMM of inputs.WORKLOADS or a quantiser of
    QUANTISERS): operands as the bench builds them, ``warmup`` launches,
    then ``steps`` launches, eagerly on the current stream (so a profiler
    sees each dispatch), then a synchronisation."""
    from dense_matmul_amd import inputs

    if name in QUANTISERS or name in PRESHUFFLES:
        fn = prep_fn(dmm, torch, name)
        repeat(fn, warmup)
        torch.cuda.synchronize()
        ms = event_ms(lambda: repeat(fn, steps), steps)
        print(json.dumps({"workload": name, "launches": steps, "us_per_launch": round(ms * 1e3, 2),
                          "alg_GB/s": round(quantiser_bytes(name) / (ms * 1e-3) / 1e9)}), flush=True)
        return
    mode, m, n, k, seed_a, seed_b = inputs.WORKLOADS[name]
    if mode == "bf16":
        a32, b_kn = inputs.bf16_operands(m, k, n, seed_a)
        a = torch.from_numpy(a32).to(torch.bfloat16).to("cuda:0")
        b = torch.from_numpy(b_kn.T.copy()).to(torch.bfloat16).to("cuda:0")
        out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
        fn = lambda: dmm.gemm_bf16(a, b, out=out)
    else:
        qa, bs, sa, sb = headline_operands(dmm, torch, m, n, k, seed_a, seed_b, mode)
        out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
        g = {"ptpc": dmm.gemm_a8w8_ptpc, "blockscale": dmm.gemm_a8w8_blockscale, "mxfp8": dmm.gemm_a8w8_mxfp8}[mode]
        fn = lambda: g(qa, bs, sa, sb, out=out)
    repeat(fn, warmup)
    torch.cuda.synchronize()
    ms = event_ms(lambda: repeat(fn, steps), steps)
    print(json.dumps({"workload": name, "mode": mode, "m": m, "n": n, "k": k, "launches": steps,
                      "us_per_launch": round(ms * 1e3, 2), "TFLOP/s": round(2.0 * m * n * k / (ms * 1e-3) / 1e12, 1)}),
          flush=True)


def extra_shapes(dmm, torch, args):
    """Secondary lines: the other scaling modes, the tail-only and gathered
    shapes, the quantisers and the bf16 GEMM, each timed with the same
    protocol (graph batches, median of 9, vendor arm alternating for the
    ptpc shapes) after at least 0.15 s of warm-up launches."""
    res = {}
    steps, warm_s = max(5, args.steps // 4), 0.15
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
        arms = {"ours": lambda: fn(qa, bs, sa, sb, out=out)}
        if mode == "ptpc":  # the vendor library has the per-row / per-column form only
            arms["vendor_eager"] = vendor_fn(torch, qa, qb, sa, sb)
        t = timed_arms(arms, steps, 20, warm_s)
        ms = t["ours"]["median"]
        tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        hbm = (m * k + n * k + 2 * m * n) / (ms * 1e-3) / 1e9
        res[name] = {"us": round(ms * 1e3, 1), "min_us": round(t["ours"]["min"] * 1e3, 1),
                     "max_us": round(t["ours"]["max"] * 1e3, 1), "TFLOP/s": round(tf, 1),
                     "pct_fp8_peak": round(100 * tf / PEAK_FP8_TFLOPS, 1), "alg_GB/s": round(hbm, 0)}
        if "vendor_eager" in t:
            res[name]["vendor_us"] = round(t["vendor_eager"]["median"] * 1e3, 1)
        del qa, bs, sa, sb, qb, out, arms
        torch.cuda.empty_cache()
    from dense_matmul_amd import inputs

    # the quantisers (run before the GEMM, not in its time), on the configured
    # shapes' operands
    for name in list(QUANTISERS) + list(PRESHUFFLES):
        fn = prep_fn(dmm, torch, name)
        t = timed_arms({"q_eager": fn}, 100, 20, warm_s)
        ms = t["q_eager"]["median"]
        gbs = quantiser_bytes(name) / (ms * 1e-3) / 1e9
        res[name] = {"us": round(ms * 1e3, 1), "alg_GB/s": round(gbs), "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 1)}
        del fn
        torch.cuda.empty_cache()

    m, k, n = 4096, 1024, 896
    a32, b_kn = inputs.bf16_operands(m, k, n, 233)
    a = torch.from_numpy(a32).to(torch.bfloat16).to("cuda:0")
    b = torch.from_numpy(b_kn.T.copy()).to(torch.bfloat16).to("cuda:0")
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    t = timed_arms({"bf16": lambda: dmm.gemm_bf16(a, b, out=out)}, 200, 20, warm_s)
    ms = t["bf16"]["median"]
    tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
    res["bf16_4096x896x1024"] = {"us": round(ms * 1e3, 2), "min_us": round(t["bf16"]["min"] * 1e3, 2),
                                 "TFLOP/s": round(tf, 1), "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 1),
                                 "alg_GB/s": round((2 * (m * k + n * k + m * n)) / (ms * 1e-3) / 1e9)}
    return res


if __name__ == "__main__":
    main()
