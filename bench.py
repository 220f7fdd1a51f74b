#!/usr/bin/env python3
"""Benchmark: blockwise FP4 fake quantization on one MI355X.

One step is one pass of the whole fake-quantization path over one
16384 x 4096 BF16 activation tensor (N(0,1) with 8 outlier channels x100,
seed 3) and its upstream gradient (N(0, 1e-3^2), seed 4):

  mx_rne_row      MXFP4 fake quant, round to nearest even, 1x32 row groups
  nvt_rne_row     NVFP4 (per-tensor FP32 scale) fake quant, RNE, 1x16 rows
  nv128_rne_row   NVFP4 double block (FP32 scale per 128) fake quant, RNE
  nv128_sr_row    the same with Philox stochastic rounding (seed 1234)
  nv128_sr_col    double-block SR fake quant along the transposed axis
  mx_sr_col       MXFP4 SR fake quant along the transposed axis (seed 1235)
  ste_nv128       clip-masked straight-through backward
  dequant_nv128   codes + scales -> BF16

Every op writes all of its outputs (codes, scales, outer scales, BF16).
`value` is the step's algorithmic bytes (each input read once, each output
written once) over the step time, in GB/s.  Inputs are resident in HBM.  There
are three input/output buffer sets (~1.9 GB) and op k of step s works on set
(s + k) mod 3, so consecutive ops never share an input tensor and every op
streams its operands from HBM, not from the 256 MB Infinity Cache.  The step
is captured once per starting set as a HIP graph and the graphs are replayed
(`ms_per_step`); the same ops launched one by one with events around each
(`ms_per_step_eager`) give the per-kernel times under "kernels" and the
roofline figures: each op's rate as a fraction of the 8 TB/s HBM peak
(`frac_hbm`, the target) and of the device copy measured in the same run
(`frac_copy`, context).

The QAT linear forward (X 8192x2880 @ W 2880x5760, both NVFP4 RNE) and its
backward (dY 8192x5760, gradient operands NVFP4 double block with stochastic
rounding; two products) are timed after the step and reported in TFLOP/s under
"qlinear" and "qlinear_bwd", each after 0.3 s of back-to-back calls so that the
figures are taken at the clock that sustained matrix-core work settles at (from
idle the first calls run up to 20 % slower).  The CPU oracle is
timed on a bounded sample (the first rows of the same tensors) for
"cpu_baseline".
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP4_PEAK_TFLOPS = 10100.0       # MI355X dense FP4 matrix peak, TFLOP/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense BF16 MFMA, TFLOP/s
METRIC = "FP4 fake-quant GB/s and % of HBM peak (MXFP4/NVFP4, 16384x4096 bf16)"
ROWS, COLS = 16384, 4096
NBUF = 3
WARM_SECONDS = 0.3                # sustained warm-up before each matrix-core timing


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def op_bytes(op: str, n: int) -> int:
    """Algorithmic bytes of one op on n elements (read once + outputs)."""
    x, y = 2 * n, 2 * n
    codes = n // 2
    if op.startswith("mx"):
        scales, outer = n // 32, 0
    elif op.startswith("nvt"):
        scales, outer = n // 16, 4
    else:
        scales, outer = n // 16, 4 * (n // 128)
    if op == "ste_nv128":
        return x + 2 * n + scales + outer + 2 * n          # x, dy, scales, outer -> dx
    if op == "dequant_nv128":
        return codes + scales + outer + y
    return x + y + codes + scales + outer


OPS = ["mx_rne_row", "nvt_rne_row", "nv128_rne_row", "nv128_sr_row", "nv128_sr_col",
       "mx_sr_col", "ste_nv128", "dequant_nv128"]
# the kernels each op launches (names as the rocprofv3 summaries list them;
# template arguments: format, rounding, row mapping or non-temporal stores, ...)
OP_KERNELS = {
    "mx_rne_row": ["k_quant_row<0, 0, 1, true, 0>"],
    "nvt_rne_row": ["k_absmax<false>", "k_quant_row<1, 0, 2, true, 0>"],
    "nv128_rne_row": ["k_quant_row<2, 0, 1, true, 0>"],
    "nv128_sr_row": ["k_quant_row<2, 1, 0, true, 0>"],
    "nv128_sr_col": ["k_quant_col<2, 1, true, 0, false>"],
    "mx_sr_col": ["k_quant_col<0, 1, true, 0, false>"],
    "ste_nv128": ["k_ste_row<2>"],
    "dequant_nv128": ["k_dequant_row<2>"],
}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("fq_device.hpp", "fq_kernels.hip"):
        with open(os.path.join(ROOT, "fp4_block_quantization_fq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(op: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if
    they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("kernel_source_hash") != kernel_source_hash():
        return None
    ent = data.get("ops", {}).get(op)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


def warm(fn, torch, seconds=WARM_SECONDS):
    """Run fn until the GPU has been busy with it for `seconds` of wall time.
    The matrix-core kernels run at a clock that settles only after some
    tenths of a second of sustained load (a few calls from idle run up to
    20 % slower); their figures are taken at that settled clock, as a training
    loop that calls them back to back sees it."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


CONFIG_TARGET_US = {"cfg1_mx_rne_1024x4096": 3.39, "cfg2_nvt_rne_2880x2880": 6.76,
                    "cfg4b_nvt_sr_col_4096x4096": 7.68, "cfg4c_mx_sr_col_4096x4096": 7.58}


def time_configs(fq, wl, torch, np, dev, to_dev):
    """The small configurations at their own shapes: one op per call, each call
    on its own buffer set, with enough sets (over 512 MB in all) that no call
    finds its operands in the 256 MB Infinity Cache.  One HIP graph holds one
    call per set and is replayed; the time per call includes the gaps between
    back-to-back kernels.  Bytes: input read once plus every output (and the
    per-tensor maximum pass's second read of x charged, not counted)."""
    cfgs = [
        ("cfg1_mx_rne_1024x4096", wl.mx_activation(), fq.fq_desc_mxfp4(), "fake_quant"),
        ("cfg2_nvt_rne_2880x2880", wl.nv_weight(), fq.fq_desc_nvfp4(), "fake_quant"),
        ("cfg4b_nvt_sr_col_4096x4096", wl.backward_weight(),
         fq.fq_desc_nvfp4(rounding=fq.FQ_ROUND_SR, axis=fq.FQ_AXIS_COL, seed=1234), "quantize"),
        ("cfg4c_mx_sr_col_4096x4096", wl.backward_weight(),
         fq.fq_desc_mxfp4(rounding=fq.FQ_ROUND_SR, axis=fq.FQ_AXIS_COL, seed=1235), "quantize"),
    ]
    res = {}
    for name, xb, d, kind in cfgs:
        R, C = xb.shape
        n = R * C
        nouter = 0 if d.outer == fq.FQ_OUTER_NONE else 4
        by = (2 * n + n // 2 + n // d.block_size + nouter + (2 * n if kind == "fake_quant" else 0))
        nsets = max(2, (512 << 20) // by + 2)
        xs = [to_dev(xb) for _ in range(nsets)]
        ys = [torch.empty_like(xs[0]) for _ in range(nsets)] if kind == "fake_quant" else None
        outs = [fq.alloc_outputs(d, R, C, dev) for _ in range(nsets)]
        ws = torch.empty((4096,), dtype=torch.uint8, device=dev)

        def call(i):
            if kind == "fake_quant":
                fq.fq_fake_quant(d, xs[i], y=ys[i], out=outs[i], ws=ws)
            else:
                fq.fq_quantize(d, xs[i], out=outs[i], ws=ws)
        for i in range(nsets):
            call(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=cap):
            for i in range(nsets):
                call(i)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        reps = 10
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * nsets)
        gbs = by / (us * 1e-6) / 1e9
        res[name] = {"us": round(us, 3), "bytes": by, "GBps": round(gbs, 1),
                     "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                     "target_us": CONFIG_TARGET_US[name], "buffer_sets": nsets,
                     "op": kind}
        del xs, ys, outs, g
    return res


def kernel_split(torch, fn, calls):
    """Average kernel durations (us per call) of `calls` calls made by fn,
    grouped as 'gemm' (the matrix-core product) and the rest by kernel name,
    from torch's profiler (device-side timestamps)."""
    try:
        from torch.profiler import ProfilerActivity, profile
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            fn()
            torch.cuda.synchronize()
        tot = {}
        for ev in prof.key_averages():
            dev_us = getattr(ev, "device_time_total", None)
            if dev_us is None:
                dev_us = getattr(ev, "cuda_time_total", 0.0)
            if not dev_us:
                continue
            key = ev.key
            if "k_gemm" in key:
                name = "gemm"
            elif "k_absmax" in key:
                name = "absmax"
            elif "k_quant_col" in key:
                name = "quant_col_w"
            elif "k_quant_row" in key:
                name = "quant_row_x"
            else:
                continue
            tot[name] = tot.get(name, 0.0) + dev_us / calls
        return {k: round(v, 2) for k, v in tot.items()} or None
    except Exception as e:  # the profiler is an optional diagnostic
        log(f"bench: kernel split unavailable ({e})")
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_configs(oracle, wl, np):
    """The oracle on every configuration at its full size (wall clock), a
    single-thread run of configuration 1, and configuration 5 as the oracle's
    two fake quantizations plus numpy's FP32 matmul (BLAS threads recorded)."""
    out = {}

    def timed(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    def entry(by, dt, threads):
        return {"seconds": round(dt, 3), "GBps": round(by / dt / 1e9, 4), "threads": threads}

    nt = oracle.default_threads()
    x1 = wl.mx_activation()
    n1 = x1.size
    b1 = 2 * n1 + 2 * n1 + n1 // 2 + n1 // 32
    out["cfg1"] = entry(b1, timed(lambda: oracle.fake_quant(x1, "mx", "rne")), nt)
    out["cfg1_single_thread"] = entry(b1, timed(lambda: oracle.fake_quant(x1, "mx", "rne",
                                                                          nthreads=1)), 1)
    x2 = wl.nv_weight()
    n2 = x2.size
    out["cfg2"] = entry(4 * n2 + n2 // 2 + n2 // 16 + 4,
                        timed(lambda: oracle.fake_quant(x2, "nv_tensor", "rne")), nt)
    x3 = wl.nv_activation()
    n3 = x3.size
    b3 = 4 * n3 + n3 // 2 + n3 // 16 + 4 * (n3 // 128)
    out["cfg3_rne"] = entry(b3, timed(lambda: oracle.fake_quant(x3, "nv_128", "rne")), nt)
    out["cfg3_sr"] = entry(b3, timed(lambda: oracle.fake_quant(x3, "nv_128", "sr", seed=1234)), nt)
    f3 = oracle.fake_quant(x3, "nv_128", "rne")
    dy = wl.grad_output()
    out["cfg4a_ste"] = entry(6 * n3 + n3 // 16 + 4 * (n3 // 128),
                             timed(lambda: oracle.ste_backward(x3, f3["scales"], f3["outer"], dy,
                                                               "nv_128")), nt)
    del x3, f3, dy
    w4 = wl.backward_weight()
    n4 = w4.size
    out["cfg4b"] = entry(2 * n4 + n4 // 2 + n4 // 16 + 4,
                         timed(lambda: oracle.fake_quant(w4, "nv_tensor", "sr", "col", 1234)), nt)
    out["cfg4c"] = entry(2 * n4 + n4 // 2 + n4 // 32,
                         timed(lambda: oracle.fake_quant(w4, "mx", "sr", "col", 1235)), nt)
    xm, wm = wl.linear_inputs()
    t = time.perf_counter()
    fx = oracle.fake_quant(xm, "nv_tensor", "rne", "row")
    fw = oracle.fake_quant(wm, "nv_tensor", "rne", "col")
    a = oracle.bf16_bits_to_f64(fx["y"]).astype(np.float32)
    b = oracle.bf16_bits_to_f64(fw["y"]).astype(np.float32)
    tq = time.perf_counter() - t
    t = time.perf_counter()
    a @ b
    tm = time.perf_counter() - t
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:
        blas = []
    fl = 2.0 * xm.shape[0] * xm.shape[1] * wm.shape[1]
    out["cfg5"] = {"seconds_fake_quant": round(tq, 3), "seconds_matmul_fp32": round(tm, 3),
                   "TFLOPs": round(fl / (tq + tm) / 1e12, 4), "threads": nt,
                   "blas_threads": blas[0] if blas else None}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=16384,
                    help="rows of the workload the CPU oracle is timed on")
    ap.add_argument("--qlinear-iters", type=int, default=20)
    ap.add_argument("--only", default="", help="comma-separated subset of ops (profiling)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the step from eager launches instead of HIP graph replays")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: measures one GPU only (--gpus 1); how the path shards across GPUs "
              "is a design note, not a benchmark.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp4_block_quantization_fq_amd as fq
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("bench: generating inputs")
    x_bits = wl.nv_activation(ROWS, COLS, seed=3)
    dy_bits = wl.grad_output(ROWS, COLS, seed=4)

    def to_dev(b):
        return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)

    n = ROWS * COLS
    xs = [to_dev(x_bits) for _ in range(NBUF)]
    dys = [to_dev(dy_bits) for _ in range(NBUF)]
    ys = [torch.empty_like(xs[0]) for _ in range(NBUF)]

    descs = {
        "mx_rne_row": fq.fq_desc_mxfp4(),
        "nvt_rne_row": fq.fq_desc_nvfp4(),
        "nv128_rne_row": fq.fq_desc_nvfp4(outer=fq.FQ_OUTER_BLOCK128),
        "nv128_sr_row": fq.fq_desc_nvfp4(outer=fq.FQ_OUTER_BLOCK128, rounding=fq.FQ_ROUND_SR,
                                         seed=1234),
        "nv128_sr_col": fq.fq_desc_nvfp4(outer=fq.FQ_OUTER_BLOCK128, rounding=fq.FQ_ROUND_SR,
                                         axis=fq.FQ_AXIS_COL, seed=1234),
        "mx_sr_col": fq.fq_desc_mxfp4(rounding=fq.FQ_ROUND_SR, axis=fq.FQ_AXIS_COL, seed=1235),
    }
    d_nv128 = descs["nv128_rne_row"]
    outs = {op: [fq.alloc_outputs(d, ROWS, COLS, dev) for _ in range(NBUF)]
            for op, d in descs.items()}
    ws = torch.empty((4096,), dtype=torch.uint8, device=dev)
    dxs = [torch.empty_like(xs[0]) for _ in range(NBUF)]
    # forward scales for the STE / dequant ops come from the RNE double-block op
    ops = [o for o in OPS if not args.only or o in args.only.split(",")]

    def run_op(op, i):
        if op in descs:
            fq.fq_fake_quant(descs[op], xs[i], y=ys[i], out=outs[op][i], ws=ws)
        elif op == "ste_nv128":
            fq.fq_ste_backward(d_nv128, xs[i], outs["nv128_rne_row"][i], dys[i], dx=dxs[i])
        elif op == "dequant_nv128":
            fq.fq_dequantize(d_nv128, outs["nv128_rne_row"][i], ROWS, COLS, y=dxs[i])

    # make the forward scales exist before the first STE / dequant
    for i in range(NBUF):
        fq.fq_fake_quant(d_nv128, xs[i], y=ys[i], out=outs["nv128_rne_row"][i])
    torch.cuda.synchronize()

    # Op k of step s works on buffer set (s + k) % NBUF: consecutive ops never
    # share an input, so no op finds the tensor the previous one just streamed
    # in the 256 MB Infinity Cache.
    def run_step(s):
        for k, op in enumerate(ops):
            run_op(op, (s + k) % NBUF)

    log(f"bench: warmup {args.warmup} steps")
    for s in range(args.warmup):
        run_step(s)
    torch.cuda.synchronize()

    K = args.steps
    # Per-kernel times: every op bracketed by events on the launch stream.
    ev = {op: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(K)] for op in ops}
    log(f"bench: timing {K} steps op by op")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        for k, op in enumerate(ops):
            a, b = ev[op][s]
            a.record()
            run_op(op, (s + k) % NBUF)
            b.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step_eager = (t1 - t0) * 1e3 / K

    # The step itself: one HIP graph per buffer set holding the whole step
    # (every op, every launch), replayed K times.  The same kernels on the same
    # buffers; the graph only removes the per-launch host and queue overhead.
    ms_per_step = ms_per_step_eager
    graphs = []
    if not args.no_graph:
        log("bench: capturing the step as HIP graphs")
        cap = torch.cuda.Stream()
        for i in range(NBUF):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                run_step(i)
            graphs.append(g)
        for s in range(2 * NBUF):
            graphs[s % NBUF].replay()
        torch.cuda.synchronize()
        log(f"bench: timing {K} graph steps")
        t0 = time.perf_counter()
        for s in range(K):
            graphs[s % NBUF].replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_per_step = (t1 - t0) * 1e3 / K

    kernels = {}
    step_bytes = 0
    for op in ops:
        times = [a.elapsed_time(b) for a, b in ev[op]]
        avg = float(np.mean(times))
        by = op_bytes(op, n)
        step_bytes += by
        # mean (what a profiler's per-kernel average compares with) and median
        kernels[op] = {"ms": round(avg, 5), "ms_median": round(float(np.median(times)), 5),
                       "bytes": by,
                       "GBps": round(by / (avg * 1e-3) / 1e9, 1),
                       "frac_hbm": round(by / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # dominant single-kernel op: the largest share of the step time (the
    # per-tensor op is two kernels, so it is reported beside it instead)
    single = [o for o in ops if o != "nvt_rne_row"]
    dom = max(single or ops, key=lambda o: kernels[o]["ms"])
    achieved = kernels[dom]["GBps"]
    roofline = {"bound": "hbm", "kernel": dom, "kernels": OP_KERNELS.get(dom),
                "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": load_traffic(dom)}
    low = min(ops, key=lambda o: kernels[o]["frac_hbm"])
    roofline["lowest_op"] = {"op": low, "frac": kernels[low]["frac_hbm"],
                             "kernels": OP_KERNELS.get(low), "traffic": load_traffic(low)}

    # ---------------- copy yardstick (achievable bandwidth) ----------------
    # torch's device copy of one 16384x4096 BF16 tensor: 2 B read + 2 B written
    # per element.  Not part of the library; it is the reference the roofline
    # fractions and the HBM byte counters are compared against.
    log("bench: copy yardstick")
    for i in range(NBUF):
        dxs[i].copy_(xs[i])
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for s in range(10):
        dxs[s % NBUF].copy_(xs[s % NBUF])
    c1.record()
    torch.cuda.synchronize()
    copy_ms = c0.elapsed_time(c1) / 10
    copy = {"op": "torch copy_ of 16384x4096 bf16", "bytes": 4 * n, "ms": round(copy_ms, 5),
            "GBps": round(4 * n / (copy_ms * 1e-3) / 1e9, 1)}
    # second fraction, as context: each op's rate against the measured copy
    for op in ops:
        kernels[op]["frac_copy"] = round(kernels[op]["GBps"] / copy["GBps"], 4)

    # ---------------- the configurations at their own shapes ----------------
    per_config = None
    if not args.only:
        log("bench: per-config timings")
        per_config = time_configs(fq, wl, torch, np, dev, to_dev)

    # ---------------- QAT linear ----------------
    qlin = None
    if not args.only:
        log("bench: qlinear")
        M, Kd, N = 8192, 2880, 5760
        xm, wm = wl.linear_inputs(M, Kd, N)
        xq, wq = to_dev(xm), to_dev(wm)
        dxd = fq.fq_desc_nvfp4()
        dwd = fq.fq_desc_nvfp4(axis=fq.FQ_AXIS_COL)
        qws = fq.qlinear_workspace(dxd, dwd, M, Kd, N, dev)
        yq = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        warm(lambda: fq.fq_qlinear_fwd(dxd, dwd, xq, wq, y=yq, ws=qws), torch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.qlinear_iters):
            fq.fq_qlinear_fwd(dxd, dwd, xq, wq, y=yq, ws=qws)
        e1.record()
        torch.cuda.synchronize()
        qms = e0.elapsed_time(e1) / args.qlinear_iters
        flops = 2.0 * M * Kd * N
        tf = flops / (qms * 1e-3) / 1e12
        # cold operands: three independent (X, W, workspace, Y) sets in turn,
        # 0.76 GB in all, so no call finds its operands in the Infinity Cache
        sets = [(to_dev(xm), to_dev(wm), fq.qlinear_workspace(dxd, dwd, M, Kd, N, dev),
                 torch.empty((M, N), dtype=torch.bfloat16, device=dev)) for _ in range(3)]
        run_cold = lambda i: fq.fq_qlinear_fwd(dxd, dwd, sets[i % 3][0], sets[i % 3][1],
                                               y=sets[i % 3][3], ws=sets[i % 3][2])
        warm(lambda: [run_cold(i) for i in range(3)], torch)
        e0.record()
        for i in range(args.qlinear_iters):
            run_cold(i)
        e1.record()
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / args.qlinear_iters
        split = kernel_split(torch, lambda: [run_cold(i) for i in range(6)], 6)
        qlin = {"workload": "X 8192x2880 N(0,1) @ W 2880x5760 N(0,0.02^2), NVFP4 RNE both",
                "ms": round(qms, 4), "TFLOPs": round(tf, 1),
                "ms_cold": round(cms, 4),
                "TFLOPs_cold": round(flops / (cms * 1e-3) / 1e12, 1),
                "kernels_us": split,
                "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                             "frac_cold": round(flops / (cms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}}
        if split and "gemm" in split:
            gtf = flops / (split["gemm"] * 1e-6) / 1e12
            qlin["gemm_only"] = {"us": split["gemm"], "TFLOPs": round(gtf, 1),
                                 "frac": round(gtf / BF16_PEAK_TFLOPS, 4)}
            qlin["prologue_us"] = round(sum(v for k, v in split.items() if k != "gemm"), 2)
        del sets

    # ---------------- the same linear with MXFP4 operands (FP4 matrix cores) ----------------
    qmx = None
    if not args.only:
        log("bench: qlinear mxfp4")
        dxm = fq.fq_desc_mxfp4()
        dwm = fq.fq_desc_mxfp4(axis=fq.FQ_AXIS_COL)
        warm(lambda: fq.fq_qlinear_fwd(dxm, dwm, xq, wq, y=yq, ws=qws), torch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.qlinear_iters):
            fq.fq_qlinear_fwd(dxm, dwm, xq, wq, y=yq, ws=qws)
        e1.record()
        torch.cuda.synchronize()
        mms = e0.elapsed_time(e1) / args.qlinear_iters
        tfm = 2.0 * M * Kd * N / (mms * 1e-3) / 1e12
        qmx = {"workload": "the same X @ W with both operands MXFP4 RNE: codes and E8M0 scales "
                           "multiplied on the scaled FP4 matrix cores",
               "ms": round(mms, 4), "TFLOPs": round(tfm, 1),
               "roofline": {"bound": "mfma", "achieved": round(tfm, 1), "peak": FP4_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(tfm / FP4_PEAK_TFLOPS, 4)}}

    # ---------------- QAT linear backward ----------------
    qbwd = None
    if not args.only:
        log("bench: qlinear backward")
        dym = wl.normal_bf16((M, N), 1e-3, 8)
        dyq = to_dev(dym)
        dgd = fq.fq_desc_nvfp4(outer=fq.FQ_OUTER_BLOCK128, rounding=fq.FQ_ROUND_SR, seed=1234)
        bws = fq.qlinear_bwd_workspace(dxd, dwd, dgd, M, Kd, N, dev)
        gx = torch.empty((M, Kd), dtype=torch.bfloat16, device=dev)
        gw = torch.empty((Kd, N), dtype=torch.bfloat16, device=dev)
        warm(lambda: fq.fq_qlinear_bwd(dxd, dwd, dgd, xq, wq, dyq, dx=gx, dw=gw, ws=bws), torch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.qlinear_iters):
            fq.fq_qlinear_bwd(dxd, dwd, dgd, xq, wq, dyq, dx=gx, dw=gw, ws=bws)
        e1.record()
        torch.cuda.synchronize()
        bms = e0.elapsed_time(e1) / args.qlinear_iters
        tfb = 4.0 * M * Kd * N / (bms * 1e-3) / 1e12
        qbwd = {"workload": "dY 8192x5760 N(0,1e-6) through the linear above; dX and dW "
                            "products on NVFP4 double-block SR operands (seed 1234)",
                "ms": round(bms, 4), "TFLOPs": round(tfb, 1),
                "roofline": {"bound": "mfma", "achieved": round(tfb, 1),
                             "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(tfb / BF16_PEAK_TFLOPS, 4)}}

    # ---------------- the backward with MXFP4 everywhere (FP4 matrix cores) ----------------
    qbwd_mx = None
    if not args.only:
        log("bench: qlinear backward mxfp4")
        mxd_x, mxd_w = fq.fq_desc_mxfp4(), fq.fq_desc_mxfp4(axis=fq.FQ_AXIS_COL)
        mxd_g = fq.fq_desc_mxfp4(rounding=fq.FQ_ROUND_SR, seed=1234)
        bws_mx = fq.qlinear_bwd_workspace(mxd_x, mxd_w, mxd_g, M, Kd, N, dev)
        warm(lambda: fq.fq_qlinear_bwd(mxd_x, mxd_w, mxd_g, xq, wq, dyq, dx=gx, dw=gw,
                                       ws=bws_mx), torch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.qlinear_iters):
            fq.fq_qlinear_bwd(mxd_x, mxd_w, mxd_g, xq, wq, dyq, dx=gx, dw=gw, ws=bws_mx)
        e1.record()
        torch.cuda.synchronize()
        bmx = e0.elapsed_time(e1) / args.qlinear_iters
        tfx = 4.0 * M * Kd * N / (bmx * 1e-3) / 1e12
        qbwd_mx = {"workload": "the same backward with MXFP4 forward operands and MXFP4 SR "
                               "gradient operands (seed 1234): both products on the scaled "
                               "FP4 matrix cores",
                   "ms": round(bmx, 4), "TFLOPs": round(tfx, 1),
                   "roofline": {"bound": "mfma", "achieved": round(tfx, 1),
                                "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                                "frac": round(tfx / FP4_PEAK_TFLOPS, 4)}}

    # ---------------- STE from the bit-packed keep mask ----------------
    ste_mask = None
    if not args.only:
        log("bench: ste from keep mask")
        keeps = [fq.fq_fake_quant_mask(d_nv128, xs[i], y=ys[i])[1] for i in range(NBUF)]
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(K):
            fq.fq_ste_backward_mask(keeps[s % NBUF], dys[s % NBUF], dx=dxs[s % NBUF])
        e1.record()
        torch.cuda.synchronize()
        sms = e0.elapsed_time(e1) / K
        sb = 2 * n + n // 8 + 2 * n
        ste_mask = {"op": "dx = keep ? dy : 0 on 16384x4096 (dy, 1-bit mask -> dx)",
                    "ms": round(sms, 5), "bytes": sb,
                    "GBps": round(sb / (sms * 1e-3) / 1e9, 1),
                    "frac_hbm": round(sb / (sms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    # ---------------- TetraJet-v2 controls: retained channels, OsciReset ----------------
    outc = None
    if not args.only:
        log("bench: retained channels and oscillation tracker")
        kret = COLS // 10
        amax = fq.fq_channel_absmax(xs[0])
        retain, cscale = fq.fq_select_channels(amax, kret)
        ret_outs = [fq.alloc_outputs(d_nv128, ROWS, COLS, dev) for _ in range(NBUF)]
        for i in range(NBUF):
            fq.fq_fake_quant_retain(d_nv128, xs[i], retain, cscale, y=ys[i], out=ret_outs[i], ws=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(K):
            fq.fq_fake_quant_retain(d_nv128, xs[s % NBUF], retain, cscale, y=ys[s % NBUF], ws=ws,
                                    out=ret_outs[s % NBUF])
        e1.record()
        torch.cuda.synchronize()
        tms = e0.elapsed_time(e1) / K
        tb = op_bytes("nv128_rne_row", n)
        outc = {"retain_nv128_rne_row": {
                    "op": f"NVFP4 double-block RNE fake quant of 16384x4096 with {kret} of "
                          f"{COLS} channels kept in FP8 E4M3", "ms": round(tms, 5), "bytes": tb,
                    "GBps": round(tb / (tms * 1e-3) / 1e9, 1),
                    "frac_hbm": round(tb / (tms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
        # the tracker and the check over the 2880x5760 weight (16.6 M weights),
        # q and its codes from the NVFP4 per-tensor quantizer along K (the
        # linear's weight); the check resets to the bin centre
        wr, wc = 2880, 5760
        nw = wr * wc
        d_wq = fq.fq_desc_nvfp4(axis=fq.FQ_AXIS_COL)
        wts = [torch.randn(wr, wc, device=dev, dtype=torch.float32) * 0.02 for _ in range(NBUF)]
        wq_outs = [fq.alloc_outputs(d_wq, wr, wc, dev) for _ in range(NBUF)]
        qts = [fq.fq_fake_quant(d_wq, w.to(torch.bfloat16), out=o) for w, o in zip(wts, wq_outs)]
        sts = [fq.osci_state(nw, dev) for _ in range(NBUF)]
        for i in range(NBUF):
            fq.fq_osci_track(wts[i], qts[i], sts[i], first=True)
        torch.cuda.synchronize()
        for name, fn, by in (("osci_track", lambda i: fq.fq_osci_track(wts[i], qts[i], sts[i]),
                              34 * nw),
                             ("osci_reset", lambda i: fq.fq_osci_reset(wts[i], qts[i], sts[i], 4.0,
                                                                       d_wq, wq_outs[i]),
                              32 * nw)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for s in range(K):
                fn(s % NBUF)
            e1.record()
            torch.cuda.synchronize()
            oms = e0.elapsed_time(e1) / K
            outc[name] = {"op": f"{name} over 2880x5760 FP32 master weights", "ms": round(oms, 5),
                          "bytes": by, "GBps": round(by / (oms * 1e-3) / 1e9, 1),
                          "frac_hbm": round(by / (oms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    # ---------------- random Hadamard transform ----------------
    rht = None
    if not args.only:
        log("bench: hadamard")
        rht = {}
        for name, ax in (("row128", fq.FQ_AXIS_ROW), ("col128", fq.FQ_AXIS_COL)):
            for i in range(NBUF):
                fq.fq_hadamard(xs[i], 128, ax, 77, y=ys[i])
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for s in range(K):
                fq.fq_hadamard(xs[s % NBUF], 128, ax, 77, y=ys[s % NBUF])
            e1.record()
            torch.cuda.synchronize()
            hms = e0.elapsed_time(e1) / K
            rht[name] = {"ms": round(hms, 5), "bytes": 4 * n,
                         "GBps": round(4 * n / (hms * 1e-3) / 1e9, 1),
                         "frac_hbm": round(4 * n / (hms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        # the backward again with both products' operands rotated (128-blocks)
        bws_r = fq.qlinear_bwd_workspace(dxd, dwd, dgd, M, Kd, N, dev, rht_block=128)
        warm(lambda: fq.fq_qlinear_bwd(dxd, dwd, dgd, xq, wq, dyq, dx=gx, dw=gw, ws=bws_r,
                                       rht_block=128, rht_seed=55), torch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.qlinear_iters):
            fq.fq_qlinear_bwd(dxd, dwd, dgd, xq, wq, dyq, dx=gx, dw=gw, ws=bws_r,
                              rht_block=128, rht_seed=55)
        e1.record()
        torch.cuda.synchronize()
        rms = e0.elapsed_time(e1) / args.qlinear_iters
        rht["qlinear_bwd_rht128"] = {"ms": round(rms, 4),
                                     "TFLOPs": round(4.0 * M * Kd * N / (rms * 1e-3) / 1e12, 1)}

    # ---------------- CPU oracle baseline ----------------
    cpu = None
    if not args.no_cpu_baseline and not args.only:
        import oracle
        log(f"bench: cpu oracle on {args.cpu_rows} rows and on each configuration")
        r = args.cpu_rows
        xs_c = np.ascontiguousarray(x_bits[:r])
        dy_c = np.ascontiguousarray(dy_bits[:r])
        nthreads = oracle.default_threads()
        nc = r * COLS
        t = time.perf_counter()
        oracle.fake_quant(xs_c, "mx", "rne")
        oracle.fake_quant(xs_c, "nv_tensor", "rne")
        f = oracle.fake_quant(xs_c, "nv_128", "rne")
        oracle.fake_quant(xs_c, "nv_128", "sr", seed=1234)
        oracle.fake_quant(xs_c, "nv_128", "sr", "col", seed=1234)
        oracle.fake_quant(xs_c, "mx", "sr", "col", seed=1235)
        oracle.ste_backward(xs_c, f["scales"], f["outer"], dy_c, "nv_128")
        oracle.dequantize(f["codes"], f["scales"], f["outer"], "nv_128", xs_c.shape)
        dt = time.perf_counter() - t
        cbytes = sum(op_bytes(o, nc) for o in OPS)
        cpu = {"value": round(cbytes / dt / 1e9, 4), "unit": "GB/s", "cores": nthreads,
               "kind": "oracle", "seconds": round(dt, 2),
               "sample": f"the same 8-op step on the first {r} of {ROWS} rows "
                         f"({nc} elements per op)",
               "cpu_model": cpu_model(), "per_config": cpu_configs(oracle, wl, np)}

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_eager": round(ms_per_step_eager, 4), "step_launch": "graph" if graphs else "eager",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "FP4 fake-quant step over a 16384x4096 bf16 activation "
                               "(N(0,1), 8 outlier channels x100) and its gradient",
                   "rows": ROWS, "cols": COLS, "ops": ops, "step_bytes": step_bytes,
                   "frac_hbm_step": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "copy_yardstick": copy,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "per_config": per_config,
        "qlinear": qlin,
        "qlinear_mxfp4": qmx,
        "qlinear_bwd": qbwd,
        "qlinear_bwd_mxfp4": qbwd_mx,
        "ste_mask": ste_mask,
        "outcontrol": outc,
        "hadamard": rht,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
