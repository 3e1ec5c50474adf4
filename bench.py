"""Benchmark of libgemm355 on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle S]
                    [--no-cpu-baseline] [--no-detail] [--workload NAME]

A step is one call of the library on the headline workload (bf16
4096 x 4096 x 4096, A row-major, B column-major, bf16 C, fp32 accumulate)
with inputs already resident in HBM.  Before the W untimed warm-up steps the
device runs the same call untimed for S seconds (default 0.5): from idle the
shader clock takes some tens of milliseconds of load to reach its
(power-limited) operating point.  Prints ONE JSON line: throughput in
TFLOP/s of useful work 2MNK per step (section "Shape the operation" of page
"10. Tensor Cores, shapes, and tile alignment"), the roofline of the main
kernel (achieved vs the dense bf16 MFMA peak, timed with HIP events on the
launch stream; also the median and minimum of per-call kernel times), the
CPU oracle timed on a bounded sample, and a per-workload detail list (every
named workload, each timed the same way, HBM-bound shapes rotating input
copies so they cannot sit in the 256 MB last-level cache, each with the
oracle timed on a bounded sample of it).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "e4m3": 5033.2, "fp4": 10066.3}   # MI355X dense MFMA, 2.4 GHz (fp6 as fp4)
PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20
KERNEL_SOURCES = ["dense_tiled_gemm_fp8_amd/csrc/kernels.hip", "dense_tiled_gemm_fp8_amd/csrc/sched.h",
                  "dense_tiled_gemm_fp8_amd/csrc/tiles.h", "dense_tiled_gemm_fp8_amd/csrc/plan.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_bf16_4096cube.json")


def kernel_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle", type=float, default=None, metavar="SECONDS",
                    help="untimed calls for this long before the warm-up of each workload "
                         "(the clock ramps up from idle); default 0.5 s, 0 with --profile")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--workload", default=None, help="time only this workload name (detail)")
    ap.add_argument("--profile", default=None, metavar="NAME[:INDEX]",
                    help="only run warmup + steps calls of this workload shape (for counter "
                         "collection under rocprofv3) and print its time")
    ap.add_argument("--tile", type=int, default=-1,
                    help="with --profile: force this tile-table entry instead of the planner's")
    ap.add_argument("--stamps", action="store_true",
                    help="with --profile: one more call with the per-unit clock hook; prints the "
                         "measured eta, shader clock and MFMA cycle efficiency")
    ap.add_argument("--sustain", type=float, default=0.0, metavar="SECONDS",
                    help="with --profile: after the timed calls, keep calling for this long and "
                         "print the sustained time per call; the device's socket power and "
                         "graphics clocks are sampled (amd-smi) half way through")
    ap.add_argument("--vendor", action="store_true",
                    help="with --profile and a bf16 workload: time the vendor library "
                         "(torch.matmul into bf16 C, torch.mm with out_dtype float32 for fp32 C, "
                         "on the same operand copies) instead of this library, as context")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes 5 times "
                         "(reference kernel for scaling the HBM byte counters)")
    ap.add_argument("--pass-floor", type=int, default=0, metavar="BYTES",
                    help="only time two reference passes, 300 times each: an in-place add on one "
                         "float (what any extra launch costs) and on BYTES of floats (a plain pass "
                         "reading and writing that many bytes, to set beside the split-K combine)")
    return ap.parse_args()


def copy_reference(nbytes: int) -> None:
    """A plain device-to-device copy, 5 times: the reference kernel for
    scaling the HBM byte counters, and the stream rate a simple kernel
    reaches (each copy reads and writes nbytes)."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 5
    print(json.dumps({"copy_bytes": nbytes, "us_per_copy": round(us, 2),
                      "read_plus_write_tb_s": round(2 * nbytes / (us * 1e-6) / 1e12, 3)}), flush=True)
    log("copy reference: 5 x %d bytes" % nbytes)


def pass_floor(nbytes: int) -> None:
    """Two reference passes on the benchmark's stream, 300 times each: an
    in-place add on one float (the cost of one more launch with next to no
    work) and on nbytes of floats (one dependent read and write of every
    byte).  The split-K combine is such a pass over the partial sums."""
    import torch
    one = torch.zeros(1, dtype=torch.float32, device="cuda")
    big = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    out = {"pass_floor_bytes": nbytes}
    for name, t in (("us_one_float", one), ("us_per_pass", big)):
        for _ in range(20):
            t.add_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(300):
            t.add_(1.0)
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(e0.elapsed_time(e1) * 1e3 / 300, 2)
    print(json.dumps(out), flush=True)
    log("pass floor: 300 x one float, 300 x %d bytes" % nbytes)


def per_xcd(st, grid: int):
    """Shader clock (MHz) and last finish (us after the first start) of the
    units each XCD ran, from the per-unit stamps st[u] = (real-time start,
    real-time end, cycles at start, cycles at end, ...), the real-time clock
    ticking at 100 MHz.  The hardware deals workgroups to the 8 XCDs
    round-robin and the kernel renumbers them so that XCD x runs the logical
    slots [x q, (x + 1) q), q = grid / 8; unit u runs in slot u % grid.  None
    when grid is not a multiple of 8 (the renumbering is then uneven)."""
    import numpy as np
    if grid <= 0 or grid % 8:
        return None
    slot_xcd = (np.arange(len(st)) % grid) // (grid // 8)
    t0 = st[:, 0].min()
    out = {"sclk_mhz": [], "last_end_us": []}
    for x in range(8):
        m = slot_xcd == x
        rt = (st[m, 1] - st[m, 0]).sum()
        out["sclk_mhz"].append(round(float(100.0 * (st[m, 3] - st[m, 2]).sum() / rt), 0) if rt > 0 else None)
        out["last_end_us"].append(round(float((st[m, 1].max() - t0) / 100.0), 2) if m.any() else None)
    return out


class Case:
    """Device-resident operands of one workload shape (with rotation copies
    for HBM-bound shapes) and a callable that runs one step."""

    def __init__(self, w, si, torch, g, inputs, tile=-1):
        self.w, self.si = w, si
        ops = inputs.workload_operands(w, si)
        self.ops = ops
        self.M, self.N, self.K, self.batch = ops.M, ops.N, ops.K, ops.batch
        self.fmt = w.fmt
        view = __import__("numpy").int16 if w.fmt == "bf16" else __import__("numpy").uint8
        esize = 2 if w.fmt == "bf16" else 1
        in_bytes = ops.A.nbytes + ops.B.nbytes
        self.copies = 1
        flops = 2.0 * self.M * self.N * self.K * self.batch
        out_es = 2 if w.out == "bf16" else 4
        self.alg_bytes = in_bytes + self.M * self.N * self.batch * out_es
        self.flops = flops
        ai = flops / self.alg_bytes
        self.hbm_bound = ai < (PEAK_TFLOPS[w.fmt] * 1e12) / (PEAK_HBM_GBS * 1e9)
        if self.hbm_bound:
            self.copies = max(1, math.ceil(2 * MALL_BYTES / in_bytes))
        A = torch.from_numpy(ops.A.view(view)).cuda()
        B = torch.from_numpy(ops.B.view(view)).cuda()
        self.As = [A] + [A.clone() for _ in range(self.copies - 1)]
        self.Bs = [B] + [B.clone() for _ in range(self.copies - 1)]
        shape = (self.batch, self.M, self.N) if self.batch > 1 else (self.M, self.N)
        self.C = torch.empty(shape, dtype=torch.bfloat16 if w.out == "bf16" else torch.float32,
                             device="cuda")
        self.sa = torch.tensor(ops.scale_a, dtype=torch.float32, device="cuda") if w.fmt == "e4m3" else None
        self.sb = torch.tensor(ops.scale_b, dtype=torch.float32, device="cuda") if w.fmt == "e4m3" else None
        dt = {("bf16", "f32"): g.BF16_F32, ("bf16", "bf16"): g.BF16_BF16,
              ("e4m3", "f32"): g.E4M3_F32, ("e4m3", "bf16"): g.E4M3_BF16}[(w.fmt, w.out)]
        self.args = []
        for i in range(self.copies):
            a = g.make_args(self.M, self.N, self.K, A=self.As[i], B=self.Bs[i], C=self.C, dtype=dt,
                            batch=self.batch, stride_a=self.M * self.K, stride_b=self.N * self.K,
                            stride_c=self.M * self.N, scale_a=self.sa, scale_b=self.sb, tile=tile)
            self.args.append(a)
        self.plan = g.gemm355_plan(self.args[0])
        if self.plan["workspace_bytes"]:
            self.ws = torch.empty(self.plan["workspace_bytes"], dtype=torch.uint8, device="cuda")
            for a in self.args:
                a.workspace = self.ws.data_ptr()
                a.workspace_bytes = self.plan["workspace_bytes"]
        self.g = g
        self.i = 0

    def measured_eta(self, torch):
        """One extra call with the per-unit clock hook.  Returns the summed
        busy time of all units over (compute units x resident groups x
        makespan), the shader clock over the units (MHz) and the MFMA
        cycle efficiency inside units: the dense-MFMA cycles of the executed
        (padded) tile work over the measured shader cycles."""
        import numpy as np
        p = self.plan
        if not p["units"]:
            return None
        stamps = torch.zeros(6 * p["units"], dtype=torch.int64, device="cuda")
        a = self.args[0]
        a.unit_stamps = stamps.data_ptr()
        try:
            self.g.gemm355_gemm_ex(a, torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
        finally:
            a.unit_stamps = None
        st = stamps.view(-1, 6).cpu().numpy().astype("float64")
        span = st[:, 1].max() - st[:, 0].min()
        busy_rt = (st[:, 1] - st[:, 0]).sum()
        cycles = (st[:, 3] - st[:, 2]).sum()
        if span <= 0 or busy_rt <= 0 or cycles <= 0:
            return None
        # dense MFMA FLOPs per clock of one compute unit, shared by b groups
        per_clk = (4096.0 if self.fmt == "bf16" else 8192.0) / p["b"]
        ideal = 2.0 * p["T_M"] * p["T_N"] * p["T_K"] * p["G"] * p["nK"] / per_clk
        n = float(len(st))
        xcd = per_xcd(st, p["grid"])
        return {"eta": float(busy_rt / (p["S"] * p["b"] * span)),
                "sclk_mhz": float(100.0 * cycles / busy_rt),
                "mfma_cycle_eff": float(ideal / cycles),
                # mean shader cycles per unit: main loop (prologue included),
                # epilogue until its stores are issued, and their completion
                "unit_cycles": {"loop": round(float((st[:, 4] - st[:, 2]).sum()) / n),
                                "epilogue": round(float((st[:, 5] - st[:, 4]).sum()) / n),
                                "store_drain": round(float((st[:, 3] - st[:, 5]).sum()) / n)},
                "per_xcd": xcd}

    def step(self, stream):
        a = self.args[self.i % self.copies]
        self.i += 1
        self.g.gemm355_gemm_ex(a, stream)

    def name(self):
        shp = "%dx%dx%d" % (self.M, self.N, self.K)
        if self.batch > 1:
            shp = "%dx(%s)" % (self.batch, shp)
        return "%s %s" % (self.w.name, shp)


def settle(case, torch, seconds):
    """Untimed calls for `seconds` of wall time before the warm-up: the shader
    clock rises from idle over some tens of milliseconds of load, so a short
    region right after idle measures the ramp, not the kernel."""
    if seconds <= 0:
        return
    sp = torch.cuda.current_stream().cuda_stream
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            case.step(sp)
        torch.cuda.synchronize()


def time_case(case, torch, steps, warmup, settle_s=0.0):
    """Settle and warm up, then time `steps` back-to-back calls: wall clock
    around the whole region (synchronised on both sides) and one HIP event
    pair on the launch stream around the same calls.  Returns (wall seconds,
    event seconds), both for all `steps` calls."""
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    settle(case, torch, settle_s)
    for _ in range(warmup):
        case.step(sp)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        case.step(sp)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) * 1e-3


def per_call_times(case, torch, calls):
    """After the timed region: `calls` back-to-back calls, each bracketed by
    its own HIP event pair on the launch stream; median and min of the
    per-call durations (events only, no host synchronisation in between)."""
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for e0, e1 in evs:
        e0.record(stream)
        case.step(sp)
        e1.record(stream)
    torch.cuda.synchronize()
    us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
    return {"calls": calls, "median_us": round(us[len(us) // 2], 3), "min_us": round(us[0], 3),
            "max_us": round(us[-1], 3)}


def sample_smi():
    """Socket power (W) and graphics clocks (MHz) from amd-smi, or None."""
    import re
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "--power", "--clock"], capture_output=True, text=True,
                           timeout=20)
    except (OSError, subprocess.TimeoutExpired):
        return None
    txt = r.stdout
    pw = re.findall(r"SOCKET_POWER:\s*([0-9.]+)\s*W", txt)
    gfx = []
    for block in re.split(r"\n\s*GFX_\d+:", txt)[1:]:
        m = re.search(r"^\s*CLK:\s*([0-9.]+)\s*MHz", block, re.M)
        if m:
            gfx.append(float(m.group(1)))
    return {"socket_power_w": float(pw[0]) if pw else None, "gfx_clk_mhz": gfx}


def sustain(case, torch, seconds):
    """Call the case back to back for `seconds` (synchronising every 50
    calls), sample power and clocks half way, and return the sustained time
    per call."""
    import threading
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    smi = {}
    t = threading.Timer(seconds / 2, lambda: smi.update(sample_smi() or {}))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    n = 0
    t0 = time.perf_counter()
    e0.record(stream)
    t.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            case.step(sp)
        n += 50
        torch.cuda.synchronize()
    e1.record(stream)
    torch.cuda.synchronize()
    t.join()
    us = e0.elapsed_time(e1) * 1e3 / n
    return {"sustained_us_per_call": round(us, 2), "sustained_calls": n,
            "sustained_tflops": round(case.flops / us / 1e6, 1), "smi": smi or None}


class _Steps:
    """A callable sequence of launches timed as one step by time_case."""

    def __init__(self, fn, flops):
        self.fn, self.flops = fn, flops

    def step(self, stream):
        self.fn(stream)


def fp8_end_to_end(torch, g, inputs, args):
    """8192^3 products whose operands start as bf16 N(0,1) matrices on the
    device: per-tensor quantisation of A and B on the device (the library's
    quantiser) followed by the 8-bit product with the device scales, timed
    as one step and its parts separately; for E4M3 and for E5M2."""
    import numpy as np
    M = N = K = 8192
    log("bench: detail fp8 end to end", (M, N, K))
    xs = []
    for operand in (0, 1):
        x = inputs.draw(inputs.rng(inputs.seed_for(5, 0, operand)), (M, K), "normal")
        xs.append(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).cuda())
        del x
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    qb = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty(1, dtype=torch.float32, device="cuda")
    sb = torch.empty(1, dtype=torch.float32, device="cuda")
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    flops = 2.0 * M * N * K
    out = []
    for fmt, fq, dt in (("e4m3", g.FP8_E4M3, g.E4M3_F32), ("e5m2", g.FP8_E5M2, g.E5M2_F32)):
        a = g.make_args(M, N, K, A=qa, B=qb, C=C, dtype=dt, scale_a=sa, scale_b=sb)
        p = g.gemm355_plan(a)

        def quant(sp, fq=fq):
            g.gemm355_quantize(xs[0], M * K, 1, g.SRC_BF16, fq, qa, sa, sp)
            g.gemm355_quantize(xs[1], N * K, 1, g.SRC_BF16, fq, qb, sb, sp)

        def gemm(sp, a=a):
            g.gemm355_gemm_ex(a, sp)

        def both(sp):
            quant(sp)
            gemm(sp)

        times = {}
        for name, fn in (("quantize", quant), ("gemm", gemm), ("step", both)):
            c = _Steps(fn, flops)
            n = max(10, args.steps // 10)
            _, ev = time_case(c, torch, n, max(3, args.warmup // 10), args.settle / 4)
            times[name] = ev / n
        out.append({
            "workload": "%s end to end 8192x8192x8192 (bf16 N(0,1) operands quantised on the device, "
                        "then the product, fp32 C)" % fmt,
            "dtype": fmt, "out": "f32",
            "us_median": round(times["step"] * 1e6, 2),
            "us_gemm": round(times["gemm"] * 1e6, 2),
            "us_quantize_a_and_b": round(times["quantize"] * 1e6, 2),
            "quantize_share": round(times["quantize"] / times["step"], 4),
            "tflops": round(flops / times["step"] / 1e12, 1),
            "tflops_gemm_only": round(flops / times["gemm"] / 1e12, 1),
            "pct_mfma_peak": round(100 * flops / times["step"] / 1e12 / PEAK_TFLOPS["e4m3"], 1),
            # quantiser bytes: read bf16 A and B twice (amax, then quantise), write the codes
            "quantize_hbm_gbs": round((2 * 2 * (M + N) * K + (M + N) * K) / times["quantize"] / 1e9, 1),
            "tile": [p["T_M"], p["T_N"], p["T_K"]], "split": p["split"],
        })
        if not args.no_cpu_baseline:
            from types import SimpleNamespace
            from oracle import quant as quant_oracle
            xa = xs[0].float().cpu().numpy().reshape(-1)
            q_cpu = sampled_oracle(lambda n: quant_oracle.quantize(xa[:n * 65536], fmt), M * K // 65536, 65536.0,
                                   2.0 * M * K / 65536, "gelem_s",
                                   "the first %d x 65536 elements of A (maximum, scale, codes)")
            torch.cuda.synchronize()
            ops_q = SimpleNamespace(M=M, N=N, K=K, A=qa.cpu().numpy(), B=qb.cpu().numpy(), fmt=fmt, fmt_a=fmt,
                                    fmt_b=fmt, batch=1)
            out[-1]["cpu_oracle"] = {"quantize": q_cpu, "gemm": oracle_sample(ops_q, budget_s=1.0),
                                     "full_s_estimate": None}
            out[-1]["cpu_oracle"]["full_s_estimate"] = round(
                q_cpu["full_s_estimate"] + out[-1]["cpu_oracle"]["gemm"]["full_s_estimate"], 2)
            del xa, ops_q
    del xs
    torch.cuda.empty_cache()
    return out


def mx_products(torch, g, inputs, args):
    """8192^3 block-scaled products (E8M0 scale per 32 K-values of each row
    of A and column of B), E4M3, E5M2, FP6 (E2M3, E3M2) and FP4 (E2M1)
    elements, fp32 C, timed
    like the per-tensor E4M3 product beside them (same shape, same box)."""
    import numpy as np
    M = N = K = 8192
    flops = 2.0 * M * N * K
    out = []
    for fmt, dt in (("mxe4m3", g.MXE4M3_F32), ("mxe5m2", g.MXE5M2_F32), ("mxfp6e2m3", g.MXFP6_E2M3_F32),
                    ("mxfp6e3m2", g.MXFP6_E3M2_F32), ("mxfp4", g.MXFP4_F32)):
        log("bench: detail block-scaled", fmt, (M, N, K))
        ops = inputs.make_operands(M, N, K, fmt, "normal", inputs.seed_for(6, 0, 0), inputs.seed_for(6, 0, 1))
        A = torch.from_numpy(ops.A).cuda()
        B = torch.from_numpy(ops.B).cuda()
        sa = torch.from_numpy(ops.bsa).cuda()
        sb = torch.from_numpy(ops.bsb).cuda()
        cpu = None
        if not args.no_cpu_baseline:
            from oracle import mx as mx_oracle
            ncol = 1024
            Bc, sbc = ops.B[:ncol], ops.bsb[:ncol]
            cpu = sampled_oracle(
                lambda n: mx_oracle.gemm(ops.A[:n], ops.bsa[:n], Bc, sbc, ops.fmt_a, ops.fmt_b), M,
                2.0 * ncol * K, M * (N / ncol), "gflops",
                "the first %%d rows x the first %d columns of the product (binary64 values decoded from "
                "codes and block scales, then one matrix product)" % ncol)
        del ops
        C = torch.empty((M, N), dtype=torch.float32, device="cuda")
        a = g.make_args(M, N, K, A=A, B=B, C=C, dtype=dt, block_scale_a=sa, block_scale_b=sb)
        p = g.gemm355_plan(a)
        c = _Steps(lambda sp, a=a: g.gemm355_gemm_ex(a, sp), flops)
        settle(c, torch, args.settle / 2)
        reps = []
        for _ in range(3):
            n = max(10, args.steps // 10)
            _, ev = time_case(c, torch, n, max(3, args.warmup // 10))
            reps.append(ev / n)
        reps.sort()
        med = reps[1]
        out.append({
            "workload": "%s 8192x8192x8192 (block-scaled: E8M0 scale per 32 K-values, entries N(0,1) "
                        "quantised per block, fp32 C)" % fmt,
            "dtype": fmt, "out": "f32", "us_median": round(med * 1e6, 2), "us_min": round(reps[0] * 1e6, 2),
            "tflops": round(flops / med / 1e12, 1),
            "pct_mfma_peak": round(100 * flops / med / 1e12 / PEAK_TFLOPS["e4m3" if fmt in ("mxe4m3", "mxe5m2") else "fp4"], 1),
            "tile": [p["T_M"], p["T_N"], p["T_K"]], "split": p["split"], "grid": p["grid"],
        })
        if cpu is not None:
            out[-1]["cpu_oracle"] = cpu
        del A, B, sa, sb, C
        torch.cuda.empty_cache()
    return out


def conv_layers(torch, g, inputs, args):
    """Implicit-GEMM convolutions (bf16 NHWC images and KRSC filters, fp32
    accumulate, bf16 NPQK output) of ResNet-like shapes, each next to the
    plain product of the same M x N x K (A given as a matrix) on the same
    box."""
    import numpy as np
    layers = [
        # N, H, W, C, K, R, S, pad
        (32, 56, 56, 128, 128, 3, 3, 1),
        (64, 28, 28, 256, 256, 3, 3, 1),
        (32, 56, 56, 256, 64, 1, 1, 0),
    ]
    out = []
    for (N, Hh, W, C, K, R, S, pad) in layers:
        log("bench: detail convolution", (N, Hh, W, C, K, R, S, pad))
        P, Q = g.gemm355_conv2d_out_size(g.make_conv_args(N, Hh, W, C, K, R, S, pad_h=pad, pad_w=pad))
        M, Kg = N * P * Q, R * S * C
        flops = 2.0 * M * K * Kg
        gen = np.random.Generator(np.random.PCG64(7000 + C + K + R))
        x = torch.from_numpy(gen.standard_normal((N, Hh, W, C), dtype=np.float32)).to(torch.bfloat16).cuda()
        w = torch.from_numpy(gen.standard_normal((K, R, S, C), dtype=np.float32)).to(torch.bfloat16).cuda()
        y = torch.empty((N, P, Q, K), dtype=torch.bfloat16, device="cuda")
        a = g.make_conv_args(N, Hh, W, C, K, R, S, x=x, w=w, y=y, pad_h=pad, pad_w=pad, dtype=g.BF16_BF16)
        p = g.gemm355_conv2d_plan(a)
        A = torch.empty((M, Kg), dtype=torch.bfloat16, device="cuda").normal_()
        ga = g.make_args(M, K, Kg, A=A, B=w, C=y, dtype=g.BF16_BF16)
        res = {}
        for name, fn in (("conv", lambda sp, a=a: g.gemm355_conv2d(a, sp)),
                         ("gemm", lambda sp, ga=ga: g.gemm355_gemm_ex(ga, sp))):
            c = _Steps(fn, flops)
            settle(c, torch, args.settle / 4)
            reps = []
            for _ in range(3):
                n = max(10, args.steps // 10)
                _, ev = time_case(c, torch, n, max(3, args.warmup // 10))
                reps.append(ev / n)
            reps.sort()
            res[name] = reps[1]
        out.append({
            "workload": "convolution N=%d %dx%dx%d -> %d, %dx%d filter, pad %d (implicit GEMM M=%d N=%d K=%d, "
                        "bf16 in, bf16 out)" % (N, Hh, W, C, K, R, S, pad, M, K, Kg),
            "dtype": "bf16", "out": "bf16", "us_median": round(res["conv"] * 1e6, 2),
            "tflops": round(flops / res["conv"] / 1e12, 1),
            "pct_mfma_peak": round(100 * flops / res["conv"] / 1e12 / PEAK_TFLOPS["bf16"], 1),
            "us_same_size_gemm": round(res["gemm"] * 1e6, 2),
            "tile": [p["T_M"], p["T_N"], p["T_K"]], "split": p["split"], "grid": p["grid"],
        })
        if not args.no_cpu_baseline:
            from oracle import conv as conv_oracle
            xc = x.view(torch.int16).cpu().numpy().view(np.uint16)
            wc = w.view(torch.int16).cpu().numpy().view(np.uint16)
            out[-1]["cpu_oracle"] = sampled_oracle(
                lambda n: conv_oracle.conv2d(xc[:n], wc, pad, pad), N, 2.0 * P * Q * K * Kg, N, "gflops",
                "the first %d images (binary64, one matrix product per filter tap)")
        del x, w, y, A
        torch.cuda.empty_cache()
    return out


def _numpy_threads():
    """Threads of the BLAS numpy calls into (the oracle's matrix products)."""
    try:
        from threadpoolctl import threadpool_info
        n = sum(x.get("num_threads", 0) for x in threadpool_info() if x.get("user_api") == "blas")
        if n:
            return n
    except Exception:   # threadpoolctl missing or unreadable: report the affinity set
        pass
    return len(os.sched_getaffinity(0))


def sampled_oracle(run, n_max, work_per_item, full_items, unit, label, budget_s=1.0):
    """Time the oracle (as it stands) on a bounded sample: run(n) computes n
    items (rows, images, elements) of a workload of full_items; a probe at a
    small n sizes the sample to about budget_s.  Returns seconds, the rate in
    `unit` (work_per_item per item) and the full workload's time at that
    rate."""
    n0 = max(1, min(n_max, 8))
    t0 = time.perf_counter()
    run(n0)
    probe = max(time.perf_counter() - t0, 1e-6)
    n = int(min(n_max, max(n0, n0 * budget_s / probe)))
    t0 = time.perf_counter()
    run(n)
    t = time.perf_counter() - t0
    if t < budget_s / 3 and n < n_max:
        # the probe carried one-time costs: size once more from this run
        n = int(min(n_max, n * budget_s / max(t, 1e-6)))
        t0 = time.perf_counter()
        run(n)
        t = time.perf_counter() - t0
    return {"seconds": round(t, 3), unit: round(n * work_per_item / t / 1e9, 3), "cores": _numpy_threads(),
            "sample": label % (n,), "full_s_estimate": round(t * full_items / n, 2)}


def oracle_sample(ops, budget_s=2.0):
    """The oracle (as it stands) on a bounded sample of one workload: the
    first R rows of A (R from a 16-row probe, about budget_s seconds) against
    all of B, of the first batch entry.  Returns the sample's wall seconds,
    its oracle GFLOP/s and the full workload's time at that rate."""
    from oracle import reference as oracle
    M, N, K = ops.M, ops.N, ops.K
    A = ops.A[0] if ops.A.ndim == 3 else ops.A
    B = ops.B[0] if ops.B.ndim == 3 else ops.B
    kw = {} if ops.fmt == "bf16" else {"fmt_a": ops.fmt_a, "fmt_b": ops.fmt_b}
    # two probes separate the fixed cost (decoding all of B) from the per-row cost
    times = []
    probes = (min(M, 8), min(M, 24))
    for r in probes:
        t0 = time.perf_counter()
        oracle.gemm(r, N, K, A[:r].reshape(-1), K, B.reshape(-1), K, **kw)
        times.append(time.perf_counter() - t0)
    per_row = max((times[1] - times[0]) / max(probes[1] - probes[0], 1), 1e-7)
    fixed = max(times[0] - probes[0] * per_row, 0.0)
    rows = int(min(M, max(probes[1], budget_s / per_row)))
    t0 = time.perf_counter()
    oracle.gemm(rows, N, K, A[:rows].reshape(-1), K, B.reshape(-1), K, **kw)
    t = time.perf_counter() - t0
    gflops = 2.0 * rows * N * K / t / 1e9
    per_row = max((t - fixed) / rows, 1e-9)
    full = ops.batch * (fixed + per_row * M)
    return {"seconds": round(t, 3), "gflops": round(gflops, 2), "cores": oracle.threads(),
            "sample": "rows 0..%d of %s (binary64 triple loop with W, decode of all of B included)" % (
                rows - 1, "batch entry 0" if ops.batch > 1 else "the product"),
            "full_s_estimate": round(full, 2)}


def cpu_baseline(torch, budget_s=15.0):
    """The oracle (as it stands) on a bounded sample of the headline product:
    the first R rows of A against all of B, R sized from a short probe to
    take roughly budget_s seconds."""
    import numpy as np
    from dense_tiled_gemm_fp8_amd import inputs
    from oracle import reference as oracle
    w = inputs.WORKLOADS[1]
    ops = inputs.workload_operands(w)
    M, N, K = ops.M, ops.N, ops.K
    # two probes separate the fixed cost (decoding all of B) from the per-row cost
    times = []
    for r in (16, 48):
        t0 = time.perf_counter()
        oracle.gemm(r, N, K, ops.A[:r].reshape(-1), K, ops.B.reshape(-1), K)
        times.append(time.perf_counter() - t0)
    per_row = max((times[1] - times[0]) / 32, 1e-6)
    fixed = max(times[0] - 16 * per_row, 0.0)
    rows = int(min(M, max(16, (budget_s - fixed) / per_row)))
    rows = max(16, rows // 16 * 16)
    t0 = time.perf_counter()
    oracle.gemm(rows, N, K, ops.A[:rows].reshape(-1), K, ops.B.reshape(-1), K)
    t = time.perf_counter() - t0
    return {"value": round(2.0 * rows * N * K / t / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.threads(), "kind": "oracle",
            "sample": "rows 0..%d of the bf16 4096x4096x4096 product (%d x 4096 x 4096 multiply-adds, "
                      "binary64 triple loop, decode of all of B included), %.1f s" % (rows - 1, rows, t)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU; --gpus %d is not supported (the product would shard by "
              "row blocks of C, one per GPU, each running this library on its block)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_bytes:
        copy_reference(args.copy_bytes)
        return
    if args.pass_floor:
        pass_floor(args.pass_floor)
        return
    import numpy as np
    import torch
    from dense_tiled_gemm_fp8_amd import gemm355 as g
    from dense_tiled_gemm_fp8_amd import inputs

    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)

    if args.profile:
        name, _, si = args.profile.partition(":")
        w = next(x for x in inputs.WORKLOADS if x.name == name)
        c = Case(w, int(si or 0), torch, g, inputs, tile=args.tile)
        if args.vendor:
            if w.fmt != "bf16" or c.batch != 1:
                sys.exit("--vendor: bf16 single products only")
            # the same operand copies in turn as the library's calls (cold
            # inputs on memory-bound shapes); fp32 C through the bf16 x bf16
            # -> fp32 product
            Avs = [x.view(torch.bfloat16) for x in c.As]
            Bvs = [x.view(torch.bfloat16).t() for x in c.Bs]

            def vendor_step(stream):
                i = c.i % c.copies
                c.i += 1
                if c.C.dtype == torch.float32:
                    torch.mm(Avs[i], Bvs[i], out_dtype=torch.float32)
                else:
                    torch.matmul(Avs[i], Bvs[i], out=c.C)
            c.step = vendor_step
        _, ev = time_case(c, torch, args.steps, args.warmup, args.settle or 0.0)
        me = c.measured_eta(torch) if args.stamps and not args.vendor else None
        out = {"workload": c.name(), "us_per_call": round(ev / args.steps * 1e6, 2),
               "tile": c.plan["tile"], "split": c.plan["split"],
               "tail": [c.plan["tail_tiles"], c.plan["tail_split"]], "measured": me,
               "vendor": bool(args.vendor)}
        if args.sustain > 0:
            out.update(sustain(c, torch, args.sustain))
        print(json.dumps(out), flush=True)
        return

    head_w = inputs.WORKLOADS[1]
    log("bench: building inputs for", head_w.name)
    head = Case(head_w, 0, torch, g, inputs)
    log("bench: plan", {k: head.plan[k] for k in ("tile", "T_M", "T_N", "T_K", "G", "grid", "split")})
    torch.cuda.synchronize()
    # timed region: barrier (single rank) + synchronize on both sides
    if args.settle is None:
        args.settle = 0.5
    wall, ev = time_case(head, torch, args.steps, args.warmup, args.settle)
    ms_per_step = wall / args.steps * 1e3
    value = head.flops * args.steps / wall / 1e12
    kern_avg = ev / args.steps
    achieved = head.flops / kern_avg / 1e12
    log("bench: %.3f ms/step wall, kernel avg %.2f us, %.1f TFLOP/s" % (ms_per_step, kern_avg * 1e6, achieved))
    per_call = per_call_times(head, torch, max(args.steps, 20))
    log("bench: per-call kernel us median %.2f min %.2f" % (per_call["median_us"], per_call["min_us"]))

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_hash") == kernel_hash():
            traffic = tr.get("bytes_per_launch")

    detail = []
    if not args.no_detail:
        for w in inputs.WORKLOADS:
            for si in range(len(w.shapes)):
                if args.workload and args.workload != w.name:
                    continue
                log("bench: detail", w.name, w.shapes[si])
                c = head if (w is head_w and si == 0) else Case(w, si, torch, g, inputs)
                # three timed repetitions; the median of their per-call averages
                settle(c, torch, args.settle / 2)
                reps = []
                for _ in range(3):
                    n = max(10, args.steps // 2)
                    _, ev_c = time_case(c, torch, n, max(3, args.warmup // 2))
                    reps.append(ev_c / n)
                reps.sort()
                med = reps[1]
                p = c.plan
                detail.append({
                    "workload": c.name(), "dtype": w.fmt, "out": w.out,
                    "us_median": round(med * 1e6, 2), "us_min": round(reps[0] * 1e6, 2),
                    "tflops": round(c.flops / med / 1e12, 1),
                    "pct_mfma_peak": round(100 * c.flops / med / 1e12 / PEAK_TFLOPS[w.fmt], 1),
                    "hbm_gbs": round(c.alg_bytes / med / 1e9, 1),
                    "bound": "hbm" if c.hbm_bound else "mfma", "rotated_copies": c.copies,
                    "tile": [p["T_M"], p["T_N"], p["T_K"]], "b": p["b"], "split": p["split"],
                    "persistent": p["persistent"], "tail": [p["tail_tiles"], p["tail_split"]],
                    "grid": p["grid"], "units": p["units"],
                    "eta_wave": [p["eta_wave_num"], p["eta_wave_den"]],
                    "eta_pad": [p["eta_pad_num"], p["eta_pad_den"]],
                    "eta_sched": [p["eta_sched_num"], p["eta_sched_den"]],
                })
                if not args.no_cpu_baseline:
                    detail[-1]["cpu_oracle"] = oracle_sample(c.ops)
                me = c.measured_eta(torch)
                detail[-1]["eta_measured"] = None if me is None else round(me["eta"], 4)
                detail[-1]["sclk_mhz"] = None if me is None else round(me["sclk_mhz"], 0)
                detail[-1]["mfma_cycle_eff"] = None if me is None else round(me["mfma_cycle_eff"], 4)
                detail[-1]["unit_cycles"] = None if me is None else me["unit_cycles"]
                detail[-1]["per_xcd"] = None if me is None else me["per_xcd"]
                if c is not head:
                    del c
                    torch.cuda.empty_cache()

    if not args.no_detail and (args.workload in (None, "fp8-end-to-end")):
        detail.extend(fp8_end_to_end(torch, g, inputs, args))
    if not args.no_detail and (args.workload in (None, "block-scaled")):
        detail.extend(mx_products(torch, g, inputs, args))
    if not args.no_detail and (args.workload in (None, "convolution")):
        detail.extend(conv_layers(torch, g, inputs, args))

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline")
        cpu = cpu_baseline(torch)

    p = head.plan
    line = {
        "metric": "GEMM TFLOP/s and % of MFMA peak (bf16 4096^3; skinny split-K shapes)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_s": args.settle, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "bf16 GEMM 4096x4096x4096, A row-major, B column-major, C bf16, "
                               "fp32 accumulate, entries N(0,1) rounded to bf16",
                   "M": 4096, "N": 4096, "K": 4096, "tile": [p["T_M"], p["T_N"], p["T_K"]],
                   "grid": p["grid"], "split_k": p["split"],
                   "eta_wave": p["eta_wave_num"] / p["eta_wave_den"],
                   "eta_pad": p["eta_pad_num"] / p["eta_pad_den"]},
        "pct_of_peak": round(100 * value / PEAK_TFLOPS["bf16"], 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
                     "traffic": traffic, "kernel_us": round(kern_avg * 1e6, 3)},
        "per_call_kernel_us": per_call,
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
