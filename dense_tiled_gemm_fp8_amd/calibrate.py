"""Refit the planner's tile priors from timed forced plans on this device.

    python -m dense_tiled_gemm_fp8_amd.calibrate sweep OUT.json [--groups bf16,e4m3,conv]
    python -m dense_tiled_gemm_fp8_amd.calibrate fit OUT.json [--per-tile]

sweep (GPU): for each calibration shape of a group, every tile of the group,
one-shot and persistent, timed with HIP events around a sustained loop.
Products bound by memory rotate through operand copies of twice the 256 MB
last-level cache, as the benchmark does; convolutions read one copy.  Each
record keeps the plan the library made for the forced knobs, including the
inputs of its time estimate (gemm355_plan_t.model_*).

fit (CPU): per tile a new stream_eff, per group one scale of the mfma_eff
priors and one per-unit fill and epilogue time, minimising the squared log
error of the planning model against the timings, weighted toward plans
within 30 % of their shape's best (--per-tile: one mfma_eff scale per tile;
more parameters than the sweep pins down, so the picks it gives are not
better overall).  It prints the refitted priors (to be
written into csrc/tiles.h, and the per-unit time into csrc/plan.hip) and,
per shape, the measured time of the model's pick among the timed plans over
the best timed plan, with the current and with the refitted priors.
"""
import argparse
import json
import math
import sys
import time

HBM_PLAN = 5.0e12                 # planning rate of the model, bytes/s
GROUPS = ("bf16", "e4m3", "conv")
SHAPES = {
    # M x N x K (x batch); the named products plus short-K, narrow-N and
    # mid-size ones
    "bf16": [(100352, 64, 256, 1), (100352, 128, 1152, 1), (50176, 256, 2304, 1), (1000, 3000, 777, 1),
             (4096, 4096, 4096, 1), (256, 256, 65536, 1), (128, 512, 131072, 1), (64, 64, 262144, 1),
             (8192, 8192, 1024, 1), (16384, 512, 512, 1), (2048, 2048, 2048, 1), (4096, 1024, 512, 1),
             (32768, 256, 1024, 1), (3072, 3072, 3072, 1), (768, 3072, 2048, 1), (2560, 1024, 2048, 1),
             (6144, 6144, 1024, 1), (768, 1000, 1024, 1)],
    "e4m3": [(8192, 8192, 8192, 1), (512, 1024, 4096, 64), (256, 256, 131072, 1), (100352, 128, 2304, 1),
             (16384, 512, 1024, 1), (2048, 2048, 2048, 1), (4096, 1024, 1024, 1), (32768, 256, 2048, 1),
             (64, 64, 524288, 1), (512, 3000, 4096, 1), (4096, 2560, 4096, 1)],
    # N, H, W, C, K, R, S, pad: ResNet-like layers
    "conv": [(32, 56, 56, 128, 128, 3, 3, 1), (64, 28, 28, 256, 256, 3, 3, 1), (32, 56, 56, 256, 64, 1, 1, 0),
             (32, 56, 56, 64, 64, 3, 3, 1), (32, 14, 14, 512, 512, 3, 3, 1), (64, 56, 56, 64, 256, 1, 1, 0),
             (32, 28, 28, 128, 512, 1, 1, 0), (8, 112, 112, 64, 128, 3, 3, 1)],
}
PLAN_KEYS = ("tile", "split", "persistent", "grid", "b", "units", "model_seconds", "model_mfma_peak_seconds",
             "model_mfma_eff", "model_bytes", "model_spread", "model_stream_eff", "model_copy_seconds",
             "model_fixed_seconds", "model_units_in_turn")


def group_tiles(g, group):
    out = []
    t = 0
    while True:
        try:
            info = g.gemm355_tile_info(t)
        except Exception:
            break
        cls, op = info["dtype_class"], info["op"]
        if (group == "bf16" and cls == 0 and op == 0) or (group == "e4m3" and cls == 1 and op == 0) or \
                (group == "conv" and cls == 0 and op == 1):
            out.append(t)
        t += 1
    return out


def _timed(torch, step, warm_s=0.08, run_s=0.25):
    t0 = time.time()
    while time.time() - t0 < warm_s:
        step()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 0
    t0 = time.time()
    e0.record()
    while time.time() - t0 < run_s:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e-3


def sweep(out_path, groups):
    import torch
    from dense_tiled_gemm_fp8_amd import gemm355 as g
    torch.cuda.set_device(0)
    ws = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
    recs = []
    for group in groups:
        tiles = group_tiles(g, group)
        for shape in SHAPES[group]:
            if group == "conv":
                N, H, W, C, K, R, S, pad = shape
                P, Q = g.gemm355_conv2d_out_size(g.make_conv_args(N, H, W, C, K, R, S, pad_h=pad, pad_w=pad))
                x = torch.randn(N, H, W, C, device="cuda").bfloat16()
                w = torch.randn(K, R, S, C, device="cuda").bfloat16()
                y = torch.empty(N, P, Q, K, device="cuda", dtype=torch.bfloat16)
                mk = lambda t, pers: [g.make_conv_args(N, H, W, C, K, R, S, x=x, w=w, y=y, pad_h=pad, pad_w=pad,
                                                       dtype=g.BF16_BF16, tile=t, persistent=pers, workspace=ws,
                                                       workspace_bytes=ws.numel())]
                plan, run = g.gemm355_conv2d_plan, g.gemm355_conv2d
            else:
                M, N, K, bt = shape
                esz, osz = (2, 2) if group == "bf16" else (1, 4)
                flops = 2.0 * M * N * K * bt
                inb = (M + N) * K * bt * esz
                peak = 2516.6e12 if group == "bf16" else 5033.2e12
                memory_bound = flops / (inb + M * N * bt * osz) < peak / 8e12
                ncp = max(1, -(-2 * 256 * 2 ** 20 // inb)) if memory_bound else 1
                if group == "bf16":
                    As = [torch.randn(bt, M, K, device="cuda").bfloat16() for _ in range(ncp)]
                    Bs = [torch.randn(bt, N, K, device="cuda").bfloat16() for _ in range(ncp)]
                    dt = g.BF16_BF16
                else:
                    As = [torch.randint(0, 0x70, (bt, M, K), dtype=torch.uint8, device="cuda") for _ in range(ncp)]
                    Bs = [torch.randint(0, 0x70, (bt, N, K), dtype=torch.uint8, device="cuda") for _ in range(ncp)]
                    dt = g.E4M3_F32
                Cm = torch.empty(bt, M, N, device="cuda", dtype=torch.bfloat16 if group == "bf16" else torch.float32)
                mk = lambda t, pers: [g.make_args(M, N, K, A=As[i], B=Bs[i], C=Cm, dtype=dt, batch=bt,
                                                  stride_a=M * K, stride_b=N * K, stride_c=M * N, tile=t,
                                                  persistent=pers, workspace=ws, workspace_bytes=ws.numel())
                                      for i in range(ncp)]
                plan, run = g.gemm355_plan, g.gemm355_gemm_ex
            for t in tiles:
                for pers in (0, 1):
                    al = mk(t, pers)
                    try:
                        p = plan(al[0])
                    except g.Gemm355Error:
                        continue
                    it = [0]

                    def step():
                        run(al[it[0] % len(al)])
                        it[0] += 1
                    sec = _timed(torch, step)
                    rec = dict(group=group, shape=list(shape), seconds=sec, **{k: p[k] for k in PLAN_KEYS})
                    recs.append(rec)
                    print(json.dumps(rec), flush=True)
            torch.cuda.empty_cache()
    with open(out_path, "w") as f:
        json.dump(recs, f)


def predict(r, f_mfma, stream_eff, unit_s):
    t_m = r["model_mfma_peak_seconds"] / (r["model_mfma_eff"] * f_mfma)
    t_b = r["model_bytes"] / (HBM_PLAN * stream_eff * r["model_spread"])
    t_c = r["model_copy_seconds"]
    return r["model_fixed_seconds"] + (t_m ** 4 + t_b ** 4 + t_c ** 4) ** 0.25 + r["model_units_in_turn"] * unit_s


def fit_group(recs, cap=2.5, sweeps=8, per_tile=False):
    """Coordinate descent on grids: per tile stream_eff, one mfma scale (per
    tile too with per_tile), one per-unit time.  Returns (f_mfma, {tile:
    stream_eff}, unit_s, rms); f_mfma is a {tile: scale} dict with per_tile."""
    best = {}
    for r in recs:
        k = tuple(r["shape"])
        best[k] = min(best.get(k, math.inf), r["seconds"])
    w = [1.0 if r["seconds"] <= 1.3 * best[tuple(r["shape"])] else 0.2 for r in recs]

    def loss(fm, fs, u, idx=None):
        s = n = 0.0
        for i in (range(len(recs)) if idx is None else idx):
            r = recs[i]
            e = math.log(predict(r, fm[r["tile"]] if per_tile else fm, fs[r["tile"]], u) / r["seconds"])
            s += w[i] * e * e
            n += w[i]
        return s / max(n, 1e-30)

    tiles = sorted(set(r["tile"] for r in recs))
    by_tile = {t: [i for i, r in enumerate(recs) if r["tile"] == t] for t in tiles}
    fm, u = ({t: 1.0 for t in tiles} if per_tile else 1.0), 3e-6
    fs = {t: recs[by_tile[t][0]]["model_stream_eff"] for t in tiles}
    grid_s = [x / 100 for x in range(20, int(cap * 100) + 1, 2)]
    grid_m = [x / 100 for x in range(20, 161, 2)]
    grid_u = [x * 0.5e-6 for x in range(0, 11)]
    for _ in range(sweeps):
        for t in tiles:
            fs[t] = min(grid_s, key=lambda a: loss(fm, {**fs, t: a}, u, by_tile[t]))
            if per_tile:
                fm[t] = min(grid_m, key=lambda a: loss({**fm, t: a}, fs, u, by_tile[t]))
        if not per_tile:
            fm = min(grid_m, key=lambda a: loss(a, fs, u))
        u = min(grid_u, key=lambda a: loss(fm, fs, a))
    return fm, fs, u, math.sqrt(loss(fm, fs, u))


def picks(recs, fm=1.0, fs=None, u=None):
    """Per shape: measured time of the plan the model ranks fastest among the
    timed ones, over the best timed plan."""
    out = {}
    for k in sorted(set(tuple(r["shape"]) for r in recs)):
        rs = [r for r in recs if tuple(r["shape"]) == k]
        if fs is None:
            pick = min(rs, key=lambda r: r["model_seconds"])
        else:
            pick = min(rs, key=lambda r: predict(r, fm[r["tile"]] if isinstance(fm, dict) else fm, fs[r["tile"]], u))
        out[k] = pick["seconds"] / min(r["seconds"] for r in rs)
    return out


def fit(path, per_tile=False):
    recs = json.load(open(path))
    for group in GROUPS:
        rs = [r for r in recs if r["group"] == group]
        if not rs:
            continue
        fm, fs, u, rms = fit_group(rs, per_tile=per_tile)
        scale = (lambda t: fm[t]) if per_tile else (lambda t: fm)
        print("%s: %d timed plans, rms log error %.3f, %s, per-unit time %.1f us"
              % (group, len(rs), rms, "per-tile mfma_eff scales" if per_tile else "mfma_eff scale %.2f" % fm,
                 u * 1e6))
        for t in sorted(fs):
            old = next(r["model_stream_eff"] for r in rs if r["tile"] == t)
            print("  tile %2d: stream_eff %.2f -> %.2f, mfma_eff x %.2f" % (t, old, fs[t], scale(t)))
        before, after = picks(rs), picks(rs, fm, fs, u)
        for k in before:
            print("  %-32s model's pick / best: %.2f -> %.2f" % ("x".join(map(str, k)), before[k], after[k]))
        gm = lambda d: math.exp(sum(math.log(v) for v in d.values()) / len(d))
        print("  geometric mean %.3f -> %.3f" % (gm(before), gm(after)))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("sweep")
    s.add_argument("out")
    s.add_argument("--groups", default=",".join(GROUPS))
    f = sub.add_parser("fit")
    f.add_argument("path")
    f.add_argument("--per-tile", action="store_true", help="one mfma_eff scale per tile")
    a = ap.parse_args(argv)
    if a.cmd == "sweep":
        sweep(a.out, [x for x in a.groups.split(",") if x])
    else:
        fit(a.path, a.per_tile)
    return 0


if __name__ == "__main__":
    sys.exit(main())
