"""The plan reports the inputs of its time estimate, and the calibration's
fit recovers priors planted in synthetic timings (host only)."""
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BASE = dict(A=0x10000, B=0x1000000000, C=0x200000000000, cus=256)


@pytest.fixture(scope="module")
def g():
    from dense_tiled_gemm_fp8_amd import gemm355
    return gemm355


def unit_seconds():
    src = open(os.path.join(ROOT, "dense_tiled_gemm_fp8_amd", "csrc", "plan.hip")).read()
    return float(re.search(r"kUnitSec = ([0-9.eE+-]+);", src).group(1))


SHAPES = [(4096, 4096, 4096), (100352, 64, 256), (1000, 3000, 777), (256, 256, 65536), (2048, 2048, 2048),
          (50176, 256, 2304), (64, 64, 262144)]


def test_model_inputs_reproduce_the_estimate(g):
    from dense_tiled_gemm_fp8_amd import calibrate
    u = unit_seconds()
    for (M, N, K) in SHAPES:
        for dt in (g.BF16_BF16, g.E4M3_F32):
            for knobs in (dict(), dict(persistent=1), dict(split_k=4)):
                p = g.gemm355_plan(g.make_args(M, N, K, dtype=dt, **BASE, **knobs))
                t = calibrate.predict(p, 1.0, p["model_stream_eff"], u)
                assert t == pytest.approx(p["model_seconds"], rel=1e-12), (M, N, K, dt, knobs)
                assert p["model_units_in_turn"] == math.ceil(p["units"] / min(p["grid"], p["S"] * p["b"]))
    a = g.make_conv_args(32, 56, 56, 256, 64, 1, 1, x=0x10000, w=0x1000000000, y=0x200000000000,
                         dtype=g.BF16_BF16)
    p = g.gemm355_conv2d_plan(a)
    assert calibrate.predict(p, 1.0, p["model_stream_eff"], u) == pytest.approx(p["model_seconds"], rel=1e-12)


def test_fit_recovers_planted_priors(g):
    """Timings made by the model itself with an MFMA scale of 0.8, a per-unit
    time of 2 us and per-tile stream rates: the fit finds the scale and the
    per-unit time, and reproduces every timing."""
    from dense_tiled_gemm_fp8_amd import calibrate
    tiles = calibrate.group_tiles(g, "bf16")
    planted = {t: 0.9 + 0.04 * (i % 10) for i, t in enumerate(tiles)}
    recs = []
    for (M, N, K) in SHAPES:
        for t in tiles:
            for pers in (0, 1):
                try:
                    p = g.gemm355_plan(g.make_args(M, N, K, dtype=g.BF16_BF16, tile=t, persistent=pers, **BASE))
                except g.Gemm355Error:
                    continue
                r = dict(shape=[M, N, K], **{k: p[k] for k in calibrate.PLAN_KEYS})
                r["seconds"] = calibrate.predict(r, 0.8, planted[t], 2e-6)
                recs.append(r)
    fm, fs, u, rms = calibrate.fit_group(recs, sweeps=3)
    assert fm == pytest.approx(0.8) and u == pytest.approx(2e-6)
    assert rms < 1e-3
    after = calibrate.picks(recs, fm, fs, u)
    assert all(v == pytest.approx(1.0) for v in after.values())
