"""The calibration's sweep on the GPU, cut down to one product and one
convolution with two tiles each: every record carries a timing and its
plan's model inputs, which reproduce the plan's estimate."""
import json

import pytest

from tests.test_calibrate import unit_seconds

pytestmark = pytest.mark.gpu


def test_sweep_records(tmp_path, monkeypatch):
    from dense_tiled_gemm_fp8_amd import calibrate
    monkeypatch.setitem(calibrate.SHAPES, "bf16", [(512, 256, 1024, 1)])
    monkeypatch.setitem(calibrate.SHAPES, "conv", [(2, 14, 14, 64, 64, 3, 3, 1)])
    monkeypatch.setattr(calibrate, "group_tiles", lambda g, group: [1, 2] if group == "bf16" else [55, 56])
    out = tmp_path / "sweep.json"
    calibrate.sweep(str(out), ["bf16", "conv"])
    recs = json.load(open(out))
    assert sorted((r["group"], r["tile"], r["persistent"]) for r in recs) == sorted(
        (grp, t, p) for grp, ts in (("bf16", (1, 2)), ("conv", (55, 56))) for t in ts for p in (0, 1))
    u = unit_seconds()
    for r in recs:
        assert 0 < r["seconds"] < 0.01
        assert calibrate.predict(r, 1.0, r["model_stream_eff"], u) == pytest.approx(r["model_seconds"], rel=1e-9)
