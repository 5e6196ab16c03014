"""The benchmark end to end on the tiny workload: one JSON line with the
fields the measurement contract asks for, parity against the oracle, and a
roofline figure within the physically possible range."""
from __future__ import annotations

import json

import pytest

import bench

pytestmark = pytest.mark.gpu


def test_bench_json_line(capsys):
    assert bench.main(["--config", "1", "--steps", "16", "--warmup", "8", "--reps", "1"]) == 0
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    out = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "parity"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 16 and out["warmup"] == 8
    assert out["config"]["workload"] == "tiny-gdn-d64"
    assert out["value"] > 0 and out["ms_per_step"] > 0
    roof = out["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0.0 < roof["frac"] <= 1.0 and roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"])
    cpu = out["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert all(p["ok"] for p in out["parity"].values())
