"""The benchmark's JSON line, run in-process on the tiny workload (two
layers, a few steps): every field the line promises is present, typed as
stated, and consistent with the others (throughput from the step time, the
roofline fraction from the achieved rate and the peak)."""
import json
import sys

import pytest

pytestmark = pytest.mark.gpu


def test_bench_line_fields(capsys, monkeypatch):
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py", "--config", "1", "--steps", "3", "--warmup", "1", "--layers", "2",
                                      "--kernel-iters", "2", "--no-cpu-baseline"])
    bench.main()
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(lines) == 1, "one JSON line on stdout"
    d = json.loads(lines[0])
    for key, typ in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict)]:
        assert isinstance(d[key], typ), key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["vs_baseline"] is None
    assert isinstance(d["config"]["workload"], str) and d["config"]["layers_per_step"] == 2
    rows = d["config"]["query_rows_per_layer"] * d["config"]["layers_per_step"]
    assert d["value"] == pytest.approx(rows / (d["ms_per_step"] * 1e-3), rel=1e-6)
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma", "alu") and r["unit"] in ("GB/s", "TFLOP/s")
    assert r["peak"] > 0 and r["achieved"] > 0
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-9)
    assert r["traffic"] is None or r["traffic"] > 0
    assert set(d["kernels"]) == {"scan", "attention", "merge"}
