"""bench.py's output contract: one JSON line with the metric, the whole-job
value, the roofline of the decode kernel and the oracle baseline.  Runs
bench.main() in this process on the default workload (the 32-layer
Llama-3-8B-shaped GQA step), with a short oracle budget."""
import json
import sys

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def test_bench_json_contract(monkeypatch, capsys):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "3", "--warmup", "1", "--cpu-seconds", "0.5"])
    bench.main()
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["config"]["workload"] == "llama3_8b_step" and d["config"]["layers"] == 32
    assert d["config"]["n_q_heads"] == 32 and d["config"]["n_kv_heads"] == 8
    # whole-step rate from the timed region: bytes per step / time per step
    assert abs(d["value"] - d["config"]["kv_bytes_per_step"] / (d["ms_per_step"] / 1e3) / 1e9) < 0.01 * d["value"]
    r = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in r, k
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert 0 < r["frac"] < 1
    assert d["gather_probe_gbs"] > 0 and d["hbm_read_probe_gbs"] > 0
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0 and c["sample"]
