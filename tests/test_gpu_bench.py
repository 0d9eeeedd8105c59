"""The throughput benchmark's one JSON line: every field the line promises,
with the values its own definitions fix.

bench.main() runs in this process with a few steps, an 8-row CPU-oracle
sample and no platform reference, for a GEMM-bound step (the Llama-8B MLP
shard), an HBM-bound one (decode) and the graph-timed one-kernel step (the
embedding).  Checked: the fixed fields; `value` equal to the step's work
(the sum over its ops of rate x time) per measured step; the roofline object
taken from the op with the longest launch, achieved / peak = frac, the peak
the published MI355X figure for its bound; the CPU baseline object; and the
benchmark's own oracle comparison on the sampled rows within the bf16 bar.
"""
import json
import math
import sys

import pytest

import bench

pytestmark = pytest.mark.gpu


def _run(capsys, monkeypatch, wid):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", str(wid), "--steps", "3",
                                      "--warmup", "2", "--cpu-rows", "8",
                                      "--no-platform-reference"])
    capsys.readouterr()
    bench.main()
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.strip()]
    assert len(lines) == 1, lines
    return json.loads(lines[0])


@pytest.mark.parametrize("wid", [2, 4, 8])
def test_bench_json_line(wid, capsys, monkeypatch):
    print(f"bench.main() workload {wid}", file=sys.stderr, flush=True)
    d = _run(capsys, monkeypatch, wid)

    types = {"metric": str, "value": float, "unit": str, "n_gpus": int, "steps": int,
             "warmup": int, "ms_per_step": float, "higher_is_better": bool, "scaling": str,
             "dtype": str, "data": str, "config": dict, "roofline": dict, "ops": dict,
             "cpu_baseline": dict}
    for k, t in types.items():
        assert isinstance(d[k], t), (k, d.get(k))
    assert d["metric"] == bench.METRIC
    assert (d["n_gpus"], d["steps"], d["warmup"]) == (1, 3, 2)
    assert d["higher_is_better"] is True and d["scaling"] == "weak"
    assert "vs_baseline" in d and d["vs_baseline"] is None
    assert d["dtype"] == "bf16" and d["data"].startswith("synthetic")
    assert isinstance(d["config"].get("workload"), str) and d["config"]["workload"]
    assert d["value"] > 0 and d["ms_per_step"] > 0

    # value = the step's work per measured step time
    ops = d["ops"]
    if d["unit"] == "TFLOP/s":
        work = sum(o["tflops"] * 1e12 * o["avg_us"] * 1e-6 for o in ops.values() if "tflops" in o)
        assert math.isclose(d["value"] * 1e12 * d["ms_per_step"] * 1e-3, work, rel_tol=1e-9)
    else:
        assert d["unit"] == "GB/s"
        work = sum(o["algorithmic_bytes"] for o in ops.values())
        assert math.isclose(d["value"] * 1e9 * d["ms_per_step"] * 1e-3, work, rel_tol=1e-9)

    # roofline: the op with the longest launch, against the published peak
    r = d["roofline"]
    dom = max(ops, key=lambda k: ops[k]["avg_us"])
    assert r["kernel"] == dom
    assert math.isclose(r["avg_launch_us"], ops[dom]["avg_us"], rel_tol=1e-12)
    if r["bound"] == "mfma":
        assert (r["unit"], r["peak"]) == ("TFLOP/s", 2516.6)
        assert math.isclose(r["achieved"], ops[dom]["tflops"], rel_tol=1e-12)
    else:
        assert r["bound"] == "hbm"
        assert (r["unit"], r["peak"]) == ("GB/s", 8000.0)
        assert math.isclose(r["achieved"], ops[dom]["gbps"], rel_tol=1e-12)
    assert (r["bound"] == "hbm") == (wid in (4, 8))
    assert math.isclose(r["frac"], r["achieved"] / r["peak"], rel_tol=1e-12)
    assert 0 < r["frac"] < 1
    assert r["traffic"] is None or (isinstance(r["traffic"], int) and r["traffic"] > 0)

    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and isinstance(cb["cores"], int) and cb["cores"] >= 1
    assert cb["unit"] == ("GB/s" if wid == 8 else "TFLOP/s")
    assert cb["value"] > 0 and "8" in cb["sample"]

    # the benchmark's own comparison with the oracle on the sampled rows
    ps = d["parity_sample"]
    assert ps
    for name, p in ps.items():
        if "bitwise_equal" in p:
            assert p["bitwise_equal"], name
        else:
            assert p["rows"] == 8 and p["rel_l2"] <= 1e-2, (name, p)
