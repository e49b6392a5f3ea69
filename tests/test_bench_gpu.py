"""bench.py end to end: every workload and option runs one timed step through the library and
prints one JSON line with the fields the bench contract names (small shapes where the workload
takes them, so the whole file runs in about a minute).  The measurements themselves are not
checked here; the line's structure and that every code path runs are."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


SMALL = ["--B", "2", "--T", "256", "--H", "4"]
CASES = [
    SMALL + ["--cpu-seconds", "0.5"],
    SMALL + ["--algo", "scan", "--no-cpu-baseline"],
    SMALL + ["--head-first", "--no-cpu-baseline"],
    SMALL + ["--out-dtype", "bf16", "--no-cpu-baseline"],
    SMALL + ["--saved-states", "--no-cpu-baseline"],
    SMALL + ["--workload", "wkv5", "--no-cpu-baseline"],
    ["--workload", "wkv4", "--B", "2", "--T", "128", "--cpu-seconds", "0.5"],
    ["--workload", "decode", "--H", "4", "--cpu-seconds", "0.5"],
    ["--workload", "serving", "--H", "4", "--no-cpu-baseline"],
    ["--workload", "serving", "--H", "4", "--budget-mode", "slot", "--no-cpu-baseline"],
    SMALL + ["--workload", "wkv6_bwd", "--cpu-seconds", "0.5"],
    SMALL + ["--workload", "wkv6_bwd", "--saved-states", "--no-cpu-baseline"],
    SMALL + ["--workload", "wkv6_bwd", "--algo", "scan", "--no-cpu-baseline"],
    SMALL + ["--workload", "wkv7", "--cpu-seconds", "0.5"],
    SMALL + ["--workload", "wkv7", "--algo", "scan", "--no-cpu-baseline"],
    ["--workload", "wkv7", "--B", "8", "--T", "1", "--H", "4", "--no-cpu-baseline"],
]


@pytest.mark.gpu
@pytest.mark.parametrize("argv", CASES, ids=[" ".join(a) for a in CASES])
def test_bench_workload_line(argv, monkeypatch, capsys):
    bench = _bench()
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "1", "--warmup", "0", "--settle-ms", "0"] + argv)
    print(f"bench {' '.join(argv)}", file=sys.stderr, flush=True)
    bench.main()
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(lines) == 1, lines
    j = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in j, key
    assert j["n_gpus"] == 1 and j["steps"] == 1 and j["value"] > 0 and j["ms_per_step"] > 0
    assert "workload" in j["config"]
    r = j["roofline"]
    assert r["bound"] in ("hbm", "alu", "mfma") and r["peak"] > 0 and r["achieved"] > 0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    if "--no-cpu-baseline" not in argv:
        c = j["cpu_baseline"]
        assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]
