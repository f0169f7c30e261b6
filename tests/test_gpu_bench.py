"""bench.py end to end on a small parameter list (GPT-2-small shapes), in a
child process: one JSON line with every key of the benchmark contract, a
roofline record for the dominant kernel with its same-buffers traffic probes, the
fused and two-call gradient quantize, and the HIP-graph replay mode."""
import json
import os
import subprocess
import sys

import pytest

from tests.parity import log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*extra):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "gpt2_small", "--steps", "3",
           "--warmup", "2", "--no-cpu-baseline", *extra]
    log("running " + " ".join(cmd[1:]))
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def test_bench_json_contract():
    d = _run()
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["unit"] == "params/s" and d["dtype"] == "f32" and d["data"] == "synthetic"
    assert d["config"]["params"] == 124_439_808 and "gpt2_small" in d["config"]["workload"]
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["kernel"] == "o2_pass2" and 0 < rf["frac"] < 1
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert 0 < rf["same_buffers_probe"]["frac"] < 1.5
    assert set(rf["traffic_probes"]) == {"read", "copy", "update_pass_mix", "quantize_pass1_mix"}
    assert all(c["GB/s"] > 0 for c in rf["traffic_probes"].values())
    # default: the gradient quantize runs fused with pass 1 (21 bytes per parameter)
    assert d["config"]["fused_quantize"] is True and d["bytes_per_param"] == 21
    assert set(d["kernels"]) >= {"amax", "quantize_pass1", "o2_pass2"}
    # a list of under 8,192 chunks writes its meta records from the workgroup
    # that completes each tensor: no finalize launches
    assert "finalize" not in d["kernels"] and "amax_finalize" not in d["kernels"]
    assert d["optimizer_step"]["includes_grad_quantize"] is True


def test_bench_separate_quantize():
    d = _run("--separate-quantize")
    assert d["config"]["fused_quantize"] is False and d["bytes_per_param"] == 22
    assert set(d["kernels"]) >= {"amax", "quantize_fp8", "step_pass1", "o2_pass2"}


def test_bench_graph_mode():
    """Graph replay of amax + the quantizing device-constants step."""
    d = _run("--graph")
    assert d["config"]["graph"] is True and d["value"] > 0
    assert d["config"]["fused_quantize"] is True and d["bytes_per_param"] == 21


def test_bench_adam_fused():
    """Adam's fused pass also reads the FP16 weight for the L2 term: 23 bytes
    per parameter; the pass-1 probe (which has no weight read) is not run."""
    d = _run("--optimizer", "adam")
    assert d["config"]["fused_quantize"] is True and d["bytes_per_param"] == 23
    assert set(d["kernels"]) >= {"amax", "quantize_pass1", "o2_pass2"}
    assert "quantize_pass1_mix" not in d["roofline"]["traffic_probes"]
