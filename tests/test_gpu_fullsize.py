"""Full-size parameter lists through the same launch path the benchmark
times (one multi-tensor launch per pass over the whole list), checked
against the oracle on a subset of whole tensors. Tensors are independent
(per-tensor scaling, element-wise update), so a verified tensor is checked
exactly, whatever else shares the launch. Layouts: MS-AMP "Optimization
Level" page, sections O2/O3 and the table."""
import numpy as np
import pytest
import torch

from bit_adamw_optimizer_amd import workloads as W
from tests.parity import assert_bar, host, log, run_parity

pytestmark = pytest.mark.gpu


def _report(name, stats):
    log("%s: " % name + ", ".join("%s %.6f/%dulp" % (k, s.frac, s.max_ulp)
                                  for k, s in stats.items() if s.total))


def _idx(w, names):
    return [w.names.index(n) for n in names]


def _code_invariant(gs, w, verify):
    # every tensor whose new first moment is nonzero fills the E4M3 range
    mm = gs.exp_avg_meta.cpu().numpy()
    for t in verify:
        if mm[t, 0] > 0:
            assert (host(gs.exp_avg[t]) & 0x7F).max() == 0x7E, w.names[t]


def test_llama2_7b_o2_5_steps():
    w = W.make("llama2_7b")
    verify = _idx(w, ["layers.0.q_proj", "layers.31.down_proj", "layers.0.input_layernorm",
                      "layers.31.post_attention_layernorm", "norm"])
    log("llama2_7b O2: %d tensors, %d params; verifying %d tensors (%d params)"
        % (w.n, w.params, len(verify), sum(w.numel[t] for t in verify)))
    stats, gs, _ = run_parity(w, 5, verify=verify)
    _report("llama2_7b", stats)
    assert_bar(stats)
    _code_invariant(gs, w, verify)
    del gs
    torch.cuda.empty_cache()


def test_llama2_13b_o3_3_steps():
    w = W.make("llama2_13b")
    verify = _idx(w, ["layers.0.k_proj", "layers.39.input_layernorm", "norm"])
    log("llama2_13b O3: %d tensors, %d params; verifying %d tensors (%d params)"
        % (w.n, w.params, len(verify), sum(w.numel[t] for t in verify)))
    stats, gs, _ = run_parity(w, 3, verify=verify)
    _report("llama2_13b", stats)
    assert_bar(stats)
    _code_invariant(gs, w, verify)
    w8m = gs.weight_fp8_meta.cpu().numpy()
    for t in verify:
        assert (host(gs.weight_fp8[t]) & 0x7F).max() == 0x7E
        assert w8m[t, 0] > 0
    del gs
    torch.cuda.empty_cache()


def test_stress_e5m2_10_steps():
    w = W.make("stress")
    small = [t for t in range(w.n) if w.numel[t] <= 8192]
    log("stress O2 E5M2: %d tensors, %d params; verifying the %d small tensors"
        % (w.n, w.params, len(small)))
    stats, gs, _ = run_parity(w, 10, verify=small)
    _report("stress", stats)
    assert_bar(stats)
    mm = gs.exp_avg_meta.cpu().numpy()
    for t in w.zero_tensors:
        assert list(mm[t, :3]) == [0.0, 1.0, 1.0]
    del gs
    torch.cuda.empty_cache()
