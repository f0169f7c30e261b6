"""Lists of many small tensors: 1,120 tensors of 0 to 4,096 elements (the
edge sizes around the 4-, 8- and 16-element groups and the 1,024-element
wave span, and random ones) in runs between larger tensors. Every entry
point over such a list against the oracle (MS-AMP "Optimization Level" page,
sections O2 and O3 and the table), and the fused quantize-step byte for byte
against the two calls."""
import numpy as np
import pytest
import torch

import bit_adamw_optimizer_amd as M
import oracle as O
from bit_adamw_optimizer_amd import workloads as W
from tests.parity import GpuState, assert_bar, host, log, run_parity, u32

pytestmark = pytest.mark.gpu


def _report(name, stats):
    log("%s: " % name + ", ".join("%s %.6f/%dulp" % (k, s.frac, s.max_ulp)
                                  for k, s in stats.items() if s.total))


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_small_tensor_amax_quantize_dequantize_bit_exact(fmt):
    _, sizes = W.small_shapes()
    rng = np.random.default_rng(300 + fmt)
    xs = [(rng.standard_t(3, k) * 10.0 ** rng.uniform(-6, 2)).astype(np.float32) for k in sizes]
    for x in xs[::7]:
        if x.size > 8:
            x[rng.choice(x.size, 3, replace=False)] = np.array([-0.0, 1e-40, -5e-42], np.float32)
    log("small tensors amax/quantize fmt=%d: %d tensors" % (fmt, len(xs)))
    dx = [torch.from_numpy(x).to("cuda") for x in xs]
    n = len(xs)
    meta = M.new_meta(n, "cuda")
    q = [torch.full((x.size,), 0xAB, dtype=torch.uint8, device="cuda") for x in xs]
    M.amax(dx, meta)
    torch.cuda.synchronize()
    m_after_amax = meta.cpu().numpy()
    M.quantize_fp8(dx, fmt, meta, q)
    out = [torch.full((x.size,), float("nan"), dtype=torch.float32, device="cuda") for x in xs]
    M.dequantize_fp8(q, fmt, meta, out)
    torch.cuda.synchronize()
    mg = meta.cpu().numpy()
    for t, x in enumerate(xs):
        assert u32(m_after_amax[t, 0]) == u32(O.amax(x)), t
        qr, mr = O.quantize_fp8(x, fmt)
        assert np.array_equal(u32(mg[t, :3]), u32(mr[:3])), (t, mg[t], mr)
        assert np.array_equal(q[t].cpu().numpy(), qr), (t, x.size)
        dr = O.dequantize_fp8(qr, fmt, mr[2])
        assert np.array_equal(out[t].cpu().numpy().view(np.uint32), dr.view(np.uint32)), t


@pytest.mark.parametrize("wl,fused,adam", [("tiny_small", True, False), ("tiny_small", False, False),
                                           ("tiny_small_o3", True, False), ("tiny_small_o3", False, True),
                                           ("tiny_small", True, True)])
def test_small_tensor_steps_match_the_oracle(wl, fused, adam):
    w = W.make(wl)
    if adam:
        w.weight_decay = 0.1
    log("%s %s fused=%s adam=%s: %d tensors, %d params" % (wl, w.level, fused, adam, w.n, w.params))
    stats, gs, _ = run_parity(w, 3, adam=adam, fused=fused)
    _report(wl, stats)
    assert_bar(stats)


@pytest.mark.parametrize("ablation", ["delayed", "scaled_v"])
def test_small_tensor_ablations_match_the_oracle(ablation):
    w = W.make("tiny_small")
    stats, _, _ = run_parity(w, 3, **{ablation: True})
    _report("tiny_small " + ablation, stats)
    assert_bar(stats)


def test_small_tensor_fused_equals_two_calls_byte_for_byte():
    w = W.make("tiny_small_o3")
    ref = GpuState(w, "cuda")
    fus = GpuState(w, "cuda", fused=True)
    for s in range(1, 4):
        for gs in (ref, fus):
            gs.fill_grads(s)
            gs.step(s)
        torch.cuda.synchronize()
        parts = lambda g: (g.grad_q + [g.grad_meta] + g.exp_avg + [g.exp_avg_meta] + g.exp_avg_sq + g.weights
                           + g.weight_fp8 + [g.weight_fp8_meta])
        for i, (a, b) in enumerate(zip(parts(ref), parts(fus))):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (s, i)
