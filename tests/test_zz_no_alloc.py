"""The allocation-free O2 AdamW step (msamp_adamw_o2_step_noalloc, tables in
the library's static device array) against msamp_adamw_o2_step (tables in
the cached, allocated plan): two calls in a row on one device, the second on
a smaller tensor list, must leave every byte of the state and every meta
record identical (both run the same kernels on the same inputs)."""
import pytest
import torch

import bit_adamw_optimizer_amd as M
from bit_adamw_optimizer_amd import workloads as W
from tests.parity import GpuState, log

pytestmark = pytest.mark.gpu


def _snapshot(gs):
    return [x.clone() for x in gs.exp_avg + gs.exp_avg_sq + gs.weights] + [gs.exp_avg_meta.clone()]


def _equal(a, b):
    return all(torch.equal(x.view(torch.uint8), y.view(torch.uint8)) for x, y in zip(a, b))


def test_noalloc_step_matches_the_cached_entry_point_on_two_calls():
    big = W.Workload("noalloc_big", "O2", W.E4M3, 1, ["t%d" % i for i in range(9)],
                     [0, 17, 4095, 65536, 65537, 131072 + 4096 + 9, 1 << 20, 3, 300_001], seed_base=41)
    small = W.Workload("noalloc_small", "O2", W.E5M2, 1, ["s0", "s1", "s2"], [5, 4097, 70_000], lr=5e-3,
                       betas=(0.8, 0.99), eps=1e-7, weight_decay=0.05, seed_base=43)
    for call, w in enumerate((big, small), 1):
        ref = GpuState(w, "cuda")
        tst = GpuState(w, "cuda")
        for s in (1, 2):
            for gs in (ref, tst):
                gs.fill_grads(s)
                M.amax(gs.tl_g32, gs.grad_meta)
                M.quantize_fp8(gs.tl_g32, w.grad_fmt, gs.grad_meta, gs.tl_gq)
            M.adamw_o2_step(ref.tl_gq, w.grad_fmt, ref.grad_meta, ref.tl_m, ref.exp_avg_meta, ref.tl_v,
                            ref.tl_w, step=s, **w.hparams())
            M.adamw_o2_step_noalloc(tst.tl_gq, w.grad_fmt, tst.grad_meta, tst.tl_m, tst.exp_avg_meta,
                                    tst.tl_v, tst.tl_w, step=s, **w.hparams())
            torch.cuda.synchronize()
            assert torch.equal(ref.grad_meta, tst.grad_meta)
            assert _equal(_snapshot(ref), _snapshot(tst)), (w.name, s)
            nz = sum(int((m != 0).sum()) for m in tst.exp_avg)
            assert nz > 0, "the step wrote no first-moment codes"
        log("noalloc call %d (%s, %d tensors, %d params): identical over 2 steps" % (call, w.name, w.n, w.params))
