"""The plan lookup: a call whose pointer and size arrays equal those of the
list its operation used last reuses that list's tables without re-checking
every tensor; any other list, including the same host arrays changed in
place, is looked up (and checked) in full."""
import ctypes

import pytest
import torch

import bit_adamw_optimizer_amd as M
from bit_adamw_optimizer_amd import workloads as W
from tests.parity import GpuState

pytestmark = pytest.mark.gpu


def _meta_of(tl, dev="cuda"):
    meta = M.new_meta(tl.n, dev)
    M.amax(tl, meta)
    torch.cuda.synchronize()
    return meta[:, 0].cpu()


def test_lists_of_equal_sizes_are_told_apart():
    a = torch.full((5000,), 2.0, device="cuda")
    b = torch.full((5000,), 3.0, device="cuda")
    c = torch.full((7000,), 5.0, device="cuda")
    ab = M.TensorList([a, b, c], "f32")
    ba = M.TensorList([b, a, c], "f32")
    for _ in range(2):
        assert _meta_of(ab).tolist() == [2.0, 3.0, 5.0]
        assert _meta_of(ba).tolist() == [3.0, 2.0, 5.0]
    # the same host arrays, changed in place between calls
    tl = M.TensorList([a, b, c], "f32")
    assert _meta_of(tl).tolist() == [2.0, 3.0, 5.0]
    tl.ptrs[0], tl.ptrs[1] = b.data_ptr(), a.data_ptr()
    assert _meta_of(tl).tolist() == [3.0, 2.0, 5.0]
    d = torch.full((7000,), 9.0, device="cuda")
    tl.ptrs[2] = d.data_ptr()
    assert _meta_of(tl).tolist() == [3.0, 2.0, 9.0]
    # sizes changed in place: the shorter prefix of c
    tl.ptrs[2] = c.data_ptr()
    c[6000:] = 11.0
    assert _meta_of(tl).tolist() == [3.0, 2.0, 11.0]
    tl.numel[2] = 6000
    assert _meta_of(tl).tolist() == [3.0, 2.0, 5.0]


def test_a_list_changed_in_place_is_checked_again():
    """After a successful step on a list, the same host arrays with a NULL,
    a misaligned pointer or a negative size are refused before any launch,
    and the restored arrays step again."""
    w = W.Workload("lookup", "O2", W.E4M3, 2, ["a", "b"], [4096, 300], seed_base=21)
    gs = GpuState(w, "cuda")
    gs.fill_grads(1)
    gs.step(1)
    torch.cuda.synchronize()
    before = [t.clone() for t in gs.weights + gs.exp_avg]
    hp = w.hparams()
    keep_ptr = gs.tl_m.ptrs[1]
    spare = torch.zeros(400, dtype=torch.uint8, device="cuda")
    cases = [(lambda: gs.tl_m.ptrs.__setitem__(1, None), 1),
             (lambda: gs.tl_m.ptrs.__setitem__(1, spare.data_ptr() + 1), 2)]
    for spoil, status in cases:
        spoil()
        with pytest.raises(M.MsampError) as e:
            M.adamw_o2_step(gs.tl_gq, w.grad_fmt, gs.grad_meta, gs.tl_m, gs.exp_avg_meta, gs.tl_v, gs.tl_w,
                            step=2, **hp)
        assert e.value.status == status
        gs.tl_m.ptrs[1] = keep_ptr
    # a negative size, given through the raw entry point (the binding's size
    # arrays are its own)
    numel = (ctypes.c_int64 * 2)(4096, -1)
    hpc = M._hp(**hp)
    st = M.lib().msamp_adamw_o2_step(2, numel, gs.tl_gq.ptrs, int(w.grad_fmt),
                                     ctypes.c_void_p(gs.grad_meta.data_ptr()), gs.tl_m.ptrs,
                                     ctypes.c_void_p(gs.exp_avg_meta.data_ptr()), gs.tl_v.ptrs, gs.tl_w.ptrs,
                                     ctypes.byref(hpc), 2, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 1
    torch.cuda.synchronize()
    after = gs.weights + gs.exp_avg
    assert all(torch.equal(x.view(torch.uint8), y.view(torch.uint8)) for x, y in zip(before, after))
    gs.fill_grads(2)
    gs.step(2)
    torch.cuda.synchronize()
    assert not torch.equal(before[0], gs.weights[0])


def test_interleaved_lists_step_as_each_alone():
    """Two optimizers with lists of the same sizes, stepped alternately, give
    each one's results alone, byte for byte."""
    w = W.make("tiny_llama")
    w2 = W.make("tiny_llama")
    w2.seed_base = 99
    alone = GpuState(w, "cuda")
    a = GpuState(w, "cuda")
    b = GpuState(w2, "cuda")
    for s in range(1, 4):
        for gs in (alone, a, b):
            gs.fill_grads(s)
        alone.step(s)
        a.step(s)
        b.step(s)
    torch.cuda.synchronize()
    for x, y in zip(alone.weights + alone.exp_avg + alone.exp_avg_sq, a.weights + a.exp_avg + a.exp_avg_sq):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    assert not torch.equal(a.weights[0], b.weights[0])
