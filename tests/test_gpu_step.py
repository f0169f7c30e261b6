"""The O2 and O3 AdamW steps through the C ABI against the oracle, at sizes
the oracle finishes in seconds: independent trajectories over the steps of
each workload, gradient codes and scales bit-exact, optimizer outputs at the
bar (>= 99.99% identical, the rest within 1 ulp). Layouts: MS-AMP
"Optimization Level" page, sections O2 and O3 and the table."""
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


def test_single_1m_o2_10_steps():
    w = W.make("single_1m")
    log("single_1m O2, %d params, 10 steps" % w.params)
    stats, _, _ = run_parity(w, 10)
    _report("single_1m", stats)
    assert_bar(stats)


def test_tiny_llama_o2_10_steps():
    w = W.make("tiny_llama")
    log("tiny_llama O2, %d tensors, %d params" % (w.n, w.params))
    stats, _, _ = run_parity(w, 10)
    _report("tiny_llama", stats)
    assert_bar(stats)


def test_tiny_llama_o3_10_steps():
    w = W.make("tiny_llama_o3")
    log("tiny_llama O3, %d tensors, %d params" % (w.n, w.params))
    stats, _, _ = run_parity(w, 10)
    _report("tiny_llama_o3", stats)
    assert_bar(stats)


def test_tiny_stress_e5m2_10_steps():
    w = W.make("tiny_stress")
    log("tiny_stress O2 E5M2, %d tensors, %d params, %d zero" % (w.n, w.params, len(w.zero_tensors)))
    stats, gs, ost = run_parity(w, 10)
    _report("tiny_stress", stats)
    assert_bar(stats)
    # all-zero gradient tensors keep zero moments and scale 1
    mm = gs.exp_avg_meta.cpu().numpy()
    for t in w.zero_tensors:
        assert (host(gs.exp_avg[t]) == 0).all()
        assert list(mm[t, :3]) == [0.0, 1.0, 1.0]


@pytest.mark.parametrize("level", ["O2", "O3"])
def test_adam_coupled_l2_10_steps(level):
    """torch.optim.Adam variant (MS-AMP README, Usage): L2 weight decay on the
    gradient, no decoupled decay."""
    w = W.make("tiny_llama_o3" if level == "O3" else "tiny_llama")
    w.weight_decay = 0.1
    log("Adam %s tiny_llama, %d params" % (level, w.params))
    stats, _, _ = run_parity(w, 10, adam=True)
    _report("adam_" + level, stats)
    assert_bar(stats)


def test_adam_ragged_e5m2():
    sizes = [0, 1, 15, 17, 4097, 65537, 131072 + 4096 + 9]
    w = W.Workload("adam_ragged", "O2", W.E5M2, 4, ["t%d" % i for i in range(len(sizes))], sizes,
                   grad_kind="student_t3", lr=5e-3, betas=(0.8, 0.99), eps=1e-7, weight_decay=0.2,
                   seed_base=14)
    stats, _, _ = run_parity(w, 4, adam=True)
    _report(w.name, stats)
    assert_bar(stats)


def test_delayed_scaling_ablation_10_steps():
    """One-pass delayed-scaling O2 step (an ablation entry point): parity with
    the oracle's ablation, and its step-1 failure (first moment stored as
    +-0) on the GPU."""
    # gradients ~ N(0, 1e-3): |m1| = 0.1|g| stays below half the smallest
    # E4M3 subnormal (2^-10), so with scale 1 every code is +-0
    w1 = W.make("single_1m")
    stats, gs, _ = run_parity(w1, 1, delayed=True)
    assert_bar(stats)
    assert ((host(gs.exp_avg[0]) & 0x7F) == 0).all()
    w = W.make("tiny_llama")
    stats, _, _ = run_parity(w, 10, delayed=True)
    _report("delayed", stats)
    assert_bar(stats)


def test_scaled_v_ablation_10_steps():
    """O2 AdamW with a per-tensor-scaled FP16 second moment (an ablation
    entry point): parity with the oracle's ablation, including the v meta;
    at gradient scale 1e-3 its v stays representable where the literal FP16
    v of the O2 step underflows to zero."""
    w = W.make("single_1m")
    stats, gs, _ = run_parity(w, 10, scaled_v=True)
    _report("scaled_v single_1m", stats)
    assert_bar(stats)
    v_scaled = host(gs.exp_avg_sq[0])
    _, gp, _ = run_parity(w, 1)
    v_plain = host(gp.exp_avg_sq[0])
    assert (v_scaled != 0).mean() > 0.99
    assert (v_plain != 0).mean() < 0.01
    sizes = [0, 1, 15, 17, 4097, 65537, 131072 + 4096 + 9]
    wr = W.Workload("scaled_v_ragged", "O2", W.E5M2, 4, ["t%d" % i for i in range(len(sizes))],
                    sizes, grad_kind="student_t3", lr=5e-3, betas=(0.8, 0.99), eps=1e-7,
                    weight_decay=0.2, seed_base=15)
    stats, _, _ = run_parity(wr, 4, scaled_v=True)
    _report(wr.name, stats)
    assert_bar(stats)
    stats, _, _ = run_parity(W.make("tiny_llama"), 10, scaled_v=True)
    _report("scaled_v tiny_llama", stats)
    assert_bar(stats)


def test_scaled_v_ablation_second_moment_above_first():
    """Pass 1 of the scaled-v ablation reduces two maxima per workgroup,
    amax(m1) and amax(v1). At gradient scale 1000, v1 = (1-b2) g^2 exceeds
    |m1| = (1-b1)|g| wherever |g| > 100, so amax(v1) is far above amax(m1) in
    every workgroup: a reduction that mixed the two would store m with the
    v scale and fail parity."""
    w = W.make("tiny_llama")
    w.grad_sigma = 1000.0
    stats, gs, ost = run_parity(w, 6, scaled_v=True)
    _report("scaled_v sigma=1000", stats)
    assert_bar(stats)
    for t, o in ost.items():
        if w.numel[t] >= 1024:
            assert o.v_meta[0] > 2.0 * o.m_meta[0], (w.names[t], o.v_meta, o.m_meta)


def test_ragged_sizes_o2_and_o3():
    """Sizes around the 16-element vector, the 4096-element tile and the
    65536-element chunk, including empty tensors; O3 with both gradient
    formats."""
    sizes = [0, 1, 7, 15, 16, 17, 31, 4095, 4096, 4097, 65535, 65536, 65537, 131072 + 4096 + 9, 0, 3]
    for level, fmt in (("O2", W.E4M3), ("O3", W.E4M3), ("O3", W.E5M2)):
        w = W.Workload("ragged_%s_%d" % (level, fmt), level, fmt, 4, ["t%d" % i for i in range(len(sizes))],
                       sizes, lr=5e-3, betas=(0.8, 0.99), eps=1e-7, weight_decay=0.05, seed_base=11)
        log("ragged %s fmt %d" % (level, fmt))
        stats, gs, _ = run_parity(w, 4)
        _report(w.name, stats)
        assert_bar(stats)
        mm = gs.exp_avg_meta.cpu().numpy()
        for t, k in enumerate(sizes):
            if k == 0:
                assert list(mm[t, :3]) == [0.0, 1.0, 1.0]


def test_mid_size_list_takes_3_tile_chunks():
    """A list of 3,126 tiles of 4,096 elements is split into chunks of 3
    tiles (12,288 elements: small lists get smaller chunks so that every
    compute unit has work); O2 and O3 against the oracle."""
    sizes = [6_000_001, 4_500_007, 2_300_000]
    tiles = sum(-(-k // 4096) for k in sizes)
    assert tiles // 1024 == 3
    for level in ("O2", "O3"):
        w = W.Workload("mid_" + level, level, W.E4M3, 3, ["a", "b", "c"], sizes, seed_base=17)
        stats, _, _ = run_parity(w, 3)
        _report(w.name, stats)
        assert_bar(stats)


def test_gpt2_small_o2_10_steps():
    w = W.make("gpt2_small")
    log("gpt2_small O2, %d tensors, %d params" % (w.n, w.params))
    stats, _, _ = run_parity(w, 10)
    _report("gpt2_small", stats)
    assert_bar(stats)


def test_deterministic_and_resume_bit_exact():
    """Two runs from the same state are bit-identical, and 3 steps + a
    save/restore of the whole state + 3 steps equals 6 straight steps."""
    w = W.make("tiny_llama_o3")
    log("determinism / resume")

    def snapshot(gs):
        return [t.clone() for t in gs.exp_avg + gs.exp_avg_sq + gs.weights + gs.weight_fp8] + \
            [gs.exp_avg_meta.clone(), gs.weight_fp8_meta.clone()]

    a = GpuState(w, "cuda")
    b = GpuState(w, "cuda")
    for s in range(1, 4):
        for gs in (a, b):
            gs.fill_grads(s)
            gs.step(s)
    torch.cuda.synchronize()
    sa, sb = snapshot(a), snapshot(b)
    assert all(torch.equal(x, y) for x, y in zip(sa, sb))
    # save to host, clobber, restore
    saved = [t.cpu() for t in snapshot(b)]
    for t in b.exp_avg + b.exp_avg_sq + b.weights + b.weight_fp8:
        t.fill_(0)
    live = b.exp_avg + b.exp_avg_sq + b.weights + b.weight_fp8 + [b.exp_avg_meta, b.weight_fp8_meta]
    for dst, src in zip(live, saved):
        dst.copy_(src)
    for s in range(4, 7):
        for gs in (a, b):
            gs.fill_grads(s)
            gs.step(s)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(snapshot(a), snapshot(b)))


def test_nonfinite_gradient_step_is_skipped_and_training_resumes():
    """The caller-side skip of a step on a non-finite gradient (what
    GradScaler does; MS-AMP README, Usage): Inf and NaN planted in one tensor
    make msamp_amax report a non-finite amax for that tensor only; the caller
    reads the amax column, skips the quantize and the step, and the state is
    untouched; the next step, with finite gradients and the same step count,
    equals an uninterrupted run byte for byte."""
    w = W.make("tiny_llama_o3")
    ref = GpuState(w, "cuda")
    sk = GpuState(w, "cuda")

    def state(gs):
        return [t.clone().view(torch.uint8) if t.dtype == torch.float16 else t.clone()
                for t in gs.exp_avg + gs.exp_avg_sq + gs.weights + gs.weight_fp8 +
                [gs.exp_avg_meta, gs.weight_fp8_meta]]

    for gs in (ref, sk):
        gs.fill_grads(1)
        gs.step(1)
    torch.cuda.synchronize()
    before = state(sk)
    bad = max(range(w.n), key=lambda t: w.numel[t])
    sk.fill_grads(2)
    sk.grad_f32[bad][3] = float("inf")
    sk.grad_f32[bad][7] = float("nan")
    M.amax(sk.tl_g32, sk.grad_meta)
    amax = sk.grad_meta[:, 0]
    finite = torch.isfinite(amax)
    assert not bool(finite[bad]) and bool(finite[torch.arange(w.n, device="cuda") != bad].all())
    skip = not bool(finite.all())
    assert skip  # the caller enqueues neither the quantize nor the step
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(before, state(sk)))
    # step 2 again with finite gradients
    for gs in (ref, sk):
        gs.fill_grads(2)
        gs.step(2)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(state(ref), state(sk)))


def test_o3_weight_copy_overwrites_every_element_and_max_code():
    w = W.Workload("cover", "O3", W.E4M3, 1, ["a", "b", "c"], [4097, 65537, 33], seed_base=12)
    gs = GpuState(w, "cuda")
    for t in gs.weight_fp8:
        t.fill_(0x7F)  # NaN code: never produced by the step
    gs.fill_grads(1)
    gs.step(1)
    torch.cuda.synchronize()
    for t in range(w.n):
        w8 = host(gs.weight_fp8[t])
        assert not (w8 == 0x7F).any() and not (w8 == 0xFF).any()
        assert (w8 & 0x7F).max() == 0x7E
        assert (host(gs.exp_avg[t]) & 0x7F).max() == 0x7E


def test_step_argument_errors():
    w = W.Workload("err", "O2", W.E4M3, 1, ["a"], [100], seed_base=13)
    gs = GpuState(w, "cuda")
    before = gs.weights[0].clone()
    hp = w.hparams()
    for bad in (dict(step=0), dict(step=1, eps=0.0), dict(step=1, betas=(1.0, 0.999)),
                dict(step=1, lr=float("nan"))):
        kw = dict(hp)
        kw.update(bad)
        with pytest.raises(M.MsampError) as e:
            M.adamw_o2_step(gs.tl_gq, 0, gs.grad_meta, gs.tl_m, gs.exp_avg_meta, gs.tl_v, gs.tl_w, **kw)
        assert e.value.status == 1
    shifted = torch.zeros(101, dtype=torch.uint8, device="cuda")[1:]  # 1-byte offset
    with pytest.raises(M.MsampError) as e:
        M.adamw_o2_step(gs.tl_gq, 0, gs.grad_meta, [shifted], gs.exp_avg_meta,
                        gs.tl_v, gs.tl_w, step=1, **hp)
    assert e.value.status == 2
    torch.cuda.synchronize()
    assert torch.equal(before, gs.weights[0])


def test_rmw_probe_leaves_every_stream_unchanged():
    """msamp_rmw_probe (measurement aid) rewrites m, v and w with their own
    values and never writes g, on ragged sizes and both tails."""
    sizes = [0, 1, 15, 17, 4097, 65537, 131072 + 4096 + 9]
    g = [torch.randint(0, 256, (k,), dtype=torch.uint8, device="cuda") for k in sizes]
    m = [torch.randint(0, 256, (k,), dtype=torch.uint8, device="cuda") for k in sizes]
    v = [torch.randint(0, 1 << 15, (k,), dtype=torch.int16, device="cuda").view(torch.float16) for k in sizes]
    w = [torch.randint(0, 1 << 15, (k,), dtype=torch.int16, device="cuda").view(torch.float16) for k in sizes]
    before = [t.clone() for t in g + m + v + w]
    for _ in range(3):
        M.rmw_probe(g, m, v, w)
    torch.cuda.synchronize()
    after = g + m + v + w
    assert all(torch.equal(a.view(torch.uint8), b.view(torch.uint8)) for a, b in zip(after, before))


def test_stream_probe_copies_exactly_and_leaves_the_source():
    """msamp_stream_probe (measurement aid): a copy reproduces the source byte
    for byte, over whole 16 KB workgroup tiles and a ragged last one, writes
    nothing past the copied bytes, and neither kind changes the source."""
    for nbytes in (16, 16 * 1024, 16 * 1024 * 37 + 48):
        src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
        keep = src.clone()
        dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
        M.stream_probe(src)
        M.stream_probe(src, dst[:nbytes])
        torch.cuda.synchronize()
        assert torch.equal(src, keep)
        assert torch.equal(dst[:nbytes], src)
        assert int(dst[nbytes:].count_nonzero()) == 0


@pytest.mark.parametrize("level,adam,wl,fused", [("O2", False, "tiny_llama", False),
                                                 ("O3", True, "tiny_llama_o3", False),
                                                 ("O2", False, "tiny_stress", False),
                                                 ("O2", True, "tiny_stress", True),
                                                 ("O3", False, "tiny_llama_o3", True),
                                                 ("O2", False, "tiny_small", True)])
def test_graph_captured_step_replays_later_steps_bit_exact(level, adam, wl, fused):
    """amax + quantize + the device-constants step (or amax + the quantizing
    device-constants step, fused=True) captured once in a HIP graph
    (torch.cuda.graph) and replayed for steps 2..6, with the step's constants
    rewritten in device memory and new gradients written between replays
    (eager work and a synchronization in between every time). After every
    replay the whole state equals the eager by-value unfused entry points'
    bit for bit."""
    w = W.make(wl)
    if adam:
        w.weight_decay = 0.1
    log("graph replay %s %s adam=%s fused=%s" % (wl, level, adam, fused))
    ref = GpuState(w, "cuda", adam=adam)
    gr = GpuState(w, "cuda", adam=adam)
    consts = torch.empty(9, dtype=torch.float32, device="cuda")

    def graph_step():
        M.amax(gr.tl_g32, gr.grad_meta)
        if fused and level == "O3":
            M.quantize_adamw_o3_step_devconst(gr.tl_g32, w.grad_fmt, gr.grad_meta, gr.tl_gq, gr.tl_m,
                                              gr.exp_avg_meta, gr.tl_v, gr.tl_w, gr.tl_w8, gr.weight_fp8_meta,
                                              consts, adam=adam)
            return
        if fused:
            M.quantize_adamw_o2_step_devconst(gr.tl_g32, w.grad_fmt, gr.grad_meta, gr.tl_gq, gr.tl_m,
                                              gr.exp_avg_meta, gr.tl_v, gr.tl_w, consts, adam=adam)
            return
        M.quantize_fp8(gr.tl_g32, w.grad_fmt, gr.grad_meta, gr.tl_gq)
        if level == "O3":
            M.adamw_o3_step_devconst(gr.tl_gq, w.grad_fmt, gr.grad_meta, gr.tl_m, gr.exp_avg_meta,
                                     gr.tl_v, gr.tl_w, gr.tl_w8, gr.weight_fp8_meta, consts, adam=adam)
        else:
            M.adamw_o2_step_devconst(gr.tl_gq, w.grad_fmt, gr.grad_meta, gr.tl_m, gr.exp_avg_meta,
                                     gr.tl_v, gr.tl_w, consts, adam=adam)

    def state(gs):
        ts = gs.exp_avg + gs.exp_avg_sq + gs.weights + gs.grad_q + [gs.exp_avg_meta, gs.grad_meta]
        if level == "O3":
            ts += gs.weight_fp8 + [gs.weight_fp8_meta]
        return [t.view(torch.uint8) if t.dtype == torch.float16 else t for t in ts]

    graph = None
    for s in range(1, 7):
        ref.fill_grads(s)
        ref.step(s)
        gr.fill_grads(s)
        consts.copy_(M.step_constants(step=s, adam=adam, **w.hparams()))
        if s == 1:
            graph_step()  # eager: builds the cached tables before the capture
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                graph_step()
        else:
            graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(state(ref), state(gr)):
            assert torch.equal(a, b), "step %d differs" % s


def test_captured_tables_survive_eviction_and_release_until_unpinned():
    """The tables a captured graph uses are pinned: pushing 80 other lists
    through the cache (past its 64-list bound) and calling
    msamp_release_cache() frees every other table but not those, and the
    graph still replays the exact eager trajectory. Unpinning lets
    release_cache free them."""
    w = W.make("tiny_llama")
    ref = GpuState(w, "cuda")
    gr = GpuState(w, "cuda")
    consts = torch.empty(9, dtype=torch.float32, device="cuda")

    def graph_step():
        M.amax(gr.tl_g32, gr.grad_meta)
        M.quantize_fp8(gr.tl_g32, w.grad_fmt, gr.grad_meta, gr.tl_gq)
        M.adamw_o2_step_devconst(gr.tl_gq, w.grad_fmt, gr.grad_meta, gr.tl_m, gr.exp_avg_meta, gr.tl_v,
                                 gr.tl_w, consts)

    pinned0 = M.cache_stats()["pinned"]
    graph = None
    for s in range(1, 5):
        ref.fill_grads(s)
        ref.step(s)
        gr.fill_grads(s)
        consts.copy_(M.step_constants(step=s, **w.hparams()))
        if s == 1:
            graph_step()  # eager: builds the three tables
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                graph_step()
            torch.cuda.synchronize()
            st = M.cache_stats()
            assert st["pinned"] == pinned0 + 3, st
            # 80 other lists, then a release: only pinned tables remain
            meta = M.new_meta(1, "cuda")
            for i in range(80):
                M.amax([torch.ones(64 + 16 * i, device="cuda")], meta)
            torch.cuda.synchronize()
            assert M.cache_stats()["lists"] <= 64 + st["pinned"]
            M.release_cache()
            st2 = M.cache_stats()
            assert st2["pinned"] == st["pinned"] and st2["lists"] == st["pinned"], st2
        else:
            graph.replay()
        torch.cuda.synchronize()
        parts_r = ref.exp_avg + ref.exp_avg_sq + ref.weights + [ref.exp_avg_meta, ref.grad_meta]
        parts_g = gr.exp_avg + gr.exp_avg_sq + gr.weights + [gr.exp_avg_meta, gr.grad_meta]
        for a, b in zip(parts_r, parts_g):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "step %d differs" % s
    del graph
    M.unpin_captured_tables()
    M.release_cache()
    assert M.cache_stats() == {"lists": 0, "bytes": 0, "pinned": 0}


@pytest.mark.parametrize("hp", [
    dict(lr=0.0, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01),
    dict(lr=1e-2, betas=(0.0, 0.999), eps=1e-8, weight_decay=0.01),
    dict(lr=1e-2, betas=(0.9, 0.0), eps=1e-8, weight_decay=0.01),
    dict(lr=1e-2, betas=(0.9, 0.999), eps=1.0, weight_decay=0.0),
], ids=["lr0", "beta1_0", "beta2_0", "eps1"])
def test_degenerate_hyperparameters(hp):
    """Limits of the AdamW definition (lr = 0: the weight stays put; beta1 =
    0; beta2 = 0; eps dominating the denominator), O2 and O3, against the
    oracle."""
    sizes = [17, 4097, 65537 + 16]
    for level in ("O2", "O3"):
        w = W.Workload("degenerate_" + level, level, W.E4M3, 3, ["t%d" % i for i in range(len(sizes))],
                       sizes, seed_base=16, **hp)
        stats, gs, _ = run_parity(w, 3)
        _report(w.name, stats)
        assert_bar(stats)
        if hp["lr"] == 0.0:
            w0 = W.init_weights(w, "cuda")
            assert all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(gs.weights, w0))


def test_release_cache_mid_run_is_bit_exact():
    """Freeing the cached device tables between steps only makes the next
    call rebuild them: the trajectory is bit-identical to an uninterrupted
    one."""
    w = W.make("tiny_llama_o3")
    a = GpuState(w, "cuda")
    b = GpuState(w, "cuda")
    for s in range(1, 5):
        for gs in (a, b):
            gs.fill_grads(s)
            gs.step(s)
        if s == 2:
            torch.cuda.synchronize()
            M.release_cache()
    torch.cuda.synchronize()
    for x, y in zip(a.exp_avg + a.exp_avg_sq + a.weights + a.weight_fp8 + [a.exp_avg_meta, a.weight_fp8_meta],
                    b.exp_avg + b.exp_avg_sq + b.weights + b.weight_fp8 + [b.exp_avg_meta, b.weight_fp8_meta]):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


def _slice_bounds(numel, ranks):
    """Per tensor, the bounds of each rank's contiguous slice (starts rounded
    up to 16 elements, so that every slice keeps a 16-byte aligned base)."""
    return [[min(k, -(-(k * r // ranks) // 16) * 16) for r in range(ranks)] + [k] for k in numel]


@pytest.mark.parametrize("level,adam,wl", [("O2", False, "tiny_llama"), ("O3", False, "tiny_llama_o3"),
                                           ("O3", True, "tiny_llama_o3"), ("O2", True, "tiny_stress"),
                                           ("O3", False, "tiny_small_o3")])
def test_sharded_phases_equal_the_unsharded_step(level, adam, wl):
    """Three data-parallel ranks emulated on one GPU, each holding a slice of
    every tensor, run the split-phase step; the per-tensor amaxes are
    combined with a MAX between the phases (what an all-reduce MAX over the
    ranks would do). Over 4 steps every byte of the state and every meta
    record equals the unsharded step's, and the sharded state meets the
    parity bar against the oracle run on the whole tensors."""
    ranks = 3
    w = W.make(wl)
    if adam:
        w.weight_decay = 0.1
    hp = w.hparams()
    log("sharded phases %s %s adam=%s" % (wl, level, adam))
    ref = GpuState(w, "cuda", adam=adam)
    sh = GpuState(w, "cuda", adam=adam)
    bounds = _slice_bounds(w.numel, ranks)
    torch.cuda.synchronize()
    ost = [O.TensorState(host(x), level, adam=adam) for x in sh.weights]
    from tests.parity import Stats

    def piece(lst, r, kind):
        return M.TensorList([x[bounds[t][r]:bounds[t][r + 1]] for t, x in enumerate(lst)], kind)

    R = []
    for r in range(ranks):
        d = dict(g32=piece(sh.grad_f32, r, "f32"), gq=piece(sh.grad_q, r, "u8"), m=piece(sh.exp_avg, r, "u8"),
                 v=piece(sh.exp_avg_sq, r, "f16"), w=piece(sh.weights, r, "f16"),
                 gmeta=M.new_meta(w.n, "cuda"), mmeta=M.new_meta(w.n, "cuda"),
                 w8=piece(sh.weight_fp8, r, "u8") if level == "O3" else None,
                 w8meta=M.new_meta(w.n, "cuda") if level == "O3" else None,
                 amax_m=torch.zeros(w.n, dtype=torch.float32, device="cuda"),
                 amax_w=torch.zeros(w.n, dtype=torch.float32, device="cuda"))
        R.append(d)

    def phase(p, d, **kw):
        M.adamw_step_phase(p, level, d["gq"], w.grad_fmt, d["gmeta"], d["m"], d["mmeta"], d["v"], d["w"],
                           d["w8"], d["w8meta"], adam=adam, **kw)

    for s in range(1, 5):
        ref.fill_grads(s)
        ref.step(s)
        sh.fill_grads(s)
        for d in R:
            M.amax(d["g32"], d["gmeta"])
        gmax = torch.stack([d["gmeta"][:, 0] for d in R]).max(0).values
        for d in R:
            d["gmeta"][:, 0] = gmax
            M.quantize_fp8(d["g32"], w.grad_fmt, d["gmeta"], d["gq"])
        for d in R:
            phase(1, d, amax_out=d["amax_m"], step=s, **hp)
        am = torch.stack([d["amax_m"] for d in R]).max(0).values
        for d in R:
            phase(2, d, amax_in=am, amax_out=d["amax_w"], step=s, **hp)
        if level == "O3":
            aw = torch.stack([d["amax_w"] for d in R]).max(0).values
            for d in R:
                phase(3, d, amax_in=aw)
        torch.cuda.synchronize()
        roles = ["exp_avg", "exp_avg_sq", "weights", "grad_q"] + (["weight_fp8"] if level == "O3" else [])
        for role in roles:
            for a, b in zip(getattr(ref, role), getattr(sh, role)):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (s, role)
        for d in R:
            assert torch.equal(d["gmeta"][:, :3], ref.grad_meta[:, :3]), s
            assert torch.equal(d["mmeta"], ref.exp_avg_meta), s
            if level == "O3":
                assert torch.equal(d["w8meta"], ref.weight_fp8_meta), s
        # the sharded state against the oracle on the whole tensors
        stats = {k: Stats() for k in ("m", "v", "w", "w8")}
        for t in range(w.n):
            qg, _ = O.step_tensor(ost[t], host(sh.grad_f32[t]), w.grad_fmt, s, **hp)
            assert np.array_equal(host(sh.grad_q[t]), qg), (s, t)
            stats["m"].add(host(sh.exp_avg[t]), ost[t].m, "fp8", "t%d" % t)
            stats["v"].add(host(sh.exp_avg_sq[t]), ost[t].v, "f16", "t%d" % t)
            stats["w"].add(host(sh.weights[t]), ost[t].w, "f16", "t%d" % t)
            if level == "O3":
                stats["w8"].add(host(sh.weight_fp8[t]), ost[t].w8, "fp8", "t%d" % t)
        assert_bar(stats)
