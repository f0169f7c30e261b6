"""Full-size parameter lists through the same launch path the benchmark
times (one multi-tensor launch per pass over the whole list, every role in
one flat allocation as in the benchmark), checked
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


def _code_invariant(gs, w, verify):
    # every tensor whose new first moment is nonzero fills the E4M3 range
    mm = gs.exp_avg_meta.cpu().numpy()
    for t in verify:
        if mm[t, 0] > 0:
            assert (host(gs.exp_avg[t]) & 0x7F).max() == 0x7E, w.names[t]


def _first_last_layers(w, last):
    """embed_tokens, lm_head, the final norm and every tensor of the first and
    last decoder layers: every distinct tensor size of the list."""
    keep = [t for t, nm in enumerate(w.names)
            if nm in ("embed_tokens", "lm_head", "norm") or nm.startswith("layers.0.")
            or nm.startswith("layers.%d." % last)]
    assert set(w.numel[t] for t in keep) == set(w.numel)
    return keep


def test_llama2_7b_o2_5_steps():
    w = W.make("llama2_7b")
    verify = _first_last_layers(w, 31)
    log("llama2_7b O2: %d tensors, %d params; verifying %d tensors (%d params)"
        % (w.n, w.params, len(verify), sum(w.numel[t] for t in verify)))
    stats, gs, _ = run_parity(w, 5, verify=verify, flat=True)
    _report("llama2_7b", stats)
    assert_bar(stats)
    _code_invariant(gs, w, verify)
    del gs
    torch.cuda.empty_cache()


def test_llama2_13b_o3_3_steps():
    """The benchmark's O3 configuration: the gradient quantize fused with
    pass 1 (msamp_quantize_adamw_o3_step)."""
    w = W.make("llama2_13b")
    verify = _first_last_layers(w, 39)
    log("llama2_13b O3 fused: %d tensors, %d params; verifying %d tensors (%d params)"
        % (w.n, w.params, len(verify), sum(w.numel[t] for t in verify)))
    stats, gs, _ = run_parity(w, 3, verify=verify, flat=True, fused=True)
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
    """The benchmark's configuration of the stress list: the gradient
    quantize fused with pass 1."""
    w = W.make("stress")
    small = [t for t in range(w.n) if w.numel[t] <= 8192]
    big = [t for t in range(w.n) if w.numel[t] > 8192]
    verify = small + [big[0], big[-1]]
    log("stress O2 E5M2: %d tensors, %d params; verifying the %d small tensors and 2 of the %d "
        "8192x8192 ones (%d params)" % (w.n, w.params, len(small), len(big),
                                        sum(w.numel[t] for t in verify)))
    stats, gs, _ = run_parity(w, 10, verify=verify, flat=True, fused=True)
    _report("stress", stats)
    assert_bar(stats)
    mm = gs.exp_avg_meta.cpu().numpy()
    for t in w.zero_tensors:
        assert list(mm[t, :3]) == [0.0, 1.0, 1.0]
    del gs
    torch.cuda.empty_cache()


def test_one_tensor_beyond_2_pow_32_elements():
    """One tensor of 2^32 + 4099 elements (FP8 byte offsets past 2^32, FP16
    past 2^33, a ragged last chunk): gradient amax and quantize and two O2
    steps through the C ABI, checked against the oracle on windows at the
    start, around element 2^31, below 2^32 and at the end (across 2^32).
    Each step plants the largest |gradient| at one index inside the windows,
    always positive. The windows then hold the tensor's gradient amax, and,
    since the rounded update is monotone in |m0| and |g| for equal signs, its
    first-moment amax too: the oracle run on the concatenated windows sees
    the whole tensor's scales, and every other output is element-wise."""
    import bit_adamw_optimizer_amd as M
    import oracle as O
    from tests.parity import Stats, u32

    dev = "cuda"
    n = (1 << 32) + 4099
    plant = (1 << 32) + 5
    wins = [(0, 70_000), ((1 << 31) - 70_000, (1 << 31) + 70_000),
            ((1 << 32) - 200_000, (1 << 32) - 100_000), (n - 90_000, n)]
    assert all(a < b <= c for (a, b), (c, _) in zip(wins, wins[1:]))
    assert wins[3][0] <= plant < wins[3][1]
    idx = torch.cat([torch.arange(a, b, device=dev) for a, b in wins])
    log("one tensor of %d elements; checking %d of them" % (n, idx.numel()))
    gen = torch.Generator(device=dev)
    gen.manual_seed(2024)
    w = torch.empty(n, dtype=torch.float16, device=dev)
    step_elems = 1 << 30
    for a in range(0, n, step_elems):
        b = min(n, a + step_elems)
        w[a:b] = (torch.randn(b - a, generator=gen, device=dev) * 0.02).to(torch.float16)
    m = torch.zeros(n, dtype=torch.uint8, device=dev)
    v = torch.zeros(n, dtype=torch.float16, device=dev)
    q = torch.empty(n, dtype=torch.uint8, device=dev)
    x = torch.empty(n, dtype=torch.float32, device=dev)
    gmeta, mmeta = M.new_meta(1, dev), M.new_meta(1, dev)
    hp = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
    torch.cuda.synchronize()
    ost = O.TensorState(w[idx].cpu().numpy().view(np.uint16), "O2")
    stats = {k: Stats() for k in ("m", "v", "w")}
    for s in (1, 2):
        x.uniform_(-1e-3, 1e-3, generator=gen)
        x[plant] = 0.02
        M.amax([x], gmeta)
        M.quantize_fp8([x], O.E4M3, gmeta, [q])
        M.adamw_o2_step([q], O.E4M3, gmeta, [m], mmeta, [v], [w], step=s, **hp)
        torch.cuda.synchronize()
        qg, gm = O.step_tensor(ost, x[idx].cpu().numpy(), O.E4M3, s, **hp)
        assert np.array_equal(u32(gmeta[0, :3].cpu().numpy()), u32(gm[:3])), (gmeta, gm)
        assert np.array_equal(q[idx].cpu().numpy(), qg)
        where = "step %d" % s
        stats["m"].add(m[idx].cpu().numpy(), ost.m, "fp8", where)
        stats["v"].add(v[idx].cpu().numpy().view(np.uint16), ost.v, "f16", where)
        stats["w"].add(w[idx].cpu().numpy().view(np.uint16), ost.w, "f16", where)
        assert np.array_equal(u32(mmeta[0, :3].cpu().numpy()), u32(ost.m_meta[:3]))
        assert int(m[plant]) == 0x7E
        _report("2^32+ step %d" % s, stats)
    assert_bar(stats)
    del x, q, m, v, w
    torch.cuda.empty_cache()


def test_llama2_7b_fused_quantize_step_3_steps():
    """The gradient quantize fused with pass 1 over the whole 7B list, one
    tensor of every distinct size checked against the oracle."""
    w = W.make("llama2_7b")
    verify = [w.names.index(nm) for nm in ("embed_tokens", "layers.0.q_proj", "layers.0.gate_proj",
                                            "layers.0.input_layernorm")]
    assert set(w.numel[t] for t in verify) == set(w.numel)
    log("llama2_7b O2 fused: verifying %d tensors (%d params)" % (len(verify), sum(w.numel[t] for t in verify)))
    stats, gs, _ = run_parity(w, 3, verify=verify, flat=True, fused=True)
    _report("llama2_7b fused", stats)
    assert_bar(stats)
    _code_invariant(gs, w, verify)
    del gs
    torch.cuda.empty_cache()


def test_llama2_7b_fused_adam_2_steps():
    """Adam (coupled L2) through the fused quantize-step over the whole 7B
    list (what bench.py --optimizer adam times), one tensor of every
    distinct size checked against the oracle."""
    w = W.make("llama2_7b")
    w.weight_decay = 0.1
    verify = [w.names.index(nm) for nm in ("embed_tokens", "layers.5.q_proj", "layers.5.gate_proj",
                                            "layers.5.post_attention_layernorm")]
    assert set(w.numel[t] for t in verify) == set(w.numel)
    log("llama2_7b O2 fused Adam: verifying %d tensors (%d params)" % (len(verify), sum(w.numel[t] for t in verify)))
    stats, gs, _ = run_parity(w, 2, verify=verify, flat=True, fused=True, adam=True)
    _report("llama2_7b fused adam", stats)
    assert_bar(stats)
    _code_invariant(gs, w, verify)
    del gs
    torch.cuda.empty_cache()


# One tensor of 2^30 elements is the smallest list whose step passes run the
# wide launch (512-thread workgroups over one-tile chunks of 8,192 elements,
# 131,072 chunks); one of 10,240 chunks of 65,536 elements (671,088,640
# elements) is a list of 256-thread workgroups too long to fold its meta
# writes, whose O2 update pass and O3 copy split every chunk over 16
# workgroups.
_WIDE_N, _NARROW_N = 1 << 30, 10240 * 65536


@pytest.mark.parametrize("n,level,gfmt,adam,fused", [
    (_WIDE_N, "O2", "E4M3", False, True), (_WIDE_N, "O3", "E5M2", False, True),
    (_WIDE_N, "O2", "E5M2", True, True), (_WIDE_N, "O3", "E4M3", True, True), (_WIDE_N, "O3", "E5M2", True, True),
    (_WIDE_N, "O3", "E5M2", False, False), (_WIDE_N, "O2", "E5M2", True, False),
    (_WIDE_N, "O3", "E4M3", True, False),
    (_NARROW_N, "O2", "E4M3", False, True), (_NARROW_N, "O3", "E4M3", False, True),
    (_NARROW_N, "O2", "E5M2", True, False), (_NARROW_N, "O3", "E5M2", True, False)])
def test_one_large_tensor_in_each_launch_geometry(n, level, gfmt, adam, fused):
    """One large tensor (above) through two quantize-steps, fused (the
    benchmark's path) or as two calls (every wide instantiation of both
    passes is among the cases), checked against the oracle on windows at the
    start, the middle and the end, with the tensor's largest |gradient|
    (and, for O3, largest |master weight|) planted inside them, so that the
    oracle run on the windows sees the whole tensor's scales (the argument
    of the 2^32 + 4099 test above). Gradient magnitudes lie in [0.5, 1],
    with alternating signs: (1 - beta2) g^2 then stays a normal binary16
    number, so no weight takes the large step a zero FP16 second moment
    gives, and the planted master weight stays the largest. Adam (coupled
    L2) adds wd * w to each gradient, far below the planted one."""
    import bit_adamw_optimizer_amd as M
    import oracle as O
    from tests.parity import Stats, u32

    dev = "cuda"
    fmt = getattr(O, gfmt)
    half = n // 2
    g_plant, w_plant = half + 77, 1234
    wins = [(0, 60_000), (half - 60_000, half + 60_000), (n - 60_000, n)]
    assert all(b <= c for (_, b), (c, _) in zip(wins, wins[1:]))
    assert wins[1][0] <= g_plant < wins[1][1] and wins[0][0] <= w_plant < wins[0][1]
    idx = torch.cat([torch.arange(a, b, device=dev) for a, b in wins])
    log("%s %s%s%s: one tensor of %d elements; checking %d of them"
        % (level, gfmt, " Adam" if adam else "", "" if fused else " two calls", n, idx.numel()))
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    w = (torch.randn(n, generator=gen, device=dev) * 0.02).to(torch.float16)
    if level == "O3":
        w[w_plant] = 1.0
    m = torch.zeros(n, dtype=torch.uint8, device=dev)
    v = torch.zeros(n, dtype=torch.float16, device=dev)
    q = torch.empty(n, dtype=torch.uint8, device=dev)
    x = torch.empty(n, dtype=torch.float32, device=dev)
    w8 = torch.zeros(n, dtype=torch.uint8, device=dev) if level == "O3" else None
    gmeta, mmeta = M.new_meta(1, dev), M.new_meta(1, dev)
    w8meta = M.new_meta(1, dev) if level == "O3" else None
    hp = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
    torch.cuda.synchronize()
    ost = O.TensorState(w[idx].cpu().numpy().view(np.uint16), level, adam=adam)
    stats = {k: Stats() for k in ("m", "v", "w", "w8")}
    M.release_cache()
    for s in (1, 2):
        x.uniform_(0.5, 1.0, generator=gen)
        x[::2].neg_()
        x[g_plant] = 2.0
        M.amax([x], gmeta)
        if not fused:
            M.quantize_fp8([x], fmt, gmeta, [q])
        torch.cuda.synchronize()
        before = M.cache_stats()["bytes"]
        M.profile_enable(True)
        if fused and level == "O2":
            M.quantize_adamw_o2_step([x], fmt, gmeta, [q], [m], mmeta, [v], [w], step=s, adam=adam, **hp)
        elif fused:
            M.quantize_adamw_o3_step([x], fmt, gmeta, [q], [m], mmeta, [v], [w], [w8], w8meta, step=s, adam=adam,
                                     **hp)
        elif level == "O2":
            (M.adam_o2_step if adam else M.adamw_o2_step)([q], fmt, gmeta, [m], mmeta, [v], [w], step=s, **hp)
        else:
            (M.adam_o3_step if adam else M.adamw_o3_step)([q], fmt, gmeta, [m], mmeta, [v], [w], [w8], w8meta,
                                                          step=s, **hp)
        torch.cuda.synchronize()
        launches = {k: M.profile_read(k)[0] for k in ("quantize_pass1", "step_pass1", "o2_pass2", "o3_pass2",
                                                      "o3_pass3", "finalize")}
        M.profile_enable(False)
        # more than 8,192 chunks: the meta records come from a finalize launch
        assert launches["finalize"] == 1, launches
        assert launches["quantize_pass1" if fused else "step_pass1"] == 1, launches
        assert launches["o3_pass3"] == (1 if level == "O3" else 0), launches
        if s == 1:
            # the step's tables: 256 B of amax words, 256 B of descriptors and
            # 8 B per chunk (8,192 elements wide, 65,536 otherwise); a wide
            # list adds descriptors and a map of 131,072-element chunks for
            # pass 1
            if n == _WIDE_N:
                expect = 256 + 256 + n // 8192 * 8 + 256 + n // 131072 * 8
            else:
                expect = 256 + 256 + n // 65536 * 8
            assert M.cache_stats()["bytes"] - before == expect
        qg, gm = O.step_tensor(ost, x[idx].cpu().numpy(), fmt, s, **hp)
        assert np.array_equal(u32(gmeta[0, :3].cpu().numpy()), u32(gm[:3])), (gmeta, gm)
        assert np.array_equal(q[idx].cpu().numpy(), qg)
        where = "step %d" % s
        stats["m"].add(m[idx].cpu().numpy(), ost.m, "fp8", where)
        stats["v"].add(v[idx].cpu().numpy().view(np.uint16), ost.v, "f16", where)
        stats["w"].add(w[idx].cpu().numpy().view(np.uint16), ost.w, "f16", where)
        assert np.array_equal(u32(mmeta[0, :3].cpu().numpy()), u32(ost.m_meta[:3]))
        assert int(m[g_plant]) == 0x7E
        if level == "O3":
            stats["w8"].add(w8[idx].cpu().numpy(), ost.w8, "fp8", where)
            assert np.array_equal(u32(w8meta[0, :3].cpu().numpy()), u32(ost.w8_meta[:3]))
            assert int(w8[w_plant]) & 0x7F == 0x7E
        _report("%d-element %s step %d" % (n, level, s), stats)
    assert_bar(stats)
    del x, q, m, v, w, w8
    torch.cuda.empty_cache()
