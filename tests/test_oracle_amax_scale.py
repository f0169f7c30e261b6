"""Pins of the oracle's per-tensor amax, scale rule and quantize.

amax is checked against numpy's max(|x|) by brute force on tiny tensors;
the scale rule (scale = fp8_max/amax, 1 when amax is 0 or not finite) against
closed-form special cases; quantize against a brute-force nearest-code search
and the single-element invariant (any nonzero finite value maps to +-max).
Per-tensor scaling of FP8 gradients and moments follows the MS-AMP
optimization-level table (FP8 weight gradient, FP8 first moment).
"""
import numpy as np
import pytest

import oracle as O
from tests.exact_fp import F, brute_encode_fp8, float_to_bits


def _specials_tensor(rng, n):
    pool = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-40, 1.0, -2.5, 1e-3, 3e38, -3e38], np.float32)
    x = rng.standard_normal(n).astype(np.float32) * np.float32(10.0) ** rng.integers(-8, 8, n).astype(np.float32)
    mask = rng.random(n) < 0.3
    x[mask] = rng.choice(pool, mask.sum())
    return x


def test_amax_brute_force_tiny_tensors():
    rng = np.random.default_rng(0)
    for n in list(range(0, 258)) + [1000, 4097]:
        x = _specials_tensor(rng, n)
        expect = np.float32(np.max(np.abs(x))) if n else np.float32(0.0)
        got = O.amax(x)
        assert float_to_bits(float(got)) == float_to_bits(float(expect)), n
        # -0 counts as +0: the result is never negative
        assert not np.signbit(got)


def test_amax_permutation_invariant_and_nan_inf_dominance():
    rng = np.random.default_rng(1)
    x = _specials_tensor(rng, 5000)
    a = O.amax(x)
    for _ in range(5):
        assert O.amax(rng.permutation(x)).view(np.uint32) == a.view(np.uint32)
    y = x.copy()
    y[17] = -np.inf
    assert np.isposinf(O.amax(y))
    y[4000] = np.nan
    assert np.isnan(O.amax(y))
    assert np.isnan(O.amax(rng.permutation(y)))


@pytest.mark.parametrize("fmt,fmax", [(O.E4M3, 448.0), (O.E5M2, 57344.0)])
def test_scale_rule_closed_forms(fmt, fmax):
    assert O.scale(0.0, fmax) == 1.0
    assert O.scale(np.inf, fmax) == 1.0
    assert O.scale(np.nan, fmax) == 1.0
    assert O.scale(fmax, fmax) == 1.0
    assert O.scale(1.0, fmax) == np.float32(fmax)
    for k in (-30, -20, -3, 0, 5, 40):
        assert O.scale(2.0 ** k, fmax) == np.float32(fmax * 2.0 ** -k)
    # fmax/amax overflows binary32 for amax below fmax/FLT_MAX: scale 1
    tiny = np.float32(fmax / 3.4028234663852886e38) / np.float32(2)
    assert O.scale(tiny, fmax) == 1.0
    assert O.scale(np.float32(1e-45), fmax) == 1.0
    # the largest finite amax still gives a finite positive scale
    s = O.scale(np.float32(3.4028234663852886e38), fmax)
    assert 0 < s < 1e-30


@pytest.mark.parametrize("fmt,maxcode", [(O.E4M3, 0x7E), (O.E5M2, 0x7B)])
def test_single_element_quantizes_to_max_code(fmt, maxcode):
    rng = np.random.default_rng(5)
    vals = rng.standard_normal(2000) * np.exp(rng.uniform(-80, 80, 2000))
    # below fmax/FLT_MAX the quotient overflows and the scale rule gives 1
    lo = O.fp8_max(fmt) / 3.4028234663852886e38 * 1.01
    vals = vals[(np.abs(vals) > lo) & (np.abs(vals) < 3e38)].astype(np.float32)
    for v in vals:
        q, meta = O.quantize_fp8(np.array([v], np.float32), fmt)
        assert q[0] == (maxcode | (0x80 if v < 0 else 0)), v
        assert meta[0] == abs(v)
        assert meta[2] == np.float32(1.0) / meta[1]


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_multi_element_quantize_by_brute_force(fmt):
    x = np.array([0.25, -1.0, 3.3, 0.0, -0.0, 1e-6, -0.004], np.float32)
    q, meta = O.quantize_fp8(x, fmt)
    amax = F.of(3.3)
    s = F.of(O.fp8_max(fmt)) / amax
    assert float_to_bits(float(meta[0])) == amax.b
    assert float_to_bits(float(meta[1])) == s.b
    assert float_to_bits(float(meta[2])) == (F.of(1.0) / s).b
    for xi, qi in zip(x, q):
        xs = F.of(float(xi)) * s
        assert qi == brute_encode_fp8(xs.q, fmt, bool(xs.b >> 31))
    # hand-computed codes (scaled value rounded on the OCP grid)
    expect = {O.E4M3: [0x60, 0xF0, 0x7E, 0x00, 0x80, 0x00, 0xB1],
              O.E5M2: [0x6C, 0xF4, 0x7B, 0x00, 0x80, 0x24, 0xD4]}[fmt]
    assert list(q) == expect


@pytest.mark.parametrize("fmt,maxcode", [(O.E4M3, 0x7E), (O.E5M2, 0x7B)])
def test_quantize_invariant_max_code_and_caller_amax(fmt, maxcode):
    rng = np.random.default_rng(11)
    x = (rng.standard_t(3, 100_003) * 1e-3).astype(np.float32)
    q, meta = O.quantize_fp8(x, fmt)
    assert (q & 0x7F).max() == maxcode
    # a caller-supplied amax below the true amax saturates the outliers
    q2, meta2 = O.quantize_fp8(x, fmt, amax_value=meta[0] / 8)
    assert meta2[1] == O.scale(meta[0] / 8, O.fp8_max(fmt))
    sat = np.abs(x) * meta2[1] > O.fp8_max(fmt) * 1.07
    assert sat.any() and ((q2[sat] & 0x7F) == maxcode).all()
    # all-zero tensor: scale 1, codes 0
    qz, mz = O.quantize_fp8(np.zeros(33, np.float32), fmt)
    assert (qz == 0).all() and list(mz[:3]) == [0.0, 1.0, 1.0]


def test_dequantize_is_code_times_scale_inv():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(4096) * 1e-3).astype(np.float32)
    q, meta = O.quantize_fp8(x, O.E4M3)
    d = O.dequantize_fp8(q, O.E4M3, meta[2])
    expect = O.fp8_decode(q, O.E4M3) * meta[2]
    assert np.array_equal(d.view(np.uint32), expect.view(np.uint32))
    # quantization error of E4M3: at most half a step (2^-4 relative) for
    # normal codes, half the smallest subnormal step otherwise
    err = np.abs(d.astype(np.float64) - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * meta[2]) * 1.0000001
    assert (err <= bound).all()


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_prescaled_quantize_for_fp8_allreduce(fmt):
    """O1 (MS-AMP optimization-level table: FP8 weight gradient and FP8
    all-reduce): with the common amax of N ranks and scale(amax * N), the
    exact sum of the N ranks' scaled values never exceeds the FP8 range, and
    world = 1 is the plain per-tensor quantize."""
    rng = np.random.default_rng(21 + fmt)
    fmax = O.fp8_max(fmt)
    for world in (1, 2, 3, 8, 64):
        ranks = [(rng.standard_t(3, 4096) * 1e-3 * rng.uniform(0.5, 2)).astype(np.float32)
                 for _ in range(world)]
        amax = max(O.amax(r) for r in ranks)  # what an all-reduce MAX returns
        outs = [O.quantize_fp8_prescaled(r, fmt, amax, world) for r in ranks]
        s = outs[0][1][1]
        assert all(o[1][1] == s for o in outs)
        assert s == O.scale(np.float32(amax) * np.float32(world), fmax)
        # codes: the scaled value rounded on the FP8 grid (the plain encoder)
        for r, (q, _) in zip(ranks, outs):
            assert np.array_equal(q, O.fp8_encode(r * s, fmt))
        # exact sum of the decoded (unscaled-back) codes stays within range
        total = np.sum([O.fp8_decode(q, fmt).astype(np.float64) for q, _ in outs], axis=0)
        assert np.abs(total).max() <= fmax * (1 + 2.0 ** -3)
        if world == 1:
            q1, m1 = O.quantize_fp8(ranks[0], fmt)
            assert np.array_equal(q1, outs[0][0]) and np.array_equal(m1, outs[0][1])
    with pytest.raises(ValueError):
        O.quantize_fp8_prescaled(np.ones(3, np.float32), fmt, 1.0, 0)
