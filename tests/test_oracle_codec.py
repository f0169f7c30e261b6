"""Pins of the oracle's FP8 (OCP E4M3/E5M2) and FP16 codecs.

The oracle codec (oracle/oracle.c) is checked against things other than
itself: torch's CPU float8/float16 tables and casts, numpy's float16 cast, a
brute-force nearest-value search, and closed-form values of the OCP 8-bit
floating point definitions. The two FP8 formats are the ones named in
TransformerEngine issue #131 ("FP8 questions"); their use for gradients and
the first moment comes from the MS-AMP optimization-level table.
"""
import numpy as np
import pytest
import torch

import oracle as O
from tests.exact_fp import fp8_table

FORMATS = [(O.E4M3, 448.0, 0x7E, 0x7F), (O.E5M2, 57344.0, 0x7B, 0x7F)]


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_fp8_decode_matches_torch_all_codes(fmt):
    codes = np.arange(256, dtype=np.uint8)
    ours = O.fp8_decode(codes, fmt).astype(np.float64)
    ref = fp8_table(fmt)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # signed zeros
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_fp8_decode_closed_form_key_values():
    e4 = O.fp8_decode(np.array([0x01, 0x08, 0x38, 0x7E, 0x7F, 0x80, 0xFE], np.uint8), O.E4M3)
    assert e4[0] == 2.0 ** -9 and e4[1] == 2.0 ** -6 and e4[2] == 1.0 and e4[3] == 448.0
    assert np.isnan(e4[4]) and e4[5] == 0.0 and np.signbit(e4[5]) and e4[6] == -448.0
    e5 = O.fp8_decode(np.array([0x01, 0x04, 0x3C, 0x7B, 0x7C, 0x7D, 0x7E, 0x7F, 0xFC], np.uint8), O.E5M2)
    assert e5[0] == 2.0 ** -16 and e5[1] == 2.0 ** -14 and e5[2] == 1.0 and e5[3] == 57344.0
    assert np.isposinf(e5[4]) and np.isnan(e5[5:8]).all() and np.isneginf(e5[8])
    assert O.fp8_max(O.E4M3) == 448.0 and O.fp8_max(O.E5M2) == 57344.0


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_fp8_roundtrip_all_finite_codes(fmt):
    codes = np.arange(256, dtype=np.uint8)
    vals = O.fp8_decode(codes, fmt)
    fin = np.isfinite(vals)
    assert fin.sum() == (254 if fmt == O.E4M3 else 248)
    assert np.array_equal(O.fp8_encode(vals[fin], fmt), codes[fin])


def _brute_fp8(x: np.ndarray, fmt: int) -> np.ndarray:
    """Nearest finite code with the input's sign, ties to the even code."""
    table = fp8_table(fmt)
    codes = np.arange(256)
    sign_of_code = codes >> 7
    finite = np.isfinite(table)
    out = np.empty(x.size, np.uint8)
    for lo in range(0, x.size, 4096):
        xs = x[lo:lo + 4096].astype(np.float64)
        neg = np.signbit(xs).astype(np.int64)
        # beyond 2*max the nearest finite value is +-max whatever the input;
        # clipping there keeps every float64 distance below exact
        top = np.nanmax(np.abs(table[finite]))
        xs = np.clip(xs, -2 * top, 2 * top)
        d = np.abs(table[None, :] - xs[:, None])
        bad = (~finite)[None, :] | (sign_of_code[None, :] != neg[:, None])
        d[bad] = np.inf
        dmin = d.min(axis=1, keepdims=True)
        tie = d == dmin
        # among the nearest codes take the even one (score 0 beats 1 beats 2)
        score = np.where(tie, codes[None, :] & 1, 2)
        out[lo:lo + 4096] = np.argmin(score, axis=1)
    return out


def _fp8_test_inputs(fmt: int, rng) -> np.ndarray:
    table = fp8_table(fmt)
    fin = np.sort(np.unique(np.abs(table[np.isfinite(table)])))
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)  # exact in binary32
    assert np.array_equal(mids.astype(np.float64), (fin[:-1] + fin[1:]) / 2)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    top = np.float32(fin[-1])
    beyond = np.array([top * 1.0001, top * 1.0714, top * 1.0715, top * 1.2, top * 2, 3.4e38,
                       fin[1] / 2, fin[1] / 4, 1e-30, 1e-45], np.float32)
    rand = (rng.standard_normal(200_000) * np.exp(rng.uniform(-25, 13, 200_000))).astype(np.float32)
    base = np.concatenate([fin.astype(np.float32), mids, up, dn, beyond, rand])
    return np.concatenate([base, -base])


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_fp8_encode_equals_brute_force_nearest(fmt):
    rng = np.random.default_rng(1234 + fmt)
    x = _fp8_test_inputs(fmt, rng)
    assert np.array_equal(O.fp8_encode(x, fmt), _brute_fp8(x, fmt))


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_fp8_encode_matches_torch_cast_in_range(fmt):
    # torch's CPU float8 casts round to nearest even but do not saturate, so
    # they are a second reference for every input below the overflow midpoint.
    rng = np.random.default_rng(99 + fmt)
    x = _fp8_test_inputs(fmt, rng)
    mx = O.fp8_max(fmt)
    x = x[np.abs(x) <= mx]
    ref = torch.from_numpy(x).to(fp8_dtype(fmt)).view(torch.uint8).numpy()
    assert np.array_equal(O.fp8_encode(x, fmt), ref)


def fp8_dtype(fmt):
    return torch.float8_e4m3fn if fmt == O.E4M3 else torch.float8_e5m2


@pytest.mark.parametrize("fmt,mx,maxcode,nancode", FORMATS)
def test_fp8_encode_specials_and_saturation(fmt, mx, maxcode, nancode):
    x = np.array([np.inf, -np.inf, np.nan, -np.nan, 0.0, -0.0, mx, -mx, mx * 4, -mx * 4, 3.0e38],
                 np.float32)
    q = O.fp8_encode(x, fmt)
    assert list(q) == [maxcode, 0x80 | maxcode, nancode, 0x80 | nancode, 0x00, 0x80, maxcode,
                       0x80 | maxcode, maxcode, 0x80 | maxcode, maxcode]


def test_fp8_encode_closed_form_cases():
    # Values fixed by RNE on the OCP grids: ties go to the even mantissa, the
    # half-way point below the smallest subnormal goes to zero, -tiny keeps
    # its sign.
    e4 = O.fp8_encode(np.array([17.0, 19.0, 2 ** -10, 3 * 2 ** -10, 464.0, -2 ** -11], np.float32), O.E4M3)
    assert list(e4) == [0x58, 0x5A, 0x00, 0x02, 0x7E, 0x80]
    e5 = O.fp8_encode(np.array([2 ** -17, 3 * 2 ** -17, 61440.0, 0.625], np.float32), O.E5M2)
    assert list(e5) == [0x00, 0x02, 0x7B, 0x39]


def test_f16_decode_all_patterns_matches_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.f16_decode(h)
    ref = h.view(np.float16).astype(np.float32)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin].view(np.uint32), ref[fin].view(np.uint32))


def test_f16_encode_matches_numpy_cast():
    rng = np.random.default_rng(7)
    # every rounding boundary: midpoints of adjacent binary16 values, +-1 ulp
    pos = np.arange(0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    ovf = np.float32(65520.0)  # half-way between 65504 and 2^16
    special = np.array([ovf, np.nextafter(ovf, np.float32(0)), np.nextafter(ovf, np.float32(np.inf)),
                        np.inf, 1e38, 2 ** -25, 2 ** -26, 3 * 2 ** -26, 1e-45], np.float32)
    rnd_bits = rng.integers(0, 2 ** 32, 4_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
                        pos.astype(np.float32), special, rnd_bits])
    x = np.concatenate([x, -x])
    ours = O.f16_encode(x)
    ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.isnan(ours[nan].view(np.float16)).all()
