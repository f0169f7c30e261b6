"""The gfx950 device codec (hardware OCP FP8 and FP16 converts as the kernels
use them) against the oracle's codec, on every FP8 code, every FP16 pattern,
every rounding boundary of both FP8 formats and of FP16, and random inputs.
FP8 formats E4M3/E5M2: TransformerEngine issue #131 ("FP8 questions"); their
roles: MS-AMP optimization-level table."""
import numpy as np
import pytest
import torch

import bit_adamw_optimizer_amd as M
import oracle as O
from tests.parity import log

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _probe(op, x_np, out_dtype):
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(DEV)
    out = torch.empty(x.numel(), dtype=out_dtype, device=DEV)
    M.codec_probe(op, x, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("fmt,op", [(O.E4M3, M.PROBE_E4M3_TO_F32), (O.E5M2, M.PROBE_E5M2_TO_F32)])
def test_fp8_decode_all_codes(fmt, op):
    log("probe decode fmt=%d" % fmt)
    codes = np.tile(np.arange(256, dtype=np.uint8), 3)  # every byte position
    got = _probe(op, codes, torch.float32)
    ref = O.fp8_decode(codes, fmt)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))


def _boundaries(fmt, rng):
    table = O.fp8_decode(np.arange(256, dtype=np.uint8), fmt).astype(np.float64)
    fin = np.sort(np.unique(np.abs(table[np.isfinite(table)])))
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)
    top = np.float32(fin[-1])
    extra = np.array([top * 1.0001, top * 1.0714, top * 1.0715, top * 1.5, top * 4, 3.4e38,
                      np.inf, 1e-30, 1e-40, 1e-45, 0.0], np.float32)
    rand = (rng.standard_normal(1_000_000) * np.exp(rng.uniform(-30, 14, 1_000_000))).astype(np.float32)
    bits = rng.integers(0, 2 ** 32, 1_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    base = np.concatenate([fin.astype(np.float32), mids, np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(0)), extra, rand, bits])
    return np.concatenate([base, -base, np.array([np.nan, -np.nan], np.float32)])


@pytest.mark.parametrize("fmt,op", [(O.E4M3, M.PROBE_F32_TO_E4M3), (O.E5M2, M.PROBE_F32_TO_E5M2)])
def test_fp8_encode_matches_oracle(fmt, op):
    log("probe encode fmt=%d" % fmt)
    rng = np.random.default_rng(10 + fmt)
    x = _boundaries(fmt, rng)
    got = _probe(op, x, torch.uint8)
    ref = O.fp8_encode(x, fmt)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_f16_encode_matches_oracle():
    log("probe f16 encode")
    rng = np.random.default_rng(3)
    pos = np.arange(0x7C00, dtype=np.uint32).astype(np.uint16)
    vals = O.f16_decode(pos).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    bits = rng.integers(0, 2 ** 32, 4_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
                        vals.astype(np.float32), np.array([65520.0, 65519.996, 1e38, np.inf, 1e-45], np.float32),
                        bits])
    x = np.concatenate([x, -x])
    got = _probe(M.PROBE_F32_TO_F16, x, torch.int16).view(np.uint16)
    ref = O.f16_encode(x)
    nan = np.isnan(x)
    bad = np.nonzero((got != ref) & ~nan)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]
    assert np.isnan(got[nan].view(np.float16)).all()


def test_f16_decode_all_patterns():
    log("probe f16 decode")
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = _probe(M.PROBE_F16_TO_F32, h.view(np.int16), torch.float32)
    ref = O.f16_decode(h)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))


@pytest.mark.parametrize("op,kind", [(M.PROBE_F32_TO_E4M3, O.E4M3), (M.PROBE_F32_TO_E5M2, O.E5M2),
                                     (M.PROBE_F32_TO_F16, "f16")])
def test_exhaustive_every_binary32_input(op, kind):
    """All 2^32 binary32 bit patterns through the device cast, against the
    oracle's encoder (bit-exact; FP16 NaN payloads are only checked to stay
    NaN)."""
    from concurrent.futures import ThreadPoolExecutor
    chunk = 1 << 28
    sub = chunk // 16
    pool = ThreadPoolExecutor(max_workers=16)
    out_dtype = torch.uint8 if kind != "f16" else torch.int16
    bad_total = 0
    for start in range(0, 1 << 32, chunk):
        log("exhaustive %s chunk %d/16" % (kind, start // chunk + 1))
        host_bits = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
        x = torch.from_numpy(host_bits.view(np.int32)).to(DEV)
        out = torch.empty(chunk, dtype=out_dtype, device=DEV)
        M.codec_probe(op, x, out)
        got = out.cpu().numpy()
        xf = host_bits.view(np.float32)
        if kind == "f16":
            ref = np.concatenate(list(pool.map(O.f16_encode, [xf[i:i + sub] for i in range(0, chunk, sub)])))
            got = got.view(np.uint16)
            nan = np.isnan(xf)
            bad = (got != ref) & ~nan
            assert np.isnan(got[nan].view(np.float16)).all()
        else:
            ref = np.concatenate(list(pool.map(lambda a: O.fp8_encode(a, kind),
                                               [xf[i:i + sub] for i in range(0, chunk, sub)])))
            bad = got != ref
        nbad = int(bad.sum())
        if nbad:
            i = np.nonzero(bad)[0][:5]
            raise AssertionError("%s: %d mismatches in chunk at %#x, e.g. %s" % (
                kind, nbad, start, [(hex(int(host_bits[j])), int(got[j]), int(ref[j])) for j in i]))
        bad_total += nbad
        del x, out
    pool.shutdown()
    assert bad_total == 0
