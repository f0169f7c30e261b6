"""CPU oracle for the per-tensor-scaled FP8 AdamW step (MS-AMP O2/O3).

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product path
(``bit_adamw_optimizer_amd`` and its HIP library) never imports it, and this
package imports nothing from the product.

The arithmetic lives in ``oracle.c`` (scalar C, one tensor at a time); this
module only loads it with ctypes and marshals numpy arrays. The list-level
helpers run whole tensors on a thread pool: ctypes releases the GIL during a
foreign call and tensors are independent (per-tensor scaling, elementwise
update), so the result does not depend on the thread count.

Definitions and readings are documented at the top of ``oracle.c``; in short
(MS-AMP "Optimization Level" page, section O2/O3 and its table):
O2 = FP8 grad + FP8 E4M3 first moment (own scale) + FP16 second moment + FP16
weight; O3 = O2 on an FP16 master plus an FP8 E4M3 weight copy.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

E4M3 = 0
E5M2 = 1

# Optimizer-state bytes per parameter of the two layouts on the MS-AMP
# optimization-level table: FP32+FP32 (FP16 AMP / TE / O1) and FP8+FP16 (O2/O3).
STATE_BYTES_FP32_FP32 = 4 + 4
STATE_BYTES_FP8_FP16 = 1 + 2


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (IEEE arithmetic, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = build()
        L = ctypes.CDLL(path)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        hp = ctypes.POINTER(_HParams)
        L.oracle_fp8_encode_array.argtypes = [vp, i64, i32, vp]
        L.oracle_fp8_encode_array.restype = i32
        L.oracle_fp8_decode_array.argtypes = [vp, i64, i32, vp]
        L.oracle_fp8_decode_array.restype = i32
        L.oracle_f16_encode_array.argtypes = [vp, i64, vp]
        L.oracle_f16_encode_array.restype = None
        L.oracle_f16_decode_array.argtypes = [vp, i64, vp]
        L.oracle_f16_decode_array.restype = None
        L.oracle_fp8_max.argtypes = [i32]
        L.oracle_fp8_max.restype = f32
        L.oracle_amax.argtypes = [vp, i64]
        L.oracle_amax.restype = f32
        L.oracle_scale.argtypes = [f32, f32]
        L.oracle_scale.restype = f32
        L.oracle_quantize_fp8.argtypes = [vp, i64, i32, f32, vp, vp]
        L.oracle_quantize_fp8.restype = i32
        L.oracle_quantize_fp8_prescaled.argtypes = [vp, i64, i32, f32, i32, vp, vp]
        L.oracle_quantize_fp8_prescaled.restype = i32
        L.oracle_dequantize_fp8.argtypes = [vp, i64, i32, f32, vp]
        L.oracle_dequantize_fp8.restype = i32
        L.oracle_adamw_constants.argtypes = [hp, i64, vp]
        L.oracle_adamw_constants.restype = None
        L.oracle_adamw_f32_tensor.argtypes = [i64, vp, vp, vp, vp, hp, i64, i32]
        L.oracle_adamw_f32_tensor.restype = None
        L.oracle_adamw_o2_tensor.argtypes = [i64, vp, i32, f32, vp, vp, vp, vp, hp, i64, i32]
        L.oracle_adamw_o2_tensor.restype = i32
        L.oracle_adamw_o3_tensor.argtypes = [i64, vp, i32, f32, vp, vp, vp, vp, vp, vp, hp, i64, i32]
        L.oracle_adamw_o3_tensor.restype = i32
        L.oracle_adamw_o2_tensor_delayed.argtypes = [i64, vp, i32, f32, vp, vp, vp, vp, hp, i64, i32]
        L.oracle_adamw_o2_tensor_delayed.restype = i32
        L.oracle_adamw_o2_tensor_scaled_v.argtypes = [i64, vp, i32, f32, vp, vp, vp, vp, vp, hp, i64]
        L.oracle_adamw_o2_tensor_scaled_v.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _hp(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01) -> _HParams:
    return _HParams(float(lr), float(betas[0]), float(betas[1]), float(eps), float(weight_decay))


# ---------------------------------------------------------------- codec ---

def fp8_encode(x, fmt: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    if lib().oracle_fp8_encode_array(_ptr(x), x.size, fmt, _ptr(out)) != 0:
        raise ValueError("bad FP8 format %r" % fmt)
    return out


def fp8_decode(codes, fmt: int) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float32)
    if lib().oracle_fp8_decode_array(_ptr(c), c.size, fmt, _ptr(out)) != 0:
        raise ValueError("bad FP8 format %r" % fmt)
    return out


def f16_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f16_encode_array(_ptr(x), x.size, _ptr(out))
    return out


def f16_decode(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_f16_decode_array(_ptr(h), h.size, _ptr(out))
    return out


def fp8_max(fmt: int) -> float:
    return float(lib().oracle_fp8_max(fmt))


# ------------------------------------------------------- amax / scaling ---

def amax(x) -> np.float32:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return np.float32(lib().oracle_amax(_ptr(x), x.size))


def scale(amax_value, fmax) -> np.float32:
    return np.float32(lib().oracle_scale(float(np.float32(amax_value)), float(np.float32(fmax))))


def quantize_fp8(x, fmt: int, amax_value=None):
    """Returns (codes uint8, meta float32[4] = {amax, scale, scale_inv, 0})."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if amax_value is None:
        amax_value = amax(x)
    q = np.empty(x.shape, np.uint8)
    meta = np.zeros(4, np.float32)
    if lib().oracle_quantize_fp8(_ptr(x), x.size, fmt, float(np.float32(amax_value)),
                                 _ptr(meta), _ptr(q)) != 0:
        raise ValueError("bad FP8 format %r" % fmt)
    return q, meta


def quantize_fp8_prescaled(x, fmt: int, amax_value, world: int):
    """O1 pre-scaled quantization with the common amax of 'world' ranks.
    Returns (codes, meta float32[4] = {amax, scale, scale_inv, 0})."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.empty(x.shape, np.uint8)
    meta = np.zeros(4, np.float32)
    if lib().oracle_quantize_fp8_prescaled(_ptr(x), x.size, fmt, float(np.float32(amax_value)),
                                           int(world), _ptr(meta), _ptr(q)) != 0:
        raise ValueError("bad FP8 format or world size")
    return q, meta


def dequantize_fp8(q, fmt: int, scale_inv) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(q.shape, np.float32)
    if lib().oracle_dequantize_fp8(_ptr(q), q.size, fmt, float(np.float32(scale_inv)), _ptr(out)) != 0:
        raise ValueError("bad FP8 format %r" % fmt)
    return out


# ---------------------------------------------------------------- AdamW ---

def adamw_constants(step: int, **hp) -> np.ndarray:
    """[B1, OB1, B2, OB2, EPS, SS, IBS, DEC, WD] as float32."""
    k = np.zeros(9, np.float32)
    h = _hp(**hp)
    lib().oracle_adamw_constants(ctypes.byref(h), int(step), _ptr(k))
    return k


def adamw_f32_tensor(g, m, v, w, step: int, adam: bool = False, **hp) -> None:
    """AdamW (adam=True: Adam with coupled L2) with binary32 states, in place
    on m, v, w (float32 arrays)."""
    for a in (m, v, w):
        assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"]
    g = np.ascontiguousarray(g, dtype=np.float32)
    h = _hp(**hp)
    lib().oracle_adamw_f32_tensor(g.size, _ptr(g), _ptr(m), _ptr(v), _ptr(w), ctypes.byref(h),
                                  int(step), int(bool(adam)))


def adamw_o2_tensor(qg, gfmt, g_scale_inv, qm, m_meta, v, w, step: int, adam: bool = False,
                    **hp) -> None:
    """One O2 step on one tensor, in place on qm (uint8), m_meta (float32[4]),
    v and w (uint16 FP16 bits). adam=True: Adam (coupled L2) instead of AdamW."""
    assert qm.dtype == np.uint8 and v.dtype == np.uint16 and w.dtype == np.uint16
    assert m_meta.dtype == np.float32 and m_meta.size >= 3
    qg = np.ascontiguousarray(qg, dtype=np.uint8)
    h = _hp(**hp)
    rc = lib().oracle_adamw_o2_tensor(qg.size, _ptr(qg), gfmt, float(np.float32(g_scale_inv)),
                                      _ptr(qm), _ptr(m_meta), _ptr(v), _ptr(w), ctypes.byref(h),
                                      int(step), int(bool(adam)))
    if rc != 0:
        raise RuntimeError("oracle_adamw_o2_tensor failed (%d)" % rc)


def adamw_o2_tensor_delayed(qg, gfmt, g_scale_inv, qm, m_meta, v, w, step: int, adam: bool = False,
                            **hp) -> None:
    """Ablation: one-pass O2 step with delayed scaling of the first moment
    (codes encoded with the scale of the previous step's amax)."""
    assert qm.dtype == np.uint8 and v.dtype == np.uint16 and w.dtype == np.uint16
    qg = np.ascontiguousarray(qg, dtype=np.uint8)
    h = _hp(**hp)
    rc = lib().oracle_adamw_o2_tensor_delayed(qg.size, _ptr(qg), gfmt, float(np.float32(g_scale_inv)),
                                              _ptr(qm), _ptr(m_meta), _ptr(v), _ptr(w),
                                              ctypes.byref(h), int(step), int(bool(adam)))
    if rc != 0:
        raise RuntimeError("oracle_adamw_o2_tensor_delayed failed (%d)" % rc)


def adamw_o2_tensor_scaled_v(qg, gfmt, g_scale_inv, qm, m_meta, v, v_meta, w, step: int, **hp) -> None:
    """Ablation: O2 step with a per-tensor-scaled FP16 second moment (v_meta:
    float32[4] {amax, scale, scale_inv, 0} of the stored v)."""
    assert v_meta.dtype == np.float32 and v_meta.size >= 3
    qg = np.ascontiguousarray(qg, dtype=np.uint8)
    h = _hp(**hp)
    rc = lib().oracle_adamw_o2_tensor_scaled_v(qg.size, _ptr(qg), gfmt, float(np.float32(g_scale_inv)),
                                               _ptr(qm), _ptr(m_meta), _ptr(v), _ptr(v_meta), _ptr(w),
                                               ctypes.byref(h), int(step))
    if rc != 0:
        raise RuntimeError("oracle_adamw_o2_tensor_scaled_v failed (%d)" % rc)


def adamw_o3_tensor(qg, gfmt, g_scale_inv, qm, m_meta, v, master, w8, w8_meta, step: int,
                    adam: bool = False, **hp) -> None:
    """One O3 step on one tensor, in place on qm, m_meta, v, master (FP16
    bits), w8 (uint8 E4M3) and w8_meta (float32[4])."""
    assert master.dtype == np.uint16 and w8.dtype == np.uint8 and w8_meta.dtype == np.float32
    qg = np.ascontiguousarray(qg, dtype=np.uint8)
    h = _hp(**hp)
    rc = lib().oracle_adamw_o3_tensor(qg.size, _ptr(qg), gfmt, float(np.float32(g_scale_inv)),
                                      _ptr(qm), _ptr(m_meta), _ptr(v), _ptr(master), _ptr(w8),
                                      _ptr(w8_meta), ctypes.byref(h), int(step), int(bool(adam)))
    if rc != 0:
        raise RuntimeError("oracle_adamw_o3_tensor failed (%d)" % rc)


# ----------------------------------------------------- list-level steps ---

class TensorState:
    """Host copy of one tensor's low-precision optimizer state."""

    def __init__(self, weight_f16_bits: np.ndarray, level: str = "O2", adam: bool = False,
                 delayed: bool = False, scaled_v: bool = False):
        n = weight_f16_bits.size
        self.level = level
        self.adam = adam  # Adam with coupled L2 instead of AdamW
        self.delayed = delayed  # one-pass delayed-scaling ablation (O2 only)
        self.scaled_v = scaled_v  # scaled-FP16-v ablation (O2 AdamW only)
        assert not ((delayed or scaled_v) and level != "O2")
        self.v_meta = np.array([0.0, 1.0, 1.0, 0.0], np.float32)
        self.w = np.ascontiguousarray(weight_f16_bits, dtype=np.uint16).copy()  # weight or master
        self.m = np.zeros(n, np.uint8)
        self.m_meta = np.array([0.0, 1.0, 1.0, 0.0], np.float32)
        self.v = np.zeros(n, np.uint16)
        if level == "O3":
            self.w8 = np.zeros(n, np.uint8)
            self.w8_meta = np.array([0.0, 1.0, 1.0, 0.0], np.float32)


def step_tensor(state: TensorState, grad_f32: np.ndarray, gfmt: int, step: int, **hp):
    """Gradient amax + quantize, then one O2/O3 step of one tensor's state.
    Returns the gradient (codes, meta)."""
    qg, gmeta = quantize_fp8(grad_f32, gfmt)
    if state.level == "O2" and state.scaled_v:
        adamw_o2_tensor_scaled_v(qg, gfmt, gmeta[2], state.m, state.m_meta, state.v, state.v_meta,
                                 state.w, step, **hp)
    elif state.level == "O2" and state.delayed:
        adamw_o2_tensor_delayed(qg, gfmt, gmeta[2], state.m, state.m_meta, state.v, state.w, step,
                                adam=state.adam, **hp)
    elif state.level == "O2":
        adamw_o2_tensor(qg, gfmt, gmeta[2], state.m, state.m_meta, state.v, state.w, step,
                        adam=state.adam, **hp)
    else:
        adamw_o3_tensor(qg, gfmt, gmeta[2], state.m, state.m_meta, state.v, state.w, state.w8,
                        state.w8_meta, step, adam=state.adam, **hp)
    return qg, gmeta


def step_list(states, grads_f32, gfmt: int, step: int, threads: int = 1, **hp):
    """Grad amax + quantize + one O2/O3 step for every tensor of a list.
    Returns the per-tensor (codes, meta) of the quantized gradients."""
    if threads <= 1:
        return [step_tensor(s, g, gfmt, step, **hp) for s, g in zip(states, grads_f32)]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        futs = [ex.submit(step_tensor, s, g, gfmt, step, **hp) for s, g in zip(states, grads_f32)]
        return [f.result() for f in futs]
