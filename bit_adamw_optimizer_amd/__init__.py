"""MI355X (gfx950) library for the per-tensor-scaled low-precision AdamW step
of MS-AMP's O2 and O3 optimization levels, with the per-tensor amax
reductions and saturating FP8 casts around it.

This module is the thin Python binding of ``libmsamp.so`` (C ABI declared in
``include/msamp.h``): it only checks tensor arguments and marshals device
pointers, sizes and the current HIP stream. Every step of the computation runs
in the library's HIP kernels; there is no fallback. PyTorch provides device
memory and streams.

Layouts (MS-AMP "Optimization Level" page, sections O2/O3 and the table):
  O2: grad FP8 (per-tensor scale), exp_avg FP8 E4M3 (own scale), exp_avg_sq
      FP16, weight FP16.
  O3: as O2 with the weight replaced by an FP16 master, plus an FP8 E4M3
      weight copy with its own scale.
FP8 codes are ``torch.uint8`` tensors (a ``float8_e4m3fn``/``float8_e5m2``
tensor may be passed, it is read as bytes); FP16 tensors are
``torch.float16`` (or 16-bit integer views). A meta array is a contiguous
``float32`` device tensor of shape ``(n, 4)``: ``[amax, scale, scale_inv,
reserved]`` per tensor.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "E4M3", "E5M2", "MsampError", "TensorList", "lib", "library_path", "KERNELS",
    # gradient producer
    "amax", "quantize_fp8", "quantize_fp8_prescaled", "dequantize_fp8",
    # steps
    "adamw_o2_step", "adamw_o3_step", "adam_o2_step", "adam_o3_step",
    "step_constants", "adamw_o2_step_devconst", "adamw_o3_step_devconst", "adamw_step_phase",
    "adamw_o2_step_noalloc", "quantize_adamw_o2_step", "quantize_adamw_o3_step",
    "quantize_adamw_o2_step_devconst", "quantize_adamw_o3_step_devconst",
    # ablations
    "adamw_o2_step_delayed", "adamw_o2_step_scaled_v",
    # state helpers
    "new_meta", "allocate_state", "flat_views", "state_bytes_per_param",
    # measurement and test aids
    "rmw_probe", "quantize_pass1_probe", "stream_probe", "codec_probe", "profile_enable", "profile_select", "profile_read", "release_cache",
    "unpin_captured_tables", "cache_stats",
]

E4M3 = 0
E5M2 = 1

PROBE_F32_TO_E4M3 = 0
PROBE_F32_TO_E5M2 = 1
PROBE_E4M3_TO_F32 = 2
PROBE_E5M2_TO_F32 = 3
PROBE_F32_TO_F16 = 4
PROBE_F16_TO_F32 = 5

# kernel kinds of msamp_profile_read, in enum order
KERNELS = ["amax", "quantize_fp8", "dequantize_fp8", "step_pass1", "o2_pass2", "o3_pass2",
           "o3_pass3", "finalize", "amax_finalize", "o2_delayed", "rmw_probe", "quantize_pass1",
           "read_probe", "copy_probe", "qp1_probe"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "_lib", "libmsamp.so")

_STATUS = {0: "MSAMP_OK", 1: "MSAMP_E_INVALID_ARG", 2: "MSAMP_E_MISALIGNED", 3: "MSAMP_E_HIP",
           4: "MSAMP_E_NO_MEMORY"}


class MsampError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_STATUS.get(status, str(status)), message))
        self.status = status


class _HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double)]


class _StepConstants(ctypes.Structure):
    _fields_ = [(k, ctypes.c_float) for k in ("b1", "ob1", "b2", "ob2", "eps", "ss", "ibs", "dec", "wd")]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libmsamp.so. Raises if it has not been built: there is no
    other implementation to fall back to."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libmsamp.so is not built (%s); run __graft_entry__.build() "
                               "or python -m bit_adamw_optimizer_amd.build" % _LIB_PATH)
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        st = ctypes.c_int
        L.msamp_abi_version.argtypes = []
        L.msamp_abi_version.restype = ctypes.c_int
        L.msamp_last_error.argtypes = []
        L.msamp_last_error.restype = ctypes.c_char_p
        L.msamp_amax.argtypes = [i32, vp, vp, vp, vp]
        L.msamp_amax.restype = st
        L.msamp_quantize_fp8.argtypes = [i32, vp, vp, ctypes.c_int, vp, vp, vp]
        L.msamp_quantize_fp8.restype = st
        L.msamp_quantize_fp8_prescaled.argtypes = [i32, vp, vp, ctypes.c_int, vp, i32, vp, vp]
        L.msamp_quantize_fp8_prescaled.restype = st
        L.msamp_dequantize_fp8.argtypes = [i32, vp, vp, ctypes.c_int, vp, vp, vp]
        L.msamp_dequantize_fp8.restype = st
        L.msamp_adamw_o2_step.argtypes = [i32, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp,
                                          ctypes.POINTER(_HParams), i64, vp]
        L.msamp_adamw_o2_step.restype = st
        L.msamp_adamw_o3_step.argtypes = [i32, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp,
                                          ctypes.POINTER(_HParams), i64, vp]
        L.msamp_adamw_o3_step.restype = st
        L.msamp_quantize_adamw_o2_step.argtypes = [i32, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp,
                                                   ctypes.POINTER(_HParams), i64, vp]
        L.msamp_quantize_adamw_o2_step.restype = st
        L.msamp_quantize_adamw_o3_step.argtypes = [i32, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp,
                                                   vp, ctypes.POINTER(_HParams), i64, vp]
        L.msamp_quantize_adamw_o3_step.restype = st
        L.msamp_quantize_adam_o2_step.argtypes = L.msamp_quantize_adamw_o2_step.argtypes
        L.msamp_quantize_adam_o2_step.restype = st
        L.msamp_quantize_adam_o3_step.argtypes = L.msamp_quantize_adamw_o3_step.argtypes
        L.msamp_quantize_adam_o3_step.restype = st
        L.msamp_quantize_adamw_o2_step_devconst.argtypes = [i32, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp,
                                                            vp, ctypes.c_int, vp]
        L.msamp_quantize_adamw_o2_step_devconst.restype = st
        L.msamp_quantize_adamw_o3_step_devconst.argtypes = [i32, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp,
                                                            vp, vp, vp, ctypes.c_int, vp]
        L.msamp_quantize_adamw_o3_step_devconst.restype = st
        L.msamp_adamw_o2_step_noalloc.argtypes = L.msamp_adamw_o2_step.argtypes
        L.msamp_adamw_o2_step_noalloc.restype = st
        L.msamp_adam_o2_step.argtypes = L.msamp_adamw_o2_step.argtypes
        L.msamp_adam_o2_step.restype = st
        L.msamp_adam_o3_step.argtypes = L.msamp_adamw_o3_step.argtypes
        L.msamp_adam_o3_step.restype = st
        L.msamp_adamw_o2_step_delayed.argtypes = L.msamp_adamw_o2_step.argtypes
        L.msamp_adamw_o2_step_delayed.restype = st
        L.msamp_adamw_o2_step_scaled_v.argtypes = [i32, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp,
                                                   ctypes.POINTER(_HParams), i64, vp]
        L.msamp_adamw_o2_step_scaled_v.restype = st
        o2_args = [i32, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp]
        o3_args = [i32, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp]
        hp_args = [ctypes.POINTER(_HParams), i64, ctypes.c_int]
        L.msamp_adamw_o2_step_phase1.argtypes = o2_args + hp_args + [vp, vp]
        L.msamp_adamw_o2_step_phase2.argtypes = o2_args + hp_args + [vp, vp]
        L.msamp_adamw_o3_step_phase1.argtypes = o3_args + hp_args + [vp, vp]
        L.msamp_adamw_o3_step_phase2.argtypes = o3_args + hp_args + [vp, vp, vp]
        L.msamp_adamw_o3_step_phase3.argtypes = o3_args + [vp, vp]
        for f in ("o2_step_phase1", "o2_step_phase2", "o3_step_phase1", "o3_step_phase2", "o3_step_phase3"):
            getattr(L, "msamp_adamw_" + f).restype = st
        L.msamp_quantize_pass1_probe.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp]
        L.msamp_quantize_pass1_probe.restype = st
        L.msamp_stream_probe.argtypes = [ctypes.c_int, vp, vp, i64, vp]
        L.msamp_stream_probe.restype = st
        L.msamp_rmw_probe.argtypes = [i32, vp, vp, vp, vp, vp, vp]
        L.msamp_rmw_probe.restype = st
        L.msamp_step_constants_compute.argtypes = [ctypes.POINTER(_HParams), i64, ctypes.c_int,
                                                   ctypes.POINTER(_StepConstants)]
        L.msamp_step_constants_compute.restype = st
        L.msamp_adamw_o2_step_devconst.argtypes = [i32, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp,
                                                   ctypes.c_int, vp]
        L.msamp_adamw_o2_step_devconst.restype = st
        L.msamp_adamw_o3_step_devconst.argtypes = [i32, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp,
                                                   vp, vp, ctypes.c_int, vp]
        L.msamp_adamw_o3_step_devconst.restype = st
        L.msamp_release_cache.argtypes = []
        L.msamp_release_cache.restype = st
        L.msamp_unpin_captured_tables.argtypes = []
        L.msamp_unpin_captured_tables.restype = st
        L.msamp_cache_stats.argtypes = [ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.msamp_cache_stats.restype = st
        L.msamp_codec_probe.argtypes = [ctypes.c_int, vp, vp, i64, vp]
        L.msamp_codec_probe.restype = st
        L.msamp_profile_enable.argtypes = [ctypes.c_int]
        L.msamp_profile_select.argtypes = [ctypes.c_uint32]
        L.msamp_profile_select.restype = st
        L.msamp_profile_enable.restype = st
        L.msamp_profile_read.argtypes = [ctypes.c_int, ctypes.POINTER(i64),
                                         ctypes.POINTER(ctypes.c_double)]
        L.msamp_profile_read.restype = st
        L.msamp_kernel_name.argtypes = [ctypes.c_int]
        L.msamp_kernel_name.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise MsampError(status, lib().msamp_last_error().decode())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# ------------------------------------------------------------ tensor lists ---

_BYTES = {"u8": 1, "f16": 2, "f32": 4}


def _role_ok(t: torch.Tensor, kind: str) -> bool:
    if kind == "u8":
        return t.element_size() == 1
    if kind == "f16":
        return t.dtype in (torch.float16, torch.int16, torch.uint16)
    if kind == "f32":
        return t.dtype == torch.float32
    raise ValueError(kind)


_SIZES = {}  # sizes tuple -> the one instance that equal TensorLists share


def _shared_sizes(sizes) -> tuple:
    t = tuple(sizes)
    u = _SIZES.get(t)
    if u is None:
        if len(_SIZES) >= 256:
            _SIZES.clear()
        _SIZES[t] = u = t
    return u


class TensorList:
    """Pointer array and sizes of a list of device tensors, built once.

    An optimizer holds one TensorList per role (grads, exp_avg, ...) for the
    lifetime of its parameters, so marshalling is not repeated every step.
    """

    def __init__(self, tensors: Sequence[torch.Tensor], kind: str, name: str = "tensor"):
        self.tensors = list(tensors)
        self.kind = kind
        n = len(self.tensors)
        self.n = n
        ptrs = (ctypes.c_void_p * max(n, 1))()
        numel = (ctypes.c_int64 * max(n, 1))()
        self.device = None
        for i, t in enumerate(self.tensors):
            if not isinstance(t, torch.Tensor):
                raise TypeError("%s[%d] is not a tensor" % (name, i))
            if not _role_ok(t, kind):
                raise TypeError("%s[%d] has dtype %s, expected %s" % (name, i, t.dtype, kind))
            if not t.is_contiguous():
                raise ValueError("%s[%d] is not contiguous" % (name, i))
            if t.device.type != "cuda":
                raise ValueError("%s[%d] is not on a GPU" % (name, i))
            if self.device is None:
                self.device = t.device
            elif t.device != self.device:
                raise ValueError("%s[%d] is on %s, expected %s" % (name, i, t.device, self.device))
            ptrs[i] = t.data_ptr() if t.numel() else 0
            numel[i] = t.numel()
        self.ptrs = ptrs
        self.numel = numel
        self.sizes = _shared_sizes(t.numel() for t in self.tensors)

    def matches(self, other: "TensorList", name: str) -> None:
        # lists of equal sizes built in this process share one sizes tuple,
        # so the usual check is an identity test, not n comparisons
        if other.n != self.n or (other.sizes is not self.sizes and other.sizes != self.sizes):
            raise ValueError("%s does not match the tensor sizes of the list" % name)
        if other.n and other.device != self.device:
            raise ValueError("%s is on another device" % name)


def _tl(x, kind: str, name: str) -> TensorList:
    return x if isinstance(x, TensorList) else TensorList(x, kind, name)


def _meta_ptr(meta: torch.Tensor, n: int, device, name: str):
    if not isinstance(meta, torch.Tensor) or meta.dtype != torch.float32:
        raise TypeError("%s must be a float32 tensor" % name)
    if tuple(meta.shape) != (n, 4) or not meta.is_contiguous():
        raise ValueError("%s must be a contiguous (%d, 4) tensor" % (name, n))
    if n and meta.device != device:
        raise ValueError("%s is not on %s" % (name, device))
    return ctypes.c_void_p(meta.data_ptr() if n else 0)


def new_meta(n: int, device) -> torch.Tensor:
    """Meta array of n tensors in the initial state {amax 0, scale 1,
    scale_inv 1, 0}."""
    m = torch.zeros((n, 4), dtype=torch.float32, device=device)
    m[:, 1] = 1.0
    m[:, 2] = 1.0
    return m


def _hp(lr, betas, eps, weight_decay) -> _HParams:
    return _HParams(float(lr), float(betas[0]), float(betas[1]), float(eps), float(weight_decay))


# --------------------------------------------------------------- entry points

def amax(x, meta: torch.Tensor) -> None:
    """meta[t, 0] <- amax of x[t] (binary32 tensors)."""
    x = _tl(x, "f32", "x")
    if x.n == 0:
        return
    with torch.cuda.device(x.device):
        _check(lib().msamp_amax(x.n, x.ptrs, x.numel, _meta_ptr(meta, x.n, x.device, "meta"),
                                _stream(x.device)))


def quantize_fp8(x, fmt: int, meta: torch.Tensor, q) -> None:
    """q[t] <- saturating FP8 cast of x[t] * scale(meta[t, 0]); meta[t, 1:3]
    <- scale, 1/scale."""
    x = _tl(x, "f32", "x")
    q = _tl(q, "u8", "q")
    x.matches(q, "q")
    if x.n == 0:
        return
    with torch.cuda.device(x.device):
        _check(lib().msamp_quantize_fp8(x.n, x.ptrs, x.numel, int(fmt),
                                        _meta_ptr(meta, x.n, x.device, "meta"), q.ptrs,
                                        _stream(x.device)))


def quantize_fp8_prescaled(x, fmt: int, meta: torch.Tensor, world_size: int, q) -> None:
    """Pre-scaled quantize before an FP8 all-reduce over world_size ranks:
    meta[t, 0] holds the common amax; scale = scale(amax * world_size)."""
    x = _tl(x, "f32", "x")
    q = _tl(q, "u8", "q")
    x.matches(q, "q")
    if x.n == 0:
        return
    with torch.cuda.device(x.device):
        _check(lib().msamp_quantize_fp8_prescaled(x.n, x.ptrs, x.numel, int(fmt),
                                                  _meta_ptr(meta, x.n, x.device, "meta"),
                                                  int(world_size), q.ptrs, _stream(x.device)))


def dequantize_fp8(q, fmt: int, meta: torch.Tensor, out) -> None:
    """out[t] <- decode(q[t]) * meta[t, 2]."""
    q = _tl(q, "u8", "q")
    out = _tl(out, "f32", "out")
    q.matches(out, "out")
    if q.n == 0:
        return
    with torch.cuda.device(q.device):
        _check(lib().msamp_dequantize_fp8(q.n, q.ptrs, q.numel, int(fmt),
                                          _meta_ptr(meta, q.n, q.device, "meta"), out.ptrs,
                                          _stream(q.device)))


def adamw_o2_step(grad, grad_fmt: int, grad_meta, exp_avg, exp_avg_meta, exp_avg_sq, weight,
                  *, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01, step: int,
                  _entry: str = "msamp_adamw_o2_step") -> None:
    """One in-place AdamW step in the O2 layout (see include/msamp.h)."""
    g = _tl(grad, "u8", "grad")
    m = _tl(exp_avg, "u8", "exp_avg")
    v = _tl(exp_avg_sq, "f16", "exp_avg_sq")
    w = _tl(weight, "f16", "weight")
    for other, name in ((m, "exp_avg"), (v, "exp_avg_sq"), (w, "weight")):
        g.matches(other, name)
    if g.n == 0:
        return
    hp = _hp(lr, betas, eps, weight_decay)
    with torch.cuda.device(g.device):
        _check(getattr(lib(), _entry)(
            g.n, g.numel, g.ptrs, int(grad_fmt), _meta_ptr(grad_meta, g.n, g.device, "grad_meta"),
            m.ptrs, _meta_ptr(exp_avg_meta, g.n, g.device, "exp_avg_meta"), v.ptrs, w.ptrs,
            ctypes.byref(hp), int(step), _stream(g.device)))


def adamw_o3_step(grad, grad_fmt: int, grad_meta, exp_avg, exp_avg_meta, exp_avg_sq, master,
                  weight_fp8, weight_fp8_meta, *, lr=1e-3, betas=(0.9, 0.999), eps=1e-8,
                  weight_decay=0.01, step: int, _entry: str = "msamp_adamw_o3_step") -> None:
    """One in-place AdamW step in the O3 layout (see include/msamp.h)."""
    g = _tl(grad, "u8", "grad")
    m = _tl(exp_avg, "u8", "exp_avg")
    v = _tl(exp_avg_sq, "f16", "exp_avg_sq")
    w = _tl(master, "f16", "master")
    w8 = _tl(weight_fp8, "u8", "weight_fp8")
    for other, name in ((m, "exp_avg"), (v, "exp_avg_sq"), (w, "master"), (w8, "weight_fp8")):
        g.matches(other, name)
    if g.n == 0:
        return
    hp = _hp(lr, betas, eps, weight_decay)
    with torch.cuda.device(g.device):
        _check(getattr(lib(), _entry)(
            g.n, g.numel, g.ptrs, int(grad_fmt), _meta_ptr(grad_meta, g.n, g.device, "grad_meta"),
            m.ptrs, _meta_ptr(exp_avg_meta, g.n, g.device, "exp_avg_meta"), v.ptrs, w.ptrs,
            w8.ptrs, _meta_ptr(weight_fp8_meta, g.n, g.device, "weight_fp8_meta"),
            ctypes.byref(hp), int(step), _stream(g.device)))


def quantize_adamw_o2_step(grad_f32, grad_fmt: int, grad_meta, grad, exp_avg, exp_avg_meta, exp_avg_sq,
                           weight, *, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01,
                           step: int, adam: bool = False) -> None:
    """Gradient quantize fused with the O2 AdamW step (Adam with adam=True;
    see include/msamp.h): grad_meta must hold the gradient amax; grad
    receives the FP8 codes."""
    hp = _hp(lr, betas, eps, weight_decay)
    _quantize_step("O2", "msamp_quantize_adam_o2_step" if adam else "msamp_quantize_adamw_o2_step",
                   grad_f32, grad_fmt, grad_meta, grad, exp_avg, exp_avg_meta, exp_avg_sq, weight, None, None,
                   (ctypes.byref(hp), int(step)))


def quantize_adamw_o3_step(grad_f32, grad_fmt: int, grad_meta, grad, exp_avg, exp_avg_meta, exp_avg_sq,
                           master, weight_fp8, weight_fp8_meta, *, lr=1e-3, betas=(0.9, 0.999), eps=1e-8,
                           weight_decay=0.01, step: int, adam: bool = False) -> None:
    """Gradient quantize fused with the O3 AdamW step (Adam with adam=True;
    see include/msamp.h)."""
    hp = _hp(lr, betas, eps, weight_decay)
    _quantize_step("O3", "msamp_quantize_adam_o3_step" if adam else "msamp_quantize_adamw_o3_step",
                   grad_f32, grad_fmt, grad_meta, grad, exp_avg, exp_avg_meta, exp_avg_sq, master, weight_fp8,
                   weight_fp8_meta, (ctypes.byref(hp), int(step)))


def quantize_adamw_o2_step_devconst(grad_f32, grad_fmt: int, grad_meta, grad, exp_avg, exp_avg_meta,
                                    exp_avg_sq, weight, consts: torch.Tensor, adam: bool = False) -> None:
    """msamp_quantize_adamw_o2_step_devconst: the fused O2 step with the
    step's constants read from 'consts' (see step_constants) when it runs."""
    g = _tl(grad_f32, "f32", "grad_f32")
    _quantize_step("O2", "msamp_quantize_adamw_o2_step_devconst", grad_f32, grad_fmt, grad_meta, grad, exp_avg,
                   exp_avg_meta, exp_avg_sq, weight, None, None,
                   (_consts_ptr(consts, g.device), 1 if adam else 0))


def quantize_adamw_o3_step_devconst(grad_f32, grad_fmt: int, grad_meta, grad, exp_avg, exp_avg_meta,
                                    exp_avg_sq, master, weight_fp8, weight_fp8_meta, consts: torch.Tensor,
                                    adam: bool = False) -> None:
    """msamp_quantize_adamw_o3_step_devconst (see quantize_adamw_o2_step_devconst)."""
    g = _tl(grad_f32, "f32", "grad_f32")
    _quantize_step("O3", "msamp_quantize_adamw_o3_step_devconst", grad_f32, grad_fmt, grad_meta, grad, exp_avg,
                   exp_avg_meta, exp_avg_sq, master, weight_fp8, weight_fp8_meta,
                   (_consts_ptr(consts, g.device), 1 if adam else 0))


def _quantize_step(level, entry, grad_f32, grad_fmt, grad_meta, grad, exp_avg, exp_avg_meta, exp_avg_sq, weight,
                   weight_fp8, weight_fp8_meta, tail) -> None:
    x = _tl(grad_f32, "f32", "grad_f32")
    g = _tl(grad, "u8", "grad")
    m = _tl(exp_avg, "u8", "exp_avg")
    v = _tl(exp_avg_sq, "f16", "exp_avg_sq")
    w = _tl(weight, "f16", "weight" if level == "O2" else "master")
    lists = [(g, "grad"), (m, "exp_avg"), (v, "exp_avg_sq"), (w, "weight")]
    w8 = None
    if level == "O3":
        w8 = _tl(weight_fp8, "u8", "weight_fp8")
        lists.append((w8, "weight_fp8"))
    for other, name in lists:
        x.matches(other, name)
    if x.n == 0:
        return
    with torch.cuda.device(x.device):
        args = [x.n, x.numel, x.ptrs, int(grad_fmt), _meta_ptr(grad_meta, x.n, x.device, "grad_meta"), g.ptrs,
                m.ptrs, _meta_ptr(exp_avg_meta, x.n, x.device, "exp_avg_meta"), v.ptrs, w.ptrs]
        if level == "O3":
            args += [w8.ptrs, _meta_ptr(weight_fp8_meta, x.n, x.device, "weight_fp8_meta")]
        _check(getattr(lib(), entry)(*args, *tail, _stream(x.device)))


def step_constants(*, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01, step: int,
                   adam: bool = False) -> torch.Tensor:
    """The binary32 constants of one AdamW (adam=True: Adam) step as a CPU
    float32 tensor of 9 values (msamp_step_constants), bit-identical to what
    the by-value step entry points use."""
    out = _StepConstants()
    hp = _hp(lr, betas, eps, weight_decay)
    _check(lib().msamp_step_constants_compute(ctypes.byref(hp), int(step), int(bool(adam)),
                                              ctypes.byref(out)))
    return torch.tensor([getattr(out, k) for k, _ in _StepConstants._fields_], dtype=torch.float32)


def _consts_ptr(consts: torch.Tensor, device):
    if not isinstance(consts, torch.Tensor) or consts.dtype != torch.float32 or consts.numel() != 9 \
            or not consts.is_contiguous():
        raise ValueError("consts must be a contiguous float32 tensor of 9 values")
    if consts.device != device:
        raise ValueError("consts is not on %s" % device)
    return ctypes.c_void_p(consts.data_ptr())


def adamw_o2_step_devconst(grad, grad_fmt: int, grad_meta, exp_avg, exp_avg_meta, exp_avg_sq, weight,
                           consts: torch.Tensor, *, adam: bool = False) -> None:
    """The O2 step with its constants read from the device tensor 'consts'
    when the kernels run (capturable in a HIP graph; see
    msamp_adamw_o2_step_devconst in include/msamp.h)."""
    g = _tl(grad, "u8", "grad")
    m = _tl(exp_avg, "u8", "exp_avg")
    v = _tl(exp_avg_sq, "f16", "exp_avg_sq")
    w = _tl(weight, "f16", "weight")
    for other, name in ((m, "exp_avg"), (v, "exp_avg_sq"), (w, "weight")):
        g.matches(other, name)
    if g.n == 0:
        return
    with torch.cuda.device(g.device):
        _check(lib().msamp_adamw_o2_step_devconst(
            g.n, g.numel, g.ptrs, int(grad_fmt), _meta_ptr(grad_meta, g.n, g.device, "grad_meta"),
            m.ptrs, _meta_ptr(exp_avg_meta, g.n, g.device, "exp_avg_meta"), v.ptrs, w.ptrs,
            _consts_ptr(consts, g.device), int(bool(adam)), _stream(g.device)))


def adamw_o3_step_devconst(grad, grad_fmt: int, grad_meta, exp_avg, exp_avg_meta, exp_avg_sq, master,
                           weight_fp8, weight_fp8_meta, consts: torch.Tensor, *,
                           adam: bool = False) -> None:
    """The O3 step with its constants read from the device tensor 'consts'
    (see msamp_adamw_o3_step_devconst in include/msamp.h)."""
    g = _tl(grad, "u8", "grad")
    m = _tl(exp_avg, "u8", "exp_avg")
    v = _tl(exp_avg_sq, "f16", "exp_avg_sq")
    w = _tl(master, "f16", "master")
    w8 = _tl(weight_fp8, "u8", "weight_fp8")
    for other, name in ((m, "exp_avg"), (v, "exp_avg_sq"), (w, "master"), (w8, "weight_fp8")):
        g.matches(other, name)
    if g.n == 0:
        return
    with torch.cuda.device(g.device):
        _check(lib().msamp_adamw_o3_step_devconst(
            g.n, g.numel, g.ptrs, int(grad_fmt), _meta_ptr(grad_meta, g.n, g.device, "grad_meta"),
            m.ptrs, _meta_ptr(exp_avg_meta, g.n, g.device, "exp_avg_meta"), v.ptrs, w.ptrs,
            w8.ptrs, _meta_ptr(weight_fp8_meta, g.n, g.device, "weight_fp8_meta"),
            _consts_ptr(consts, g.device), int(bool(adam)), _stream(g.device)))


def _amax_ptr(a, n: int, device, name: str):
    if not isinstance(a, torch.Tensor) or a.dtype != torch.float32 or a.numel() != n \
            or not a.is_contiguous():
        raise ValueError("%s must be a contiguous float32 tensor of %d values" % (name, n))
    if n and a.device != device:
        raise ValueError("%s is not on %s" % (name, device))
    return ctypes.c_void_p(a.data_ptr() if n else 0)


def adamw_step_phase(phase: int, level: str, grad, grad_fmt: int, grad_meta, exp_avg, exp_avg_meta,
                     exp_avg_sq, weight, weight_fp8=None, weight_fp8_meta=None, *, amax_in=None,
                     amax_out=None, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01,
                     step: int = 1, adam: bool = False) -> None:
    """One phase of the split-phase step on a rank's slices of the tensors
    (see msamp_adamw_o2_step_phase1 in include/msamp.h). phase 1: amax_out
    <- local first-moment amax. phase 2: update with the global first-moment
    amax amax_in (O3: amax_out <- local master amax). phase 3 (O3): FP8 copy
    with the global master amax amax_in."""
    g = _tl(grad, "u8", "grad")
    m = _tl(exp_avg, "u8", "exp_avg")
    v = _tl(exp_avg_sq, "f16", "exp_avg_sq")
    w = _tl(weight, "f16", "weight")
    lists = [(m, "exp_avg"), (v, "exp_avg_sq"), (w, "weight")]
    w8 = None
    if level == "O3":
        w8 = _tl(weight_fp8, "u8", "weight_fp8")
        lists.append((w8, "weight_fp8"))
    elif level != "O2" or phase == 3:
        raise ValueError("level must be O2 (phases 1, 2) or O3 (phases 1-3)")
    for other, name in lists:
        g.matches(other, name)
    if g.n == 0:
        return
    dev = g.device
    args = [g.n, g.numel, g.ptrs, int(grad_fmt), _meta_ptr(grad_meta, g.n, dev, "grad_meta"), m.ptrs,
            _meta_ptr(exp_avg_meta, g.n, dev, "exp_avg_meta"), v.ptrs, w.ptrs]
    if level == "O3":
        args += [w8.ptrs, _meta_ptr(weight_fp8_meta, g.n, dev, "weight_fp8_meta")]
    hp = _hp(lr, betas, eps, weight_decay)
    if phase in (1, 2):
        args += [ctypes.byref(hp), int(step), int(bool(adam))]
    if phase == 2:
        args.append(_amax_ptr(amax_in, g.n, dev, "amax_in"))
    if phase == 1 or (phase == 2 and level == "O3"):
        args.append(_amax_ptr(amax_out, g.n, dev, "amax_out"))
    if phase == 3:
        args.append(_amax_ptr(amax_in, g.n, dev, "amax_in"))
    entry = "msamp_adamw_%s_step_phase%d" % (level.lower(), phase)
    with torch.cuda.device(dev):
        _check(getattr(lib(), entry)(*args, _stream(dev)))


def adamw_o2_step_noalloc(*args, **kw) -> None:
    """msamp_adamw_o2_step_noalloc: the O2 AdamW step with its tables in the
    library's static device array (no allocation in the call); same arguments
    as adamw_o2_step."""
    adamw_o2_step(*args, _entry="msamp_adamw_o2_step_noalloc", **kw)


def adam_o2_step(*args, **kw) -> None:
    """One in-place Adam (coupled L2) step in the O2 layout; arguments as
    adamw_o2_step (see msamp_adam_o2_step in include/msamp.h)."""
    adamw_o2_step(*args, _entry="msamp_adam_o2_step", **kw)


def adam_o3_step(*args, **kw) -> None:
    """One in-place Adam (coupled L2) step in the O3 layout; arguments as
    adamw_o3_step (see msamp_adam_o3_step in include/msamp.h)."""
    adamw_o3_step(*args, _entry="msamp_adam_o3_step", **kw)


def adamw_o2_step_delayed(*args, **kw) -> None:
    """ABLATION: one-pass O2 AdamW step with delayed scaling of the first
    moment (see msamp_adamw_o2_step_delayed in include/msamp.h)."""
    adamw_o2_step(*args, _entry="msamp_adamw_o2_step_delayed", **kw)


def adamw_o2_step_scaled_v(grad, grad_fmt: int, grad_meta, exp_avg, exp_avg_meta, exp_avg_sq,
                           exp_avg_sq_meta, weight, *, lr=1e-3, betas=(0.9, 0.999), eps=1e-8,
                           weight_decay=0.01, step: int) -> None:
    """ABLATION: O2 AdamW step with a per-tensor-scaled FP16 second moment
    (see msamp_adamw_o2_step_scaled_v in include/msamp.h)."""
    g = _tl(grad, "u8", "grad")
    m = _tl(exp_avg, "u8", "exp_avg")
    v = _tl(exp_avg_sq, "f16", "exp_avg_sq")
    w = _tl(weight, "f16", "weight")
    for other, name in ((m, "exp_avg"), (v, "exp_avg_sq"), (w, "weight")):
        g.matches(other, name)
    if g.n == 0:
        return
    hp = _hp(lr, betas, eps, weight_decay)
    with torch.cuda.device(g.device):
        _check(lib().msamp_adamw_o2_step_scaled_v(
            g.n, g.numel, g.ptrs, int(grad_fmt), _meta_ptr(grad_meta, g.n, g.device, "grad_meta"),
            m.ptrs, _meta_ptr(exp_avg_meta, g.n, g.device, "exp_avg_meta"), v.ptrs,
            _meta_ptr(exp_avg_sq_meta, g.n, g.device, "exp_avg_sq_meta"), w.ptrs,
            ctypes.byref(hp), int(step), _stream(g.device)))


def rmw_probe(grad, exp_avg, exp_avg_sq, weight) -> None:
    """Measurement aid: the update pass's memory traffic on these tensor
    lists with none of its arithmetic (m, v, w are rewritten unchanged; see
    msamp_rmw_probe in include/msamp.h)."""
    g = _tl(grad, "u8", "grad")
    m = _tl(exp_avg, "u8", "exp_avg")
    v = _tl(exp_avg_sq, "f16", "exp_avg_sq")
    w = _tl(weight, "f16", "weight")
    for other, name in ((m, "exp_avg"), (v, "exp_avg_sq"), (w, "weight")):
        g.matches(other, name)
    if g.n == 0:
        return
    with torch.cuda.device(g.device):
        _check(lib().msamp_rmw_probe(g.n, g.numel, g.ptrs, m.ptrs, v.ptrs, w.ptrs, _stream(g.device)))


def quantize_pass1_probe(grad_f32, grad, exp_avg, exp_avg_sq, weight) -> None:
    """Measurement aid: the fused quantize + pass 1's traffic without its
    arithmetic (msamp_quantize_pass1_probe); overwrites the gradient codes."""
    x = _tl(grad_f32, "f32", "grad_f32")
    g = _tl(grad, "u8", "grad")
    m = _tl(exp_avg, "u8", "exp_avg")
    v = _tl(exp_avg_sq, "f16", "exp_avg_sq")
    w = _tl(weight, "f16", "weight")
    for other, name in ((g, "grad"), (m, "exp_avg"), (v, "exp_avg_sq"), (w, "weight")):
        x.matches(other, name)
    if x.n == 0:
        return
    with torch.cuda.device(x.device):
        _check(lib().msamp_quantize_pass1_probe(x.n, x.numel, x.ptrs, g.ptrs, m.ptrs, v.ptrs, w.ptrs,
                                                _stream(x.device)))


def stream_probe(src: torch.Tensor, dst: Optional[torch.Tensor] = None) -> None:
    """Measurement aid: reads all of 'src' (dst None) or copies it into
    'dst' (msamp_stream_probe); contiguous tensors of a multiple of 16 bytes."""
    nbytes = src.numel() * src.element_size()
    if not src.is_contiguous() or (dst is not None and not dst.is_contiguous()):
        raise ValueError("stream_probe needs contiguous tensors")
    if dst is not None and dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    with torch.cuda.device(src.device):
        _check(lib().msamp_stream_probe(0 if dst is None else 1, ctypes.c_void_p(src.data_ptr()),
                                        ctypes.c_void_p(dst.data_ptr() if dst is not None else 0),
                                        nbytes, _stream(src.device)))


def codec_probe(op: int, inp: torch.Tensor, out: torch.Tensor) -> None:
    """Element-wise device codec (see msamp_codec_probe)."""
    if inp.device.type != "cuda" or out.device.type != "cuda":
        raise ValueError("codec_probe needs device tensors")
    if inp.numel() != out.numel() or not inp.is_contiguous() or not out.is_contiguous():
        raise ValueError("codec_probe needs contiguous tensors of equal size")
    with torch.cuda.device(inp.device):
        _check(lib().msamp_codec_probe(int(op), ctypes.c_void_p(inp.data_ptr()),
                                       ctypes.c_void_p(out.data_ptr()), inp.numel(),
                                       _stream(inp.device)))


def release_cache() -> None:
    _check(lib().msamp_release_cache())


def unpin_captured_tables() -> None:
    """msamp_unpin_captured_tables: call after destroying graphs that
    captured library calls."""
    _check(lib().msamp_unpin_captured_tables())


def cache_stats() -> dict:
    """Cached tensor-list tables: {"lists", "bytes", "pinned"}."""
    a, b, c = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib().msamp_cache_stats(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return {"lists": a.value, "bytes": b.value, "pinned": c.value}


def profile_enable(on: bool) -> None:
    _check(lib().msamp_profile_enable(1 if on else 0))


def profile_select(kernels=None) -> None:
    """Time only these kernel kinds (names from KERNELS; None: all)."""
    mask = 0xFFFFFFFF if kernels is None else sum(1 << KERNELS.index(k) for k in kernels)
    _check(lib().msamp_profile_select(ctypes.c_uint32(mask)))


def profile_read(kernel: str):
    """(launches, total milliseconds) recorded for one kernel kind."""
    kind = KERNELS.index(kernel)
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    _check(lib().msamp_profile_read(kind, ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)


# ----------------------------------------------------------- state helpers ---

# Views into one allocation start at multiples of this many bytes. The
# library needs 16-byte aligned tensors; a start that is not on a 64-byte
# memory segment makes the first and last segment of every wave-wide access
# shared with the neighbouring access, and each such segment then moves
# twice (non-temporal accesses do not keep it in L2).
FLAT_ALIGN_BYTES = 256


def flat_views(sizes: Sequence[int], dtype, device, fill=0):
    """One contiguous allocation holding len(sizes) tensors, returned as 1-D
    views, each starting at a multiple of FLAT_ALIGN_BYTES. On MI355X one
    large buffer per role streams faster than many separate allocations."""
    align = max(1, FLAT_ALIGN_BYTES // torch.tensor([], dtype=dtype).element_size())
    offsets, total = [], 0
    for k in sizes:
        offsets.append(total)
        total += -(-int(k) // align) * align
    buf = torch.full((max(total, 1),), fill, dtype=dtype, device=device)
    return [buf[o:o + int(k)] for o, k in zip(offsets, sizes)]


def allocate_state(weights: Sequence[torch.Tensor], level: str = "O2", flat: bool = True) -> dict:
    """Zero-initialized low-precision optimizer state for a list of weights
    (O2: FP16 weights; O3: FP16 master weights). Returns a dict of tensor
    lists and meta arrays on the weights' device. With flat=True each role
    lives in one allocation (see flat_views)."""
    if level not in ("O2", "O3"):
        raise ValueError("level must be 'O2' or 'O3'")
    dev = weights[0].device if len(weights) else torch.device("cpu")
    n = len(weights)
    sizes = [w.numel() for w in weights]

    def zeros(dtype):
        if flat:
            return flat_views(sizes, dtype, dev)
        return [torch.zeros(k, dtype=dtype, device=dev) for k in sizes]

    st = {"exp_avg": zeros(torch.uint8), "exp_avg_meta": new_meta(n, dev),
          "exp_avg_sq": zeros(torch.float16)}
    if level == "O3":
        st["weight_fp8"] = zeros(torch.uint8)
        st["weight_fp8_meta"] = new_meta(n, dev)
    return st


def state_bytes_per_param(level: str = "O2") -> dict:
    """Bytes per parameter of each tensor class in a layout (optimizer
    states, weight, master, gradient), from the dtypes this library uses."""
    u8 = torch.tensor([], dtype=torch.uint8).element_size()
    f16 = torch.tensor([], dtype=torch.float16).element_size()
    d = {"optimizer_states": u8 + f16, "grad": u8}
    if level == "O2":
        d.update(weight=f16, master=0)
    elif level == "O3":
        d.update(weight=u8, master=f16)
    else:
        raise ValueError(level)
    return d
