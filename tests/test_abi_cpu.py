"""Host-side checks of the C ABI and the binding (no GPU needed): the library
loads and exports every function include/msamp.h declares, argument
validation rejects bad calls before anything is enqueued, and the host
bookkeeping (state layout, workload shapes) matches the definitions."""
import ctypes
import os
import re

import pytest
import torch

import bit_adamw_optimizer_amd as M
from bit_adamw_optimizer_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "msamp.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msamp_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert "msamp_adamw_o2_step" in names and "msamp_adamw_o3_step" in names
    assert "msamp_amax" in names and "msamp_quantize_fp8" in names
    lib = M.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert lib.msamp_abi_version() == 3


def test_library_is_built_for_gfx950():
    data = open(M.library_path(), "rb").read()
    assert b"gfx950" in data


def _vp(*xs):
    return (ctypes.c_void_p * len(xs))(*xs)


def _i64(*xs):
    return (ctypes.c_int64 * len(xs))(*xs)


_HP = M._HParams  # the binding's msamp_adamw_hparams
GOOD_HP = _HP(1e-3, 0.9, 0.999, 1e-8, 0.01)


def _o2(n=1, numel=None, grad=None, fmt=0, gmeta=0x10000, m=None, mmeta=0x20000, v=None, w=None,
        hp=GOOD_HP, step=1):
    numel = numel if numel is not None else _i64(32)
    grad = grad if grad is not None else _vp(0x100000)
    m = m if m is not None else _vp(0x200000)
    v = v if v is not None else _vp(0x300000)
    w = w if w is not None else _vp(0x400000)
    st = M.lib().msamp_adamw_o2_step(n, numel, grad, fmt, ctypes.c_void_p(gmeta), m,
                                     ctypes.c_void_p(mmeta), v, w,
                                     ctypes.byref(hp) if hp is not None else None, step, None)
    return st, M.lib().msamp_last_error().decode()


def test_step_validation_rejects_before_launch():
    # every call below fails validation, so no device pointer is touched
    assert _o2(n=-1)[0] == 1
    assert _o2(numel=_i64(-5))[0] == 1
    assert _o2(fmt=2)[0] == 1
    assert _o2(step=0)[0] == 1
    assert _o2(hp=None)[0] == 1
    assert _o2(hp=_HP(1e-3, 1.0, 0.999, 1e-8, 0.01))[0] == 1
    assert _o2(hp=_HP(1e-3, 0.9, -0.1, 1e-8, 0.01))[0] == 1
    assert _o2(hp=_HP(1e-3, 0.9, 0.999, 0.0, 0.01))[0] == 1
    assert _o2(hp=_HP(float("inf"), 0.9, 0.999, 1e-8, 0.01))[0] == 1
    assert _o2(hp=_HP(1e-3, 0.9, 0.999, 1e-8, -1.0))[0] == 1
    st, msg = _o2(grad=_vp(0))
    assert st == 1 and "grad[0]" in msg
    st, msg = _o2(m=_vp(0x200001))
    assert st == 2 and "exp_avg[0]" in msg
    st, msg = _o2(w=_vp(0x400008))
    assert st == 2 and "weight[0]" in msg
    assert _o2(gmeta=0)[0] == 1
    assert _o2(mmeta=0x20004)[0] == 2
    # n == 0 is a no-op; NULL pointers are allowed for empty tensors
    assert _o2(n=0, numel=None)[0] == 0


def test_other_entry_points_validate():
    L = M.lib()
    assert L.msamp_amax(-1, None, None, None, None) == 1
    assert L.msamp_amax(1, _vp(0x1003), _i64(4), ctypes.c_void_p(0x1000), None) == 2
    assert L.msamp_quantize_fp8(1, _vp(0x1000), _i64(4), 3, ctypes.c_void_p(0x2000), _vp(0x3000), None) == 1
    assert L.msamp_dequantize_fp8(1, _vp(0), _i64(4), 0, ctypes.c_void_p(0x2000), _vp(0x3000), None) == 1
    assert L.msamp_codec_probe(9, ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), 4, None) == 1
    assert L.msamp_codec_probe(0, ctypes.c_void_p(0x1001), ctypes.c_void_p(0x2000), 4, None) == 2
    assert L.msamp_quantize_fp8_prescaled(1, _vp(0x1000), _i64(4), 0, ctypes.c_void_p(0x2000), 0,
                                          _vp(0x3000), None) == 1
    assert L.msamp_kernel_name(4) == b"o2_pass2"
    assert L.msamp_kernel_name(99) == b""


def test_binding_checks_tensor_arguments():
    with pytest.raises(ValueError):
        M.TensorList([torch.zeros(4)], "f32")  # not on a GPU
    with pytest.raises(TypeError):
        M.TensorList([torch.zeros(4, dtype=torch.float16)], "f32")


def test_state_layout_saves_62_5_percent():
    """MS-AMP "Optimization Level" page, O2: first moment FP8 + second moment
    FP16 against FP32+FP32 states, a saving of 5/8 (the page's 62.5%)."""
    w = [torch.zeros(1000, dtype=torch.float16), torch.zeros(24, dtype=torch.float16)]
    st = M.allocate_state(w, "O2")
    nbytes = sum(t.numel() * t.element_size() for t in st["exp_avg"] + st["exp_avg_sq"])
    assert nbytes == 3 * 1024
    assert 1 - nbytes / (8 * 1024) == 0.625
    assert M.state_bytes_per_param("O2")["optimizer_states"] == 3
    o3 = M.state_bytes_per_param("O3")
    assert o3["weight"] == 1 and o3["master"] == 2 and o3["grad"] == 1
    st3 = M.allocate_state(w, "O3")
    assert st3["weight_fp8"][0].dtype == torch.uint8
    assert st3["exp_avg_meta"].shape == (2, 4) and st3["exp_avg_meta"][0].tolist() == [0, 1, 1, 0]


def test_workload_shapes():
    expect = {"single_1m": (1, 1_048_576), "gpt2_small": (148, 124_439_808),
              "llama2_7b": (291, 6_738_415_616), "llama2_13b": (363, 13_015_864_320)}
    for name, (n, p) in expect.items():
        w = W.make(name)
        assert (w.n, w.params) == (n, p), name
    s = W.make("stress")
    assert s.n == 20_064 and len(s.zero_tensors) == 201
    assert 4.3e9 < s.params < 4.36e9
    small = [k for k in s.numel if k <= 8192]
    assert len(small) == 20_000 and min(small) >= 64
    assert W.make("llama2_7b").level == "O2" and W.make("llama2_13b").level == "O3"
    assert W.make("stress").grad_fmt == W.E5M2
    sh = W.make("llama2_7b", shard=8)
    assert all(k % 16 == 0 for k in sh.numel) and abs(sh.params * 8 / 6_738_415_616 - 1) < 1e-3


def test_grad_generators_are_seeded():
    w = W.make("tiny_stress")
    a = W.grad_tensor(w, 3, 2, "cpu")
    b = W.grad_tensor(w, 3, 2, "cpu")
    c = W.grad_tensor(w, 3, 3, "cpu")
    assert torch.equal(a, b) and not torch.equal(a, c)
    z = next(iter(w.zero_tensors))
    assert (W.grad_tensor(w, z, 1, "cpu") == 0).all()


def test_header_is_plain_c_and_cxx_and_a_c_program_links(tmp_path):
    """include/msamp.h compiles as C11 and as C++17, and a C program using
    only the header links against the library and gets validation errors
    back without a GPU."""
    import subprocess

    inc = os.path.join(ROOT, "include")
    src = os.path.join(ROOT, "tests", "c_abi_smoke.c")
    hdr_cpp = tmp_path / "h.cpp"
    hdr_cpp.write_text('#include "msamp.h"\nint main() { return msamp_abi_version() != MSAMP_ABI_VERSION; }\n')
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Werror", "-fsyntax-only", "-I", inc, str(hdr_cpp)],
                   check=True)
    libdir = os.path.dirname(M.library_path())
    exe = tmp_path / "c_abi_smoke"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", inc, src,
                    "-o", str(exe), "-L", libdir, "-lmsamp", "-Wl,-rpath," + libdir,
                    "-Wl,-rpath-link,/opt/rocm/lib"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stderr)
    assert "c abi ok" in r.stdout


def test_step_constants_match_the_oracle_bit_for_bit():
    """msamp_step_constants_compute (host only) against the oracle's own
    binary64-then-binary32 constants, AdamW and Adam, over many steps and
    hyperparameters."""
    import numpy as np

    import oracle as O

    for hp in (dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01),
               dict(lr=5e-3, betas=(0.8, 0.99), eps=1e-7, weight_decay=0.2)):
        for step in (1, 2, 3, 10, 100, 1000, 12345, 10**6):
            for adam in (False, True):
                got = M.step_constants(step=step, adam=adam, **hp).numpy()
                ref = np.asarray(O.adamw_constants(step, **hp), np.float32)
                if adam:
                    ref[7] = 1.0  # no decoupled decay for Adam
                assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (hp, step, adam, got, ref)
    with pytest.raises(M.MsampError):
        M.step_constants(step=0)


def test_binding_declares_the_signature_of_every_header_function():
    """Every function of include/msamp.h has explicit ctypes argument and
    return types in the binding, with as many arguments as the header
    declares (an undeclared ctypes call would pass 64-bit sizes and doubles
    through C's default promotions)."""
    text = open(os.path.join(ROOT, "include", "msamp.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lib = M.lib()
    for name, args in re.findall(r"\b(msamp_[a-z0-9_]+)\s*\(([^;{]*?)\)\s*;", text):
        fn = getattr(lib, name)
        assert fn.argtypes is not None, name
        n_decl = 0 if args.strip() in ("", "void") else args.count(",") + 1
        assert len(fn.argtypes) == n_decl, (name, len(fn.argtypes), n_decl)
        assert fn.restype is not None, name


def test_noalloc_step_rejects_lists_beyond_its_static_tables():
    """The allocation-free step checks its table size before any device work:
    one tensor of 2^35 elements needs 524,288 chunks (4 MiB of chunk map
    plus the descriptor and amax sections), one byte past the limit."""
    L = M.lib()
    limit = 4 << 20

    def call(numel):
        st = L.msamp_adamw_o2_step_noalloc(1, _i64(numel), _vp(0x100000), 0, ctypes.c_void_p(0x10000),
                                           _vp(0x200000), ctypes.c_void_p(0x20000), _vp(0x300000),
                                           _vp(0x400000), ctypes.byref(GOOD_HP), 1, None)
        return st, L.msamp_last_error().decode()

    st, msg = call(1 << 35)
    need = 256 + 256 + 8 * ((1 << 35) // 65536)
    assert need > limit
    assert st == 1 and "at most %d" % limit in msg and str(need) in msg, msg
    # validation still comes first
    st, msg = L.msamp_adamw_o2_step_noalloc(1, _i64(32), _vp(0), 0, ctypes.c_void_p(0x10000), _vp(0x200000),
                                            ctypes.c_void_p(0x20000), _vp(0x300000), _vp(0x400000),
                                            ctypes.byref(GOOD_HP), 1, None), L.msamp_last_error().decode()
    assert st == 1 and "grad[0]" in msg
