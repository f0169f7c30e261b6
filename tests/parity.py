"""Parity harness: the HIP path (through the C ABI) against the CPU oracle.

Both sides start from the same initial state and receive the same binary32
gradients every step; each evolves its own state (independent trajectories).
Gradient codes, gradient meta (amax, scale, scale_inv) are compared bit for
bit every step. For the optimizer outputs (first-moment codes, second moment,
weight / master, FP8 weight copy) the bar is: at least 99.99% of the values
identical and every other value within one unit in the last place of its
format (adjacent codes of the same sign; +-0 next to the smallest
subnormal). Their meta records must agree to within one binary32 ulp.
"""
from __future__ import annotations

import sys
import time
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

import bit_adamw_optimizer_amd as M
import oracle as O
from bit_adamw_optimizer_amd import workloads as W


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def _ordinal(bits: np.ndarray, sign_bit: int) -> np.ndarray:
    b = bits.astype(np.int64)
    mag = b & ((1 << sign_bit) - 1)
    return np.where((b >> sign_bit) & 1, -mag, mag)


def ulp_dist(a: np.ndarray, b: np.ndarray, kind: str) -> np.ndarray:
    if kind == "fp8":
        return np.abs(_ordinal(a, 7) - _ordinal(b, 7))
    if kind == "f16":
        return np.abs(_ordinal(a.view(np.uint16), 15) - _ordinal(b.view(np.uint16), 15))
    if kind == "f32":
        return np.abs(_ordinal(a.view(np.uint32), 31) - _ordinal(b.view(np.uint32), 31))
    raise ValueError(kind)


@dataclass
class Stats:
    total: int = 0
    identical: int = 0
    max_ulp: int = 0
    worst: list = field(default_factory=list)

    def add(self, gpu: np.ndarray, ref: np.ndarray, kind: str, where: str) -> None:
        same = gpu == ref
        self.total += gpu.size
        self.identical += int(same.sum())
        if not same.all():
            d = ulp_dist(gpu, ref, kind)
            m = int(d.max())
            if m > self.max_ulp:
                self.max_ulp = m
            i = int(np.argmax(d))
            self.worst.append((where, i, int(gpu.ravel()[i]), int(ref.ravel()[i]), m))

    @property
    def frac(self) -> float:
        return self.identical / self.total if self.total else 1.0

    def ok(self) -> bool:
        return self.frac >= 0.9999 and self.max_ulp <= 1


def u32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


class GpuState:
    """Device state of one workload, driven through the C ABI."""

    def __init__(self, w: W.Workload, device, adam: bool = False, delayed: bool = False,
                 scaled_v: bool = False, flat: bool = False, fused: bool = False):
        self.w = w
        self.device = device
        self.fused = fused  # gradient quantize fused with pass 1 (AdamW or Adam)
        self.adam = adam  # Adam (coupled L2) instead of AdamW
        self.delayed = delayed  # one-pass delayed-scaling ablation (O2 AdamW)
        self.scaled_v = scaled_v  # scaled-FP16-v ablation (O2 AdamW)
        # FP16 weight (O2) or master (O3); flat=True puts every role in one
        # allocation, as the benchmark does
        out = M.flat_views(w.numel, torch.float16, device) if flat else None
        self.weights = W.init_weights(w, device, out=out)
        st = M.allocate_state(self.weights, w.level)
        self.exp_avg = st["exp_avg"]
        self.exp_avg_meta = st["exp_avg_meta"]
        self.exp_avg_sq = st["exp_avg_sq"]
        self.weight_fp8 = st.get("weight_fp8")
        self.weight_fp8_meta = st.get("weight_fp8_meta")
        self.exp_avg_sq_meta = M.new_meta(w.n, device) if scaled_v else None
        if flat:
            self.grad_q = M.flat_views(w.numel, torch.uint8, device)
            self.grad_f32 = M.flat_views(w.numel, torch.float32, device)
        else:
            self.grad_q = [torch.empty(k, dtype=torch.uint8, device=device) for k in w.numel]
            self.grad_f32 = [torch.empty(k, dtype=torch.float32, device=device) for k in w.numel]
        self.grad_meta = M.new_meta(w.n, device)
        # marshalled once, as an optimizer would
        self.tl_g32 = M.TensorList(self.grad_f32, "f32", "grad_f32")
        self.tl_gq = M.TensorList(self.grad_q, "u8", "grad_q")
        self.tl_m = M.TensorList(self.exp_avg, "u8", "exp_avg")
        self.tl_v = M.TensorList(self.exp_avg_sq, "f16", "exp_avg_sq")
        self.tl_w = M.TensorList(self.weights, "f16", "weight")
        self.tl_w8 = M.TensorList(self.weight_fp8, "u8", "weight_fp8") if self.weight_fp8 else None

    def fill_grads(self, step: int) -> None:
        for t in range(self.w.n):
            W.grad_tensor(self.w, t, step, self.device, out=self.grad_f32[t])

    def step(self, step: int) -> None:
        w = self.w
        M.amax(self.tl_g32, self.grad_meta)
        if self.fused:
            assert not (self.delayed or self.scaled_v)
            if w.level == "O2":
                M.quantize_adamw_o2_step(self.tl_g32, w.grad_fmt, self.grad_meta, self.tl_gq, self.tl_m,
                                         self.exp_avg_meta, self.tl_v, self.tl_w, step=step, adam=self.adam,
                                         **w.hparams())
            else:
                M.quantize_adamw_o3_step(self.tl_g32, w.grad_fmt, self.grad_meta, self.tl_gq, self.tl_m,
                                         self.exp_avg_meta, self.tl_v, self.tl_w, self.tl_w8,
                                         self.weight_fp8_meta, step=step, adam=self.adam, **w.hparams())
            return
        M.quantize_fp8(self.tl_g32, w.grad_fmt, self.grad_meta, self.tl_gq)
        if w.level == "O2" and self.scaled_v:
            M.adamw_o2_step_scaled_v(self.tl_gq, w.grad_fmt, self.grad_meta, self.tl_m,
                                     self.exp_avg_meta, self.tl_v, self.exp_avg_sq_meta, self.tl_w,
                                     step=step, **w.hparams())
        elif w.level == "O2" and self.delayed:
            M.adamw_o2_step_delayed(self.tl_gq, w.grad_fmt, self.grad_meta, self.tl_m,
                                    self.exp_avg_meta, self.tl_v, self.tl_w, step=step, **w.hparams())
        elif w.level == "O2":
            fn = M.adam_o2_step if self.adam else M.adamw_o2_step
            fn(self.tl_gq, w.grad_fmt, self.grad_meta, self.tl_m, self.exp_avg_meta,
               self.tl_v, self.tl_w, step=step, **w.hparams())
        else:
            fn = M.adam_o3_step if self.adam else M.adamw_o3_step
            fn(self.tl_gq, w.grad_fmt, self.grad_meta, self.tl_m, self.exp_avg_meta,
               self.tl_v, self.tl_w, self.tl_w8, self.weight_fp8_meta, step=step, **w.hparams())


def host(t: torch.Tensor) -> np.ndarray:
    x = t.detach().cpu().numpy()
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    return x


def run_parity(w: W.Workload, steps: int, verify=None, threads: int = 16, device="cuda",
               adam: bool = False, delayed: bool = False, scaled_v: bool = False,
               flat: bool = False, fused: bool = False):
    """Runs 'steps' steps on the GPU and on the oracle (for the tensors in
    'verify', default all) and returns a dict of Stats per output. adam=True
    runs the Adam (coupled L2) entry points instead of AdamW."""
    verify = list(range(w.n)) if verify is None else list(verify)
    t0 = time.time()
    gs = GpuState(w, device, adam=adam, delayed=delayed, scaled_v=scaled_v, flat=flat, fused=fused)
    torch.cuda.synchronize()
    ost = {t: O.TensorState(host(gs.weights[t]), w.level, adam=adam, delayed=delayed,
                            scaled_v=scaled_v) for t in verify}
    stats = {k: Stats() for k in ("m", "v", "w", "w8", "m_meta", "v_meta", "w8_meta")}
    pool = ThreadPoolExecutor(max_workers=threads)
    hp = w.hparams()
    for s in range(1, steps + 1):
        gs.fill_grads(s)
        gs.step(s)
        torch.cuda.synchronize()
        g_host = {t: host(gs.grad_f32[t]) for t in verify}

        def ref(t):
            return O.step_tensor(ost[t], g_host[t], w.grad_fmt, s, **hp)

        refs = dict(zip(verify, pool.map(ref, verify)))
        gmeta = gs.grad_meta.cpu().numpy()
        mmeta = gs.exp_avg_meta.cpu().numpy()
        w8meta = gs.weight_fp8_meta.cpu().numpy() if w.level == "O3" else None
        vmeta = gs.exp_avg_sq_meta.cpu().numpy() if scaled_v else None
        for t in verify:
            qg, gm = refs[t]
            # gradient codes and meta: bit-exact (identical binary32 inputs)
            gq = host(gs.grad_q[t])
            if not np.array_equal(gq, qg):
                bad = np.nonzero(gq != qg)[0]
                raise AssertionError("grad codes differ: step %d tensor %d (%s) first at %d: "
                                     "gpu %#x oracle %#x (of %d)"
                                     % (s, t, w.names[t], bad[0], gq[bad[0]], qg[bad[0]], bad.size))
            if not np.array_equal(u32(gmeta[t, :3]), u32(gm[:3])):
                raise AssertionError("grad meta differs: step %d tensor %d: gpu %s oracle %s"
                                     % (s, t, gmeta[t, :3], gm[:3]))
            o = ost[t]
            where = "step %d tensor %d %s" % (s, t, w.names[t])
            stats["m"].add(host(gs.exp_avg[t]), o.m, "fp8", where)
            stats["v"].add(host(gs.exp_avg_sq[t]), o.v, "f16", where)
            stats["w"].add(host(gs.weights[t]), o.w, "f16", where)
            stats["m_meta"].add(u32(mmeta[t, :3]), u32(o.m_meta[:3]), "f32", where)
            if scaled_v:
                stats["v_meta"].add(u32(vmeta[t, :3]), u32(o.v_meta[:3]), "f32", where)
            if w.level == "O3":
                stats["w8"].add(host(gs.weight_fp8[t]), o.w8, "fp8", where)
                stats["w8_meta"].add(u32(w8meta[t, :3]), u32(o.w8_meta[:3]), "f32", where)
        log("  step %d: m %.6f v %.6f w %.6f identical (%.1fs)"
            % (s, stats["m"].frac, stats["v"].frac, stats["w"].frac, time.time() - t0))
    pool.shutdown()
    return stats, gs, ost


def assert_bar(stats) -> None:
    for k, st in stats.items():
        if st.total == 0:
            continue
        assert st.ok(), "%s: %.6f identical, max %d ulp, worst %s" % (k, st.frac, st.max_ulp,
                                                                      st.worst[:5])
