"""Seeded synthetic inputs for the AdamW-step workloads.

This module holds shapes and input generators only (none of the step's
arithmetic). Both the HIP path and the CPU oracle are fed from the same
tensors made here: a test generates them once (on the GPU when there is
one), copies them to the host for the oracle, and hands identical values to
both sides.

Workloads (parameter lists of real model shapes; values are random):
  single_1m   one 1024x1024 tensor, O2, E4M3 grads ~ N(0, 1e-3)
  gpt2_small  GPT-2 small (124,439,808 params, 148 tensors), O2, E4M3 grads
  llama2_7b   Llama-2-7B (6,738,415,616 params, 291 tensors), O2, E4M3 grads
              ~ N(0, 1e-3) x f_t, f_t log-uniform in [0.1, 10] per tensor
  llama2_13b  Llama-2-13B (13,015,864,320 params, 363 tensors), O3, E4M3
  stress      20,000 tensors of log-uniform size in [64, 8192] plus 64 of
              8192x8192, O2, E5M2 grads from a Student-t (nu = 3) scaled by
              1e-3, with 1% of the tensors all-zero
Test lists: tiny_llama / tiny_llama_o3 (reduced Llama shapes), tiny_stress
(600 small + 2 larger tensors), tiny_small / tiny_small_o3 (1,122 tensors
of at most 4,096 elements, with the edge sizes, between larger ones).
Weights (or O3 master weights) are FP16 of N(0, 0.02). Optimizer states
start at zero.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

E4M3 = 0
E5M2 = 1


@dataclass
class Workload:
    name: str
    level: str                      # "O2" or "O3"
    grad_fmt: int                   # E4M3 / E5M2
    steps: int                      # steps the parity runs take
    names: List[str]
    numel: List[int]
    grad_kind: str = "normal"       # "normal" or "student_t3"
    grad_sigma: float = 1e-3
    factor: Optional[np.ndarray] = None       # per-tensor grad factor
    zero_tensors: frozenset = field(default_factory=frozenset)
    lr: float = 1e-3
    betas: tuple = (0.9, 0.999)
    eps: float = 1e-8
    weight_decay: float = 0.01
    seed_base: int = 0

    @property
    def n(self) -> int:
        return len(self.numel)

    @property
    def params(self) -> int:
        return int(sum(self.numel))

    def hparams(self) -> dict:
        return dict(lr=self.lr, betas=self.betas, eps=self.eps, weight_decay=self.weight_decay)

    def subset(self, idx: Sequence[int]) -> "Workload":
        """The same workload restricted to some tensors (same seeds, so the
        values of a kept tensor are unchanged)."""
        w = Workload(self.name + "[subset]", self.level, self.grad_fmt, self.steps,
                     [self.names[i] for i in idx], [self.numel[i] for i in idx], self.grad_kind,
                     self.grad_sigma, None, frozenset(), self.lr, self.betas, self.eps,
                     self.weight_decay, self.seed_base)
        w._index = list(idx)
        if self.factor is not None:
            w.factor = np.asarray([self.factor[i] for i in idx])
        w.zero_tensors = frozenset(k for k, i in enumerate(idx) if i in self.zero_tensors)
        return w

    def tensor_seed(self, t: int, step: int) -> int:
        orig = getattr(self, "_index", None)
        ti = orig[t] if orig is not None else t
        return (self.seed_base * 1_000_003 + ti) * 1009 + step


# ------------------------------------------------------------------ shapes ---

def gpt2_small_shapes():
    d, ff, vocab, ctx, layers = 768, 3072, 50257, 1024, 12
    names, numel = ["wte", "wpe"], [vocab * d, ctx * d]
    for l in range(layers):
        for nm, k in (("ln_1.weight", d), ("ln_1.bias", d), ("attn.c_attn.weight", d * 3 * d),
                      ("attn.c_attn.bias", 3 * d), ("attn.c_proj.weight", d * d),
                      ("attn.c_proj.bias", d), ("ln_2.weight", d), ("ln_2.bias", d),
                      ("mlp.c_fc.weight", d * ff), ("mlp.c_fc.bias", ff),
                      ("mlp.c_proj.weight", ff * d), ("mlp.c_proj.bias", d)):
            names.append("h.%d.%s" % (l, nm))
            numel.append(k)
    names += ["ln_f.weight", "ln_f.bias"]
    numel += [d, d]
    return names, numel


def llama_shapes(hidden: int, ffn: int, layers: int, vocab: int):
    names, numel = ["embed_tokens"], [vocab * hidden]
    for l in range(layers):
        for nm, k in (("q_proj", hidden * hidden), ("k_proj", hidden * hidden),
                      ("v_proj", hidden * hidden), ("o_proj", hidden * hidden),
                      ("gate_proj", hidden * ffn), ("up_proj", hidden * ffn),
                      ("down_proj", ffn * hidden), ("input_layernorm", hidden),
                      ("post_attention_layernorm", hidden)):
            names.append("layers.%d.%s" % (l, nm))
            numel.append(k)
    names += ["norm", "lm_head"]
    numel += [hidden, vocab * hidden]
    return names, numel


def stress_shapes(n_small: int = 20000, n_big: int = 64, big: int = 8192 * 8192, seed: int = 0):
    rng = np.random.Generator(np.random.PCG64(seed))
    small = np.rint(np.exp(rng.uniform(math.log(64), math.log(8192), n_small))).astype(np.int64)
    names = ["small.%d" % i for i in range(n_small)] + ["big.%d" % i for i in range(n_big)]
    numel = [int(x) for x in small] + [big] * n_big
    n = len(numel)
    zero = rng.choice(n, size=max(1, round(0.01 * n)), replace=False)
    return names, numel, frozenset(int(i) for i in zero)


def small_shapes(seed: int = 2):
    """Eight runs of small tensors (at most 4,096 elements: the edge sizes
    around 1, 16, 1,024, 2,048 and 3,072 elements and 120 random ones from 0
    to 4,096 each), separated by larger tensors, plus a lone small tensor
    between two larger ones: 1,122 small tensors in all."""
    rng = np.random.Generator(np.random.PCG64(seed))
    edges = [0, 1, 3, 4, 5, 15, 16, 17, 1023, 1024, 1025, 2047, 2048, 2049, 3071, 3072, 3073, 4095, 4096, 7]
    seps = [4097, 70001, 5000, 65536, 8191, 131075, 4100, 9999]
    numel = []
    for r in range(8):
        numel += edges + [int(x) for x in rng.integers(0, 4097, 120)]
        numel.append(seps[r])
    numel += [12345, 2000, 77777, 300, 4097]
    names = ["t%d" % i for i in range(len(numel))]
    return names, numel


# ---------------------------------------------------------------- workloads ---

def make(name: str, shard: int = 1) -> Workload:
    """A named workload. shard > 1 keeps 1/shard of every tensor (one data-
    parallel rank's share of a flat per-tensor partition), rounded up to a
    multiple of 16 elements."""
    if name == "single_1m":
        w = Workload(name, "O2", E4M3, 10, ["w"], [1024 * 1024], seed_base=1)
    elif name == "gpt2_small":
        nm, ne = gpt2_small_shapes()
        w = Workload(name, "O2", E4M3, 10, nm, ne, seed_base=2)
    elif name == "llama2_7b":
        nm, ne = llama_shapes(4096, 11008, 32, 32000)
        rng = np.random.Generator(np.random.PCG64(0))
        f = np.exp(rng.uniform(math.log(0.1), math.log(10.0), len(ne)))
        w = Workload(name, "O2", E4M3, 5, nm, ne, factor=f, seed_base=3)
    elif name == "llama2_13b":
        nm, ne = llama_shapes(5120, 13824, 40, 32000)
        w = Workload(name, "O3", E4M3, 3, nm, ne, seed_base=4)
    elif name == "stress":
        nm, ne, zero = stress_shapes()
        w = Workload(name, "O2", E5M2, 10, nm, ne, grad_kind="student_t3", zero_tensors=zero,
                     seed_base=5)
    elif name.startswith("tiny_llama"):
        # reduced Llama shapes for quick parity runs: hidden 256, FFN 688,
        # 2 layers, vocab 1000 (ragged sizes, several chunks per tensor)
        nm, ne = llama_shapes(256, 688, 2, 1000)
        rng = np.random.Generator(np.random.PCG64(0))
        f = np.exp(rng.uniform(math.log(0.1), math.log(10.0), len(ne)))
        level = "O3" if name.endswith("o3") else "O2"
        w = Workload(name, level, E4M3, 10, nm, ne, factor=f, seed_base=6)
    elif name.startswith("tiny_small"):
        nm, ne = small_shapes()
        level = "O3" if name.endswith("o3") else "O2"
        w = Workload(name, level, E5M2 if level == "O2" else E4M3, 3, nm, ne, seed_base=8)
    elif name == "tiny_stress":
        nm, ne, zero = stress_shapes(n_small=600, n_big=2, big=300_001, seed=1)
        w = Workload(name, "O2", E5M2, 10, nm, ne, grad_kind="student_t3", zero_tensors=zero,
                     seed_base=7)
    else:
        raise KeyError(name)
    if shard > 1:
        w.numel = [max(16, -(-(k // shard) // 16) * 16) for k in w.numel]
        w.name += "/shard%d" % shard
    return w


NAMES = ["single_1m", "gpt2_small", "llama2_7b", "llama2_13b", "stress"]


# --------------------------------------------------------------- generators ---

def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def init_weights(w: Workload, device, out: Optional[List[torch.Tensor]] = None) -> List[torch.Tensor]:
    """FP16 weights (O3: master weights) = fp16(0.02 * N(0, 1)), per tensor;
    written into 'out' (a list of FP16 tensors of the right sizes) if given."""
    res = []
    for t, k in enumerate(w.numel):
        x = torch.randn(k, generator=_gen(device, w.tensor_seed(t, 0)), device=device,
                        dtype=torch.float32)
        h = (x * 0.02).to(torch.float16)
        if out is not None:
            out[t].copy_(h)
            res.append(out[t])
        else:
            res.append(h)
    return res


def grad_tensor(w: Workload, t: int, step: int, device, out: Optional[torch.Tensor] = None):
    """The binary32 gradient of tensor t at a 1-based step."""
    k = w.numel[t]
    g = _gen(device, w.tensor_seed(t, step))
    if out is None:
        out = torch.empty(k, dtype=torch.float32, device=device)
    if t in w.zero_tensors:
        out.zero_()
        return out
    if w.grad_kind == "normal":
        torch.randn(k, generator=g, device=device, out=out)
    elif w.grad_kind == "student_t3":
        # t with 3 degrees of freedom: z0 / sqrt((z1^2 + z2^2 + z3^2) / 3)
        torch.randn(k, generator=g, device=device, out=out)
        chi = torch.zeros(k, dtype=torch.float32, device=device)
        tmp = torch.empty(k, dtype=torch.float32, device=device)
        for _ in range(3):
            torch.randn(k, generator=g, device=device, out=tmp)
            chi.addcmul_(tmp, tmp)
        out.div_(torch.sqrt(chi / 3.0))
    else:
        raise ValueError(w.grad_kind)
    scale = w.grad_sigma * (float(w.factor[t]) if w.factor is not None else 1.0)
    out.mul_(scale)
    return out


def _storage_pieces(views: Sequence[torch.Tensor], piece: int):
    """The one allocation behind 'views' (views of one buffer, in order), as
    consecutive slices of at most 'piece' elements."""
    base = views[0]
    buf = torch.empty(0, dtype=base.dtype, device=base.device).set_(base.untyped_storage())
    total = buf.numel()
    return [buf[a:min(total, a + piece)] for a in range(0, total, piece)]


def _flat_seed(w: Workload, role: int, step: int) -> int:
    return ((w.seed_base * 1_000_003 + 999_983) * 1009 + step) * 7 + role


def init_weights_flat(w: Workload, views: Sequence[torch.Tensor], device, piece: int = 1 << 28) -> None:
    """FP16 weights of N(0, 0.02) drawn over the views' one allocation in a
    few launches (one generator per list, not per tensor): the same
    distribution as init_weights, for lists of many small tensors."""
    g = _gen(device, _flat_seed(w, 0, 0))
    for sl in _storage_pieces(views, piece):
        x = torch.randn(sl.numel(), generator=g, device=device, dtype=torch.float32)
        sl.copy_((x * 0.02).to(torch.float16))


def grads_flat(w: Workload, step: int, views: Sequence[torch.Tensor], device, piece: int = 1 << 28) -> None:
    """The binary32 gradients of a step drawn over the views' one allocation
    in a few launches: the distribution of grad_tensor (normal or Student-t
    with 3 degrees of freedom, times grad_sigma), zero on the all-zero
    tensors. For lists without per-tensor factors."""
    assert w.factor is None
    g = _gen(device, _flat_seed(w, 1, step))
    for sl in _storage_pieces(views, piece):
        k = sl.numel()
        torch.randn(k, generator=g, device=device, out=sl)
        if w.grad_kind == "student_t3":
            chi = torch.zeros(k, dtype=torch.float32, device=device)
            tmp = torch.empty(k, dtype=torch.float32, device=device)
            for _ in range(3):
                torch.randn(k, generator=g, device=device, out=tmp)
                chi.addcmul_(tmp, tmp)
            sl.div_(torch.sqrt(chi / 3.0))
            del chi, tmp
        elif w.grad_kind != "normal":
            raise ValueError(w.grad_kind)
        sl.mul_(w.grad_sigma)
    for t in w.zero_tensors:
        views[t].zero_()


def grads(w: Workload, step: int, device) -> List[torch.Tensor]:
    return [grad_tensor(w, t, step, device) for t in range(w.n)]


def bytes_per_param(level: str) -> int:
    """Algorithmic HBM bytes one optimizer step moves per parameter: O2 reads
    g, m (pass 1), then g, m, v, w and writes m, v, w (pass 2); O3 adds the
    FP8 weight copy (read master, write w8)."""
    return {"O2": 2 + 6 + 5, "O3": 2 + 6 + 5 + 3}[level]


GRAD_PRODUCER_BYTES = 4 + 4 + 1  # amax reads f32; quantize reads f32, writes u8
