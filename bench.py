#!/usr/bin/env python3
"""Benchmark of the FP8 AdamW hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
per-tensor amax of the binary32 gradients, their saturating FP8 quantize,
then the low-precision AdamW step (O2: two passes + meta finalize; O3: three
passes + finalize), all through the C ABI of libmsamp.so. By default the
quantize runs in the same pass as the step's pass 1
(msamp_quantize_adamw_o2_step / _o3_step: 21 bytes per parameter for O2
instead of 22); --separate-quantize runs msamp_quantize_fp8 and the step as
two calls. Inputs (weights,
states and two sets of binary32 gradients, alternated between steps) are
resident in HBM before the timed region starts.

Default workload: the Llama-2-7B parameter list (291 tensors, 6,738,415,616
parameters) in the O2 layout with E4M3 gradients.

Prints one JSON line: params updated per second over the whole path
(`value`), the achieved algorithmic HBM bandwidth, the roofline entry of the
dominant kernel (measured with HIP events on the launch stream during the
timed region) and the CPU oracle timed on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, 8 TB/s

# algorithmic bytes per parameter
GRAD_AMAX_BYTES = 4          # read f32
GRAD_QUANTIZE_BYTES = 4 + 1  # read f32, write FP8
PASS1_BYTES = 1 + 1          # read grad FP8, exp_avg FP8
PASS2_BYTES = 6 + 5          # read g, m, v, w; write m, v, w
PASS3_BYTES = 2 + 1          # read master FP16, write FP8 copy
QUANTIZE_PASS1_BYTES = 4 + 1 + 1  # read f32 grad, exp_avg FP8; write grad FP8


def kernel_source_hash() -> str:
    """Hash of the device code's sources (kernels and codec; not the host
    ABI layer) with comments and whitespace removed, to tell whether stored
    counter profiles still apply to the code."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_adamw_optimizer_amd", "csrc")
    for name in ("codec.hpp", "device.hpp", "kernels.hpp", "kernels.hip"):
        with open(os.path.join(csrc, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(name.encode() + b"\0" + text.encode())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200,
                   help="timed steps (default 200: about 5 s of GPU work on the 7B list)")
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="llama2_7b",
                   help="llama2_7b (default), llama2_13b, gpt2_small, single_1m, stress")
    p.add_argument("--optimizer", default="adamw", choices=("adamw", "adam", "adamw-delayed", "adamw-scaled-v"),
                   help="adamw (decoupled decay, default), adam (coupled L2), or the O2-only "
                        "ablations adamw-delayed (one-pass delayed scaling) and adamw-scaled-v "
                        "(per-tensor-scaled FP16 second moment)")
    p.add_argument("--separate-quantize", action="store_true",
                   help="run the gradient quantize and the AdamW step as two calls (the default "
                        "fuses the quantize into pass 1 of the AdamW or Adam step; the ablations "
                        "always run the two calls)")
    p.add_argument("--pad-gib", type=int, default=0, metavar="GIB",
                   help="allocate (and keep) this many GiB of device memory before the workload's "
                        "buffers, to move them to other physical memory (the update pass's rate "
                        "depends on where its buffers land)")
    p.add_argument("--shard", type=int, default=1,
                   help="keep 1/N of every tensor (one data-parallel rank's share)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-threads", type=int, default=16)
    p.add_argument("--graph", action="store_true",
                   help="capture amax + the quantizing device-constants step in a HIP graph per "
                        "gradient buffer and replay it (AdamW / Adam only)")
    p.add_argument("--breakdown-steps", type=int, default=3,
                   help="extra steps after the timed region in which every kernel is timed")
    p.add_argument("--no-profile", action="store_true",
                   help="do not bracket kernels with HIP events")
    p.add_argument("--calibrate-copy", type=float, default=0.0, metavar="GIB",
                   help="only run a device-to-device copy of this many GiB (counter calibration)")
    p.add_argument("--summarize-sq", nargs=2, metavar=("TRACE_DIR", "SQ_DIR"),
                   help="write the profiles/ summary of a rocprofv3 run of SQ instruction counters "
                        "(no GPU needed)")
    p.add_argument("--summarize-profiles", nargs=5, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR",
                                                            "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                   help="write profiles/ summaries from rocprofv3 CSV output directories "
                        "(no GPU needed)")
    return p.parse_args()


def calibrate_copy(gib: float) -> None:
    import torch

    n = int(gib * (1 << 30)) // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4}))


class State:
    """Device state of a workload plus two resident binary32 gradient sets."""

    def __init__(self, w, device, adam: bool = False, delayed: bool = False,
                 scaled_v: bool = False, fused: bool = False):
        import torch

        import bit_adamw_optimizer_amd as M
        from bit_adamw_optimizer_amd import workloads as W

        self.w = w
        self.adam = adam
        self.delayed = delayed
        self.scaled_v = scaled_v
        self.fused = fused  # gradient quantize fused with pass 1 of the AdamW or Adam step
        self.exp_avg_sq_meta = M.new_meta(w.n, device) if scaled_v else None
        # every role lives in one allocation (views per tensor). Lists of many
        # tensors without per-tensor factors draw their inputs over the whole
        # allocation in a few launches instead of a few per tensor.
        flat_gen = w.n > 1000 and w.factor is None
        self.weights = M.flat_views(w.numel, torch.float16, device)
        if flat_gen:
            W.init_weights_flat(w, self.weights, device)
        else:
            W.init_weights(w, device, out=self.weights)
        st = M.allocate_state(self.weights, w.level, flat=True)
        self.exp_avg_meta = st["exp_avg_meta"]
        self.weight_fp8_meta = st.get("weight_fp8_meta")
        self.tl_m = M.TensorList(st["exp_avg"], "u8", "exp_avg")
        self.tl_v = M.TensorList(st["exp_avg_sq"], "f16", "exp_avg_sq")
        self.tl_w = M.TensorList(self.weights, "f16", "weight")
        self.tl_w8 = M.TensorList(st["weight_fp8"], "u8", "weight_fp8") if w.level == "O3" else None
        self.grad_q = M.TensorList(M.flat_views(w.numel, torch.uint8, device), "u8", "grad_q")
        self.grad_meta = M.new_meta(w.n, device)
        self.grad_sets = []
        for s in (1, 2):
            g = M.flat_views(w.numel, torch.float32, device)
            if flat_gen:
                W.grads_flat(w, s, g, device)
            else:
                for t in range(w.n):
                    W.grad_tensor(w, t, s, device, out=g[t])
            self.grad_sets.append(M.TensorList(g, "f32", "grad_f32"))
        torch.cuda.synchronize()

    def enable_graphs(self, total_steps: int) -> None:
        """Switch to the device-constants step: the constants of every step
        are computed up front into a device table; each step copies its row
        into the record the kernels read and replays the graph captured for
        its gradient buffer (captured after two eager steps have built the
        cached tables)."""
        import torch

        import bit_adamw_optimizer_amd as M

        w = self.w
        dev = self.exp_avg_meta.device
        self.consts = torch.empty(9, dtype=torch.float32, device=dev)
        self.table = torch.stack([M.step_constants(step=t, adam=self.adam, **w.hparams())
                                  for t in range(1, total_steps + 1)]).to(dev)
        self.graphs = None
        self.use_graphs = True

    def _graph_body(self, g32) -> None:
        import bit_adamw_optimizer_amd as M

        w = self.w
        M.amax(g32, self.grad_meta)
        if self.fused and w.level == "O2":
            M.quantize_adamw_o2_step_devconst(g32, w.grad_fmt, self.grad_meta, self.grad_q, self.tl_m,
                                              self.exp_avg_meta, self.tl_v, self.tl_w, self.consts,
                                              adam=self.adam)
            return
        if self.fused:
            M.quantize_adamw_o3_step_devconst(g32, w.grad_fmt, self.grad_meta, self.grad_q, self.tl_m,
                                              self.exp_avg_meta, self.tl_v, self.tl_w, self.tl_w8,
                                              self.weight_fp8_meta, self.consts, adam=self.adam)
            return
        M.quantize_fp8(g32, w.grad_fmt, self.grad_meta, self.grad_q)
        if w.level == "O2":
            M.adamw_o2_step_devconst(self.grad_q, w.grad_fmt, self.grad_meta, self.tl_m,
                                     self.exp_avg_meta, self.tl_v, self.tl_w, self.consts, adam=self.adam)
        else:
            M.adamw_o3_step_devconst(self.grad_q, w.grad_fmt, self.grad_meta, self.tl_m,
                                     self.exp_avg_meta, self.tl_v, self.tl_w, self.tl_w8,
                                     self.weight_fp8_meta, self.consts, adam=self.adam)

    def step(self, step: int) -> None:
        import bit_adamw_optimizer_amd as M

        w = self.w
        g32 = self.grad_sets[(step - 1) % 2]
        if getattr(self, "use_graphs", False):
            import torch

            self.consts.copy_(self.table[step - 1])
            if step <= 2:
                self._graph_body(g32)  # eager: builds the cached tables of both buffers
                if step == 2:
                    self.graphs = []
                    for gs in self.grad_sets:
                        gr = torch.cuda.CUDAGraph()
                        with torch.cuda.graph(gr):
                            self._graph_body(gs)
                        self.graphs.append(gr)
            else:
                self.graphs[(step - 1) % 2].replay()
            return
        M.amax(g32, self.grad_meta)
        if self.fused:
            if w.level == "O2":
                M.quantize_adamw_o2_step(g32, w.grad_fmt, self.grad_meta, self.grad_q, self.tl_m,
                                         self.exp_avg_meta, self.tl_v, self.tl_w, step=step, adam=self.adam,
                                         **w.hparams())
            else:
                M.quantize_adamw_o3_step(g32, w.grad_fmt, self.grad_meta, self.grad_q, self.tl_m,
                                         self.exp_avg_meta, self.tl_v, self.tl_w, self.tl_w8,
                                         self.weight_fp8_meta, step=step, adam=self.adam, **w.hparams())
            return
        M.quantize_fp8(g32, w.grad_fmt, self.grad_meta, self.grad_q)
        if w.level == "O2" and self.scaled_v:
            M.adamw_o2_step_scaled_v(self.grad_q, w.grad_fmt, self.grad_meta, self.tl_m,
                                     self.exp_avg_meta, self.tl_v, self.exp_avg_sq_meta, self.tl_w,
                                     step=step, **w.hparams())
        elif w.level == "O2":
            fn = M.adam_o2_step if self.adam else M.adamw_o2_step
            if self.delayed:
                fn = M.adamw_o2_step_delayed
            fn(self.grad_q, w.grad_fmt, self.grad_meta, self.tl_m, self.exp_avg_meta,
               self.tl_v, self.tl_w, step=step, **w.hparams())
        else:
            fn = M.adam_o3_step if self.adam else M.adamw_o3_step
            fn(self.grad_q, w.grad_fmt, self.grad_meta, self.tl_m, self.exp_avg_meta,
               self.tl_v, self.tl_w, self.tl_w8, self.weight_fp8_meta, step=step, **w.hparams())


def storage_of(views):
    """The one allocation behind a list of views (flat_views)."""
    import torch

    base = views[0]
    return torch.empty(0, dtype=base.dtype, device=base.device).set_(base.untyped_storage())


def numerics_report(st) -> dict:
    """Value statistics of the stored state after the timed steps: fractions
    of the FP16 second moment that are +-0 or subnormal (binary16 underflows
    (1-b2)*g^2 at small gradient scales) and of first-moment codes at 0 and
    at +-max (0x7E). Counted over each role's one allocation in a few
    launches; the alignment padding between tensors holds zeros that no
    kernel writes, and is subtracted."""
    import torch

    n = sum(int(x.numel()) for x in st.tl_v.tensors)
    v = storage_of(st.tl_v.tensors).view(torch.int16)
    m = storage_of(st.tl_m.tensors)
    zero = sub = m_zero = m_max = 0
    piece = 1 << 28  # bounded temporaries
    for a in range(0, v.numel(), piece):
        vmag = v[a:a + piece] & 0x7FFF
        zero += int(torch.count_nonzero(vmag == 0))
        sub += int(torch.count_nonzero((vmag > 0) & (vmag < 0x0400)))
    for a in range(0, m.numel(), piece):
        mmag = m[a:a + piece] & 0x7F
        m_zero += int(torch.count_nonzero(mmag == 0))
        m_max += int(torch.count_nonzero(mmag == 0x7E))
    zero -= v.numel() - n
    m_zero -= m.numel() - n
    return {"v_zero_frac": zero / n, "v_subnormal_frac": sub / n,
            "m_code_zero_frac": m_zero / n, "m_code_max_frac": m_max / n}


def cpu_baseline(w, device, threads: int) -> dict:
    """The oracle on a bounded sample of the workload, one whole tensor per
    work item (the per-tensor amax couples every element of a tensor, so a
    tensor is the oracle's unit of work). For the Llama lists the sample is
    chosen so that the threads get equal work: 'threads' MLP tensors and
    twice as many attention projections (one MLP tensor and two projections
    per thread, largest first), about 8 s on 16 host threads. Other lists
    take their largest tensors, at most two per thread."""
    import numpy as np
    import torch

    import oracle as O
    from bit_adamw_optimizer_amd import workloads as W

    nthreads = max(1, threads)
    mlp = [t for t, nm in enumerate(w.names) if nm.endswith(("gate_proj", "up_proj", "down_proj"))]
    attn = [t for t, nm in enumerate(w.names) if nm.endswith(("q_proj", "k_proj", "v_proj", "o_proj"))]
    if len(mlp) >= nthreads and len(attn) >= 2 * nthreads:
        idx = mlp[:nthreads] + attn[:2 * nthreads]
        how = "%d MLP tensors and %d attention projections, one MLP tensor and two projections per thread" \
              % (nthreads, 2 * nthreads)
    else:
        idx = sorted(range(w.n), key=lambda t: -w.numel[t])[:2 * nthreads]
        how = "the %d largest tensors" % len(idx)
    idx.sort(key=lambda t: -w.numel[t])  # largest first onto the thread pool
    sub = w.subset(idx)
    weights = [x.view(torch.int16).cpu().numpy().view(np.uint16) for x in W.init_weights(sub, device)]
    grads = [W.grad_tensor(sub, t, 1, device).cpu().numpy() for t in range(sub.n)]
    states = [O.TensorState(x, w.level) for x in weights]
    # one thread on the last (smallest) tensor of the sample (fresh state, same inputs)
    one = O.TensorState(weights[-1].copy(), w.level)
    t0 = time.perf_counter()
    O.step_list([one], grads[-1:], w.grad_fmt, 1, threads=1, **w.hparams())
    dt1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.step_list(states, grads, w.grad_fmt, 1, threads=nthreads, **w.hparams())
    dt = time.perf_counter() - t0
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": sub.params / dt, "unit": "params/s", "cores": nthreads, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": "%d tensors of the list (%s), %d params, one step each (grad amax + quantize + %s "
                      "step), on a pool of %d threads" % (sub.n, how, sub.params, w.level, nthreads),
            "threads": nthreads, "cpu_model": cpu_model, "host_cpus": os.cpu_count(),
            "one_thread": {"value": sub.numel[-1] / dt1, "unit": "params/s",
                           "sample": "%s (%d params)" % (sub.names[-1], sub.numel[-1])},
            "full_step_seconds_extrapolated": round(w.params / (sub.params / dt), 2)}


def _kind_of(name: str):
    """(kernel kind, algorithmic bytes per parameter) of one of the library's
    kernels from its rocprofv3 name (template arguments included), or None."""
    if "msamp::" not in name:
        return None
    m = re.search(r"\b(k_\w+)(?:<([^>]*)>)?\(", name)
    if not m:
        return None
    fn, targs = m.group(1), [a.strip() for a in (m.group(2) or "").split(",") if a.strip()]
    if fn == "k_amax":
        return "amax", GRAD_AMAX_BYTES
    if fn == "k_quantize":
        return "quantize_fp8", GRAD_QUANTIZE_BYTES
    if fn == "k_step_pass1":  # <grad format, coupled>
        coupled = len(targs) > 1 and targs[1] == "true"
        return "step_pass1", PASS1_BYTES + (2 if coupled else 0)
    if fn == "k_step_pass2":  # <grad format, O3, coupled[, delayed]>
        if len(targs) > 3 and targs[3] == "true":
            return "o2_delayed", PASS2_BYTES
        return ("o3_pass2" if len(targs) > 1 and targs[1] == "true" else "o2_pass2"), PASS2_BYTES
    if fn == "k_o3_pass3":
        return "o3_pass3", PASS3_BYTES
    if fn == "k_quantize_pass1":  # <grad format, coupled>
        coupled = len(targs) > 1 and targs[1] == "true"
        return "quantize_pass1", QUANTIZE_PASS1_BYTES + (2 if coupled else 0)
    if fn == "k_stream_probe":  # <copy>: measurement streams (bytes are not per parameter)
        return ("copy_probe" if targs and targs[0] == "true" else "read_probe"), 0
    if fn == "k_rmw_probe":
        return "rmw_probe", PASS2_BYTES
    if fn == "k_qp1_probe":
        return "qp1_probe", QUANTIZE_PASS1_BYTES
    if fn == "k_scaled_v_pass1":  # also reads the FP16 second moment
        return "step_pass1", PASS1_BYTES + 2
    if fn == "k_scaled_v_pass2":
        return "o2_pass2", PASS2_BYTES
    return None


def summarize_profiles(dirs, workload: str) -> None:
    """Summaries of rocprofv3 runs for profiles/: the kernel-trace statistics
    of the library's kernels, and per-launch HBM bytes from FETCH_SIZE and
    WRITE_SIZE, each scaled by what the same counter reads for a plain copy of
    a known size (--calibrate-copy)."""
    import csv
    import glob

    trace_dir, fetch_dir, write_dir, cfetch_dir, cwrite_dir = dirs

    def rel(d):
        return os.path.relpath(os.path.abspath(d), ROOT)

    # the profiled program's arguments, as rocprofv3 echoed them into the
    # run's own log
    def bench_args(d):
        for f in glob.glob(os.path.join(d, "*.log")):
            for line in open(f, errors="replace"):
                m = re.search(r"\[rocprofv3\] 'python3 \S*bench\.py([^']*)'", line)
                if m:
                    return m.group(1)
        raise AssertionError("no rocprofv3 command line in %s" % d)

    def one(pattern):
        files = glob.glob(os.path.join(pattern, "**", "*.csv"), recursive=True)
        return files

    stats = [f for f in one(trace_dir) if f.endswith("_kernel_stats.csv")]
    rows = list(csv.DictReader(open(stats[0]))) if stats else []

    def counters(d, name):
        files = [f for f in one(d) if f.endswith("_counter_collection.csv")]
        agg = {}
        for r in csv.DictReader(open(files[0])):
            if r["Counter_Name"] != name:
                continue
            agg.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return agg

    def copy_kib(d, name):
        agg = counters(d, name)
        vals = [v for k, vs in agg.items() if "copyBuffer" in k or "copy" in k.lower() for v in vs]
        return max(vals)  # the one big calibration copy

    # each profiled run keeps its own output (the bench line) in <dir>/bench.log
    def source_hash(d):
        for f in glob.glob(os.path.join(d, "*.log")):
            for line in open(f, errors="replace"):
                if line.startswith("{") and "kernel_source_hash" in line:
                    return json.loads(line)["kernel_source_hash"]
        return None

    copy_bytes = None
    for f in glob.glob(os.path.join(cfetch_dir, "*.log")):
        for line in open(f, errors="replace"):
            if line.startswith("{") and "calibrate_copy_bytes_read" in line:
                copy_bytes = json.loads(line)["calibrate_copy_bytes_read"]
    assert copy_bytes, "no calibration copy output found"
    ffac = copy_bytes / (copy_kib(cfetch_dir, "FETCH_SIZE") * 1024.0)
    wfac = copy_bytes / (copy_kib(cwrite_dir, "WRITE_SIZE") * 1024.0)
    fetch = counters(fetch_dir, "FETCH_SIZE")
    write = counters(write_dir, "WRITE_SIZE")
    h = source_hash(fetch_dir)
    assert h is not None and h == source_hash(write_dir), "counter runs of different kernel sources"

    from bit_adamw_optimizer_amd import workloads as W
    w = W.make(workload)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    lines = ["# HBM traffic per launch, %s (%d params), from rocprofv3 counters" % (workload, w.params), "",
             "Commands (run from the repository root; R=$PWD; cd /tmp first):",
             "  rocprofv3 --pmc FETCH_SIZE -f csv -d $R/%s -o fetch -- python3 $R/bench.py%s "
             "> $R/%s/bench.log 2>&1" % (rel(fetch_dir), bench_args(fetch_dir), rel(fetch_dir)),
             "  rocprofv3 --pmc WRITE_SIZE -f csv -d $R/%s -o write -- python3 $R/bench.py%s "
             "> $R/%s/bench.log 2>&1" % (rel(write_dir), bench_args(write_dir), rel(write_dir)),
             "  rocprofv3 --pmc FETCH_SIZE -f csv -d $R/%s -o cfetch -- python3 $R/bench.py%s "
             "> $R/%s/bench.log 2>&1" % (rel(cfetch_dir), bench_args(cfetch_dir), rel(cfetch_dir)),
             "  rocprofv3 --pmc WRITE_SIZE -f csv -d $R/%s -o cwrite -- python3 $R/bench.py%s "
             "> $R/%s/bench.log 2>&1" % (rel(cwrite_dir), bench_args(cwrite_dir), rel(cwrite_dir)),
             "  (each run's directory is made first with mkdir -p)",
             "  python bench.py --summarize-profiles %s --workload %s"
             % (" ".join(rel(d) for d in dirs), workload),
             "",
             "Calibration: a %d-byte device copy reads FETCH_SIZE x %.4f and WRITE_SIZE x %.4f bytes;"
             " these factors scale the counters below." % (copy_bytes, ffac, wfac),
             "Kernel sources hash: %s" % h, "",
             "| kernel | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes/launch (scaled) | algorithmic bytes | ratio |",
             "|---|---|---|---|---|---|---|"]
    out = {}
    for name in sorted(set(fetch) | set(write)):
        kb = _kind_of(name)
        if kb is None:
            continue
        kind, bpp = kb
        if not bpp:
            continue  # measurement streams (run only when profiling is on)
        f = sum(fetch.get(name, [0])) / max(1, len(fetch.get(name, [0])))
        wr = sum(write.get(name, [0])) / max(1, len(write.get(name, [0])))
        hbm = f * 1024 * ffac + wr * 1024 * wfac
        alg = bpp * w.params
        out[kind] = {"fetch_kib": f, "write_kib": wr, "hbm_bytes_per_launch": hbm, "algorithmic_bytes": alg}
        lines.append("| %s | %d | %.1f | %.1f | %.4g | %.4g | %.4f |"
                     % (kind, len(fetch.get(name, [])), f, wr, hbm, alg, hbm / alg))
    with open(os.path.join(ROOT, "profiles", "path_kernels_%s_hbm_counters.md" % workload), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    for kind, d in out.items():
        d.update({"kernel": kind, "workload": workload, "kernel_source_hash": h,
                  "fetch_factor": ffac, "write_factor": wfac})
        with open(os.path.join(ROOT, "profiles", "pmc_%s_%s.json" % (kind, workload)), "w") as fh:
            json.dump(d, fh, indent=1)
    if rows:
        tl = ["# rocprofv3 kernel-trace statistics, %s (%d params)" % (workload, w.params), "",
              "Command (run from the repository root; R=$PWD; cd /tmp first):",
              "  rocprofv3 --kernel-trace --stats -f csv -d $R/%s -o %s -- python3 $R/bench.py%s "
              "> $R/%s/bench.log 2>&1"
              % (rel(trace_dir), os.path.basename(stats[0])[:-len("_kernel_stats.csv")],
                 bench_args(trace_dir), rel(trace_dir)), "",
              "Kernel sources hash: %s" % source_hash(trace_dir), "",
              "| kernel | calls | average ms | min ms | max ms | algorithmic GB/s (avg) |", "|---|---|---|---|---|---|"]
        for r in rows:
            if "msamp::" not in r["Name"]:
                continue
            kb = _kind_of(r["Name"])
            avg = float(r["AverageNs"]) * 1e-6
            gbps = kb[1] * w.params / (avg * 1e-3) / 1e9 if kb and kb[1] else float("nan")
            m = re.search(r"\b(k_\w+)", r["Name"])
            short = kb[0] if kb else (m.group(1) if m else r["Name"][:40])
            tl.append("| %s | %s | %.4f | %.4f | %.4f | %.1f |" % (short, r["Calls"], avg,
                      float(r["MinNs"]) * 1e-6, float(r["MaxNs"]) * 1e-6, gbps))
        with open(os.path.join(ROOT, "profiles", "path_kernels_%s_kernel_trace.md" % workload), "w") as fh:
            fh.write("\n".join(tl) + "\n")
    print("wrote profiles for %s" % workload)


SQ_COUNTERS = "SQ_INSTS_VALU SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR SQ_WAVES"


def summarize_sq(dirs, workload: str) -> None:
    """profiles/ summary of a rocprofv3 run of SQ instruction counters: per
    kernel, wave-level VALU and vector-memory instructions per element (x 64
    lanes / parameters), and the VALU issue time at one wave64 VALU
    instruction per compute unit per cycle (256 CUs at 2.4 GHz) beside the
    kernel's time from the kernel-trace summary of the same sources."""
    import csv
    import glob

    trace_dir, sq_dir = dirs
    from bit_adamw_optimizer_amd import workloads as W
    w = W.make(workload)

    def rel(d):
        return os.path.relpath(os.path.abspath(d), ROOT)

    files = glob.glob(os.path.join(sq_dir, "**", "*counter_collection.csv"), recursive=True)
    agg = {}
    for r in csv.DictReader(open(files[0])):
        kb = _kind_of(r["Kernel_Name"])
        if kb is None or not kb[1]:
            continue
        agg.setdefault(kb[0], {}).setdefault(r["Counter_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
        agg[kb[0]][r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    stats = glob.glob(os.path.join(trace_dir, "**", "*_kernel_stats.csv"), recursive=True)
    kms = {}
    for r in csv.DictReader(open(stats[0])):
        kb = _kind_of(r["Name"])
        if kb:
            kms[kb[0]] = float(r["AverageNs"]) * 1e-6
    args = None
    for f in glob.glob(os.path.join(sq_dir, "*.log")):
        for line in open(f, errors="replace"):
            m = re.search(r"\[rocprofv3\] 'python3 \S*bench\.py([^']*)'", line)
            if m:
                args = m.group(1)
    h = None
    for f in glob.glob(os.path.join(sq_dir, "*.log")):
        for line in open(f, errors="replace"):
            if line.startswith("{") and "kernel_source_hash" in line:
                h = json.loads(line)["kernel_source_hash"]
    lines = ["# VALU and memory-instruction counters per launch, %s (%d params)" % (workload, w.params), "",
             "Command (run from the repository root; R=$PWD; cd /tmp first):",
             "  rocprofv3 --pmc %s -f csv -d $R/%s -o sq -- python3 $R/bench.py%s > $R/%s/bench.log 2>&1"
             % (SQ_COUNTERS, rel(sq_dir), args or "", rel(sq_dir)),
             "  python bench.py --summarize-sq %s %s --workload %s" % (rel(trace_dir), rel(sq_dir), workload), "",
             "Kernel sources hash: %s" % h, "",
             "Per element: wave-level instruction counts x 64 lanes / parameters. VALU issue time: one wave64",
             "VALU instruction per CU per cycle (4 SIMDs, 4 cycles each), 256 CUs at 2.4 GHz; kernel time from",
             "the kernel-trace summary (%s)." % rel(trace_dir), "",
             "| kernel | launches | VALU instr / element | VMEM read instr / element | VMEM write instr / element "
             "| VALU issue ms | kernel ms | VALU issue / kernel time |",
             "|---|---|---|---|---|---|---|---|"]
    for kind in sorted(agg):
        c = agg[kind]

        def mean(name):
            v = list(c.get(name, {}).values())
            return sum(v) / len(v) if v else float("nan")
        valu, rd, wr = mean("SQ_INSTS_VALU"), mean("SQ_INSTS_VMEM_RD"), mean("SQ_INSTS_VMEM_WR")
        issue_ms = valu / (256 * 2.4e9) * 1e3
        kt = kms.get(kind, float("nan"))
        lines.append("| %s | %d | %.2f | %.4f | %.4f | %.2f | %.2f | %.2f |"
                     % (kind, len(c.get("SQ_INSTS_VALU", {})), valu * 64 / w.params, rd * 64 / w.params,
                        wr * 64 / w.params, issue_ms, kt, issue_ms / kt))
    with open(os.path.join(ROOT, "profiles", "path_kernels_%s_sq_counters.md" % workload), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("wrote the SQ summary for %s" % workload)


def traffic_from_profiles(kernel: str, workload: str, params: int):
    """HBM bytes per launch from committed counter runs, when they were taken
    on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "pmc_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def main() -> int:
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.workload)
        return 0
    if args.summarize_sq:
        summarize_sq(args.summarize_sq, args.workload)
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2
    import torch

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return 0

    import bit_adamw_optimizer_amd as M
    from bit_adamw_optimizer_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    M.lib()
    w = W.make(args.workload, shard=args.shard)
    print("bench: %s, %s, %d tensors, %d params; setting up" % (w.name, w.level, w.n, w.params),
          file=sys.stderr, flush=True)
    adam = args.optimizer == "adam"
    delayed = args.optimizer == "adamw-delayed"
    scaled_v = args.optimizer == "adamw-scaled-v"
    if (delayed or scaled_v) and w.level != "O2":
        print("the %s ablation exists for the O2 layout only" % args.optimizer, file=sys.stderr)
        return 2
    fused = not (args.separate_quantize or delayed or scaled_v)
    # held until the run ends, so the workload's buffers stay where it pushed them
    pad = torch.empty(args.pad_gib << 30, dtype=torch.uint8, device=device) if args.pad_gib > 0 else None
    st = State(w, device, adam=adam, delayed=delayed, scaled_v=scaled_v, fused=fused)
    if args.graph:
        if delayed or scaled_v:
            print("--graph covers the AdamW and Adam steps only", file=sys.stderr)
            return 2
        if args.warmup < 2:
            print("--graph needs --warmup >= 2 (the graphs are captured at step 2)", file=sys.stderr)
            return 2
        st.enable_graphs(args.warmup + args.steps + args.breakdown_steps)

    step = 0
    for _ in range(args.warmup):
        step += 1
        st.step(step)
    torch.cuda.synchronize()

    # A HIP event record costs a few microseconds of launch-queue time: hidden
    # under the 7B list's kernels, but a large share of a small list's step.
    # So the timed region records them around the dominant kernel only, and
    # the other kernels are timed in a few extra steps after it.
    dom = ("o2_delayed" if delayed else "o2_pass2") if w.level == "O2" else "o3_pass2"
    if not args.no_profile:
        M.profile_select([dom])
        M.profile_enable(True)
    # one event per step boundary on the launch stream (for the median step
    # time; an event between steps costs nothing measurable at these sizes)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record()
    for i in range(args.steps):
        step += 1
        st.step(step)
        marks[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    kernels = {}
    if not args.no_profile:
        M.profile_enable(False)
        n, ms = M.profile_read(dom)
        if n:
            kernels[dom] = {"launches": n, "avg_ms": ms / n, "timed_region": True}
        # breakdown of every kernel, in extra (untimed) steps
        M.profile_select(None)
        M.profile_enable(True)
        for _ in range(args.breakdown_steps):
            step += 1
            st.step(step)
        torch.cuda.synchronize()
        M.profile_enable(False)
        for k in M.KERNELS:
            n, ms = M.profile_read(k)
            if n and k not in kernels:
                kernels[k] = {"launches": n, "avg_ms": ms / n}

    # the update pass's traffic without its arithmetic, on the same buffers
    # and launch geometry: what the memory system gives that traffic alone
    probe_ms = None
    if not args.no_profile:
        M.profile_enable(True)
        for _ in range(5):
            M.rmw_probe(st.grad_q, st.tl_m, st.tl_v, st.tl_w)
        torch.cuda.synchronize()
        M.profile_enable(False)
        n_p, ms_p = M.profile_read("rmw_probe")
        probe_ms = ms_p / n_p if n_p else None
    # the fused quantize + pass 1's traffic without arithmetic, on the same
    # buffers (it overwrites the gradient codes; the timed steps are done)
    qp1_ms = None
    if not args.no_profile and fused and not adam:
        M.profile_enable(True)
        for _ in range(5):
            M.quantize_pass1_probe(st.grad_sets[0], st.grad_q, st.tl_m, st.tl_v, st.tl_w)
        torch.cuda.synchronize()
        M.profile_enable(False)
        n_q, ms_q = M.profile_read("qp1_probe")
        qp1_ms = ms_q / n_q if n_q else None
    # plain read and copy streams over the run's own binary32 gradient
    # buffers (4 bytes per parameter each; the timed steps are done, so the
    # second set may be overwritten)
    streams = {}
    if not args.no_profile:
        g0, g1 = (storage_of(gs.tensors) for gs in st.grad_sets)
        nb = (g0.numel() * 4) // 16 * 16
        M.profile_enable(True)
        for _ in range(5):
            M.stream_probe(g0)
        for _ in range(5):
            M.stream_probe(g0, g1)
        torch.cuda.synchronize()
        M.profile_enable(False)
        for kind, moved in (("read_probe", nb), ("copy_probe", 2 * nb)):
            n_p, ms_p = M.profile_read(kind)
            if n_p:
                streams[kind] = {"bytes": moved, "ms": round(ms_p / n_p, 4),
                                 "GB/s": round(moved / (ms_p / n_p * 1e-3) / 1e9, 1)}

    ms_per_step = (t1 - t0) * 1000.0 / args.steps
    P = w.params
    # Adam's pass 1 also reads the FP16 weight for its L2 term
    # (and so does the scaled-v ablation's, for its amax(v1))
    pass1_bytes = PASS1_BYTES + (2 if adam or scaled_v else 0)
    step_bytes = (0 if delayed else pass1_bytes) + PASS2_BYTES + (PASS3_BYTES if w.level == "O3" else 0)
    qp1_bytes = QUANTIZE_PASS1_BYTES + (2 if adam else 0)
    if fused:
        # the quantize writes the codes and pass 1 takes them from registers:
        # one launch reads the f32 gradient and the first moment (and, for
        # Adam, the weight), and writes the codes
        step_bytes = qp1_bytes + PASS2_BYTES + (PASS3_BYTES if w.level == "O3" else 0)
        path_bytes = GRAD_AMAX_BYTES + step_bytes
    else:
        path_bytes = GRAD_AMAX_BYTES + GRAD_QUANTIZE_BYTES + step_bytes
    gbps = path_bytes * P / (ms_per_step * 1e-3) / 1e9

    per_kernel_bytes = {"amax": GRAD_AMAX_BYTES, "quantize_fp8": GRAD_QUANTIZE_BYTES,
                        "step_pass1": pass1_bytes, "o2_pass2": PASS2_BYTES, "o3_pass2": PASS2_BYTES,
                        "quantize_pass1": qp1_bytes,
                        "o3_pass3": PASS3_BYTES, "o2_delayed": PASS2_BYTES}
    breakdown = {}
    for k, d in kernels.items():
        e = {"avg_ms": round(d["avg_ms"], 4), "launches": d["launches"],
             "measured": "timed region" if d.get("timed_region") else "extra steps"}
        if k in per_kernel_bytes:
            e["GB/s"] = round(per_kernel_bytes[k] * P / (d["avg_ms"] * 1e-3) / 1e9, 1)
        breakdown[k] = e
    roofline = None
    if dom in kernels:
        achieved = per_kernel_bytes[dom] * P / (kernels[dom]["avg_ms"] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": traffic_from_profiles(dom, w.name, P),
                    "algorithmic_bytes_per_launch": per_kernel_bytes[dom] * P}
        if probe_ms:
            # a reference, not a bound: the update pass, whose arithmetic
            # spaces out its accesses, can run faster than its traffic alone
            rate = PASS2_BYTES * P / (probe_ms * 1e-3) / 1e9
            roofline["same_buffers_probe"] = {
                "GB/s": round(rate, 1), "frac": round(achieved / rate, 4),
                "probe": "msamp_rmw_probe: the update pass's loads and stores (read 6, write 5 B/p) "
                         "without arithmetic, on the same buffers and launch geometry, %.4f ms" % probe_ms}
        # what the memory system gives plain traffic shapes on this run's
        # buffers: a pure read, a copy, and the two step passes' read/write mixes
        ceil = {}
        if "read_probe" in streams:
            ceil["read"] = dict(streams["read_probe"], probe="msamp_stream_probe READ over the f32 gradients")
        if "copy_probe" in streams:
            ceil["copy"] = dict(streams["copy_probe"], probe="msamp_stream_probe COPY between the two f32 "
                                                            "gradient sets (bytes = read + written)")
        if probe_ms:
            ceil["update_pass_mix"] = {"bytes": PASS2_BYTES * P, "ms": round(probe_ms, 4),
                                       "GB/s": round(PASS2_BYTES * P / (probe_ms * 1e-3) / 1e9, 1),
                                       "probe": "msamp_rmw_probe (read 6, write 5 B/p)"}
        if qp1_ms:
            ceil["quantize_pass1_mix"] = {"bytes": QUANTIZE_PASS1_BYTES * P, "ms": round(qp1_ms, 4),
                                          "GB/s": round(QUANTIZE_PASS1_BYTES * P / (qp1_ms * 1e-3) / 1e9, 1),
                                          "probe": "msamp_quantize_pass1_probe (read 5, write 1 B/p)"}
        roofline["traffic_probes"] = ceil
    opt_ms = sum(kernels[k]["avg_ms"] for k in ("step_pass1", "quantize_pass1", dom, "o3_pass3", "finalize")
                 if k in kernels)
    result = {
        "metric": "params updated/sec and achieved HBM GB/s (% of peak) for O2/O3 FP8 AdamW step",
        "value": P / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(step_ms[len(step_ms) // 2] if len(step_ms) % 2
                                    else 0.5 * (step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2]), 4),
        "ms_per_step_min": round(step_ms[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s: %s FP8 %s step, %d tensors, %d params, %s grads "
                               "(amax + quantize + step per iteration%s%s)"
                               % (w.name, w.level, {"adam": "Adam", "adamw": "AdamW",
                                                    "adamw-delayed": "AdamW one-pass delayed-scaling "
                                                                     "ablation",
                                                    "adamw-scaled-v": "AdamW scaled-FP16-v "
                                                                      "ablation"}[args.optimizer],
                                  w.n, P,
                                  "E4M3" if w.grad_fmt == 0 else "E5M2",
                                  ", HIP-graph replay" if args.graph else "",
                                  ", quantize fused with pass 1" if fused else ""),
                   "level": w.level, "optimizer": args.optimizer, "tensors": w.n, "params": P,
                   "graph": bool(args.graph), "fused_quantize": fused, "pad_gib": args.pad_gib},
        "hbm_gbps": round(gbps, 1),
        "pct_of_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "bytes_per_param": path_bytes,
        "optimizer_step": {"ms": round(opt_ms, 4) if kernels else None,
                           "params_per_s": P / (opt_ms * 1e-3) if kernels else None,
                           "GB/s": round(step_bytes * P / (opt_ms * 1e-3) / 1e9, 1) if kernels else None,
                           "bytes_per_param": step_bytes,
                           "includes_grad_quantize": fused},
        "kernels": breakdown,
        "roofline": roofline,
        "kernel_source_hash": kernel_source_hash(),
    }
    result["numerics"] = {k: round(v, 6) for k, v in numerics_report(st).items()}
    if not args.no_cpu_baseline:
        print("bench: timing the oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, device, args.cpu_threads)
        result["cpu_baseline"]["gpu_over_oracle"] = round(result["value"] / result["cpu_baseline"]["value"], 1)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
