"""The C ABI driven from plain C on the GPU (tests/c_abi_gpu.c, built by
__graft_entry__.build()): device memory and a stream from the HIP runtime,
no Python or PyTorch in the process. Every output bit pattern it prints is
compared with the oracle on the same inputs: the one-element worked example
(O2 and O3, one step) and a three-element O3 example over two steps."""
import os
import subprocess

import numpy as np
import pytest

import oracle as O
from tests.build_c_clients import BIN
from tests.parity import log, u32

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)


def _oracle(level, w0, grads):
    st = O.TensorState(np.array(w0, np.uint16), level)
    for t, g in enumerate(grads, 1):
        qg, gm = O.step_tensor(st, np.array(g, np.float32), O.E4M3, t, **HP)
    out = {"meta0": u32(gm[:3]).tolist(), "meta1": u32(st.m_meta[:3]).tolist(),
           "q": [int(c) for c in qg], "m": [int(c) for c in st.m], "v": [int(c) for c in st.v],
           "w": [int(c) for c in st.w]}
    if level == "O3":
        out["meta2"] = u32(st.w8_meta[:3]).tolist()
        out["w8"] = [int(c) for c in st.w8]
    return out


def _parse(line):
    name, *fields = line.split()
    rec = {}
    for f in fields:
        k, v = f.split("=")
        if k.startswith("meta"):
            rec[k] = [int(x, 16) for x in v.split(",")]
        else:
            width = 4 if k in ("v", "w") else 2
            rec[k] = [int(v[i:i + width], 16) for i in range(0, len(v), width)]
    return name, rec


def test_plain_c_client_matches_the_oracle():
    assert os.path.exists(BIN), "the C client is not built; run __graft_entry__.build()"
    log("running " + BIN)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stdout.splitlines() if l and not l.startswith("c abi gpu ok")]
    assert r.stdout.rstrip().endswith("c abi gpu ok")
    got = dict(_parse(l) for l in lines)
    cases = {"one_o2": ("O2", [0x251F], [[1e-3]]), "one_o3": ("O3", [0x251F], [[1e-3]]),
             "three_o3": ("O3", [0x3800, 0xA51F, 0x0000], [[0.5, 1e-3, 0.0], [-0.25, 2e-3, 0.0]])}
    for name, (level, w0, grads) in cases.items():
        ref = _oracle(level, w0, grads)
        for k, v in ref.items():
            assert got[name][k] == v, (name, k, got[name][k], v)
    # the hand-computed one-element example: w 0.0189972, v underflows, m at 448
    assert got["one_o2"]["w"] == [0x24DD] and got["one_o2"]["v"] == [0] and got["one_o2"]["m"] == [0x7E]
