"""The storage layouts of the oracle and of the library against the figures
the pages print (tests/golden/optimization_levels.txt, each line cited
there): the format of every role per optimization level, the 62.5% O2
optimizer-state saving and the bytes-per-weight example of the Transformer
Engine FP8 discussion."""
import os

import numpy as np
import torch

import bit_adamw_optimizer_amd as M
import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "optimization_levels.txt")
WIDTH = {"FP8": 1, "FP16": 2, "FP32": 4, "none": 0}
TORCH = {"FP8": torch.uint8, "FP16": torch.float16, "FP32": torch.float32}
NUMPY = {"FP8": np.uint8, "FP16": np.uint16}


def _load():
    table, figures = {}, {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = line.split()
        if len(parts) == 6:
            table[parts[0]] = dict(zip(("weight", "master", "weight_grad", "exp_avg", "exp_avg_sq"),
                                       parts[1:]))
        else:
            figures[parts[0]] = float(parts[1])
    return table, figures


def test_fixture_is_complete():
    table, figures = _load()
    assert set(table) == {"FP16_AMP", "NVIDIA_TE", "O1", "O2", "O3"}
    assert set(figures) == {"saving_O2_optimizer_states_percent", "bytes_half_weight_plus_fp32_master",
                            "bytes_fp8_weight_plus_fp32_weight"}


def test_library_state_layout_matches_the_table():
    table, _ = _load()
    w = [torch.zeros(1000, dtype=torch.float16), torch.zeros(17, dtype=torch.float16)]
    for level in ("O2", "O3"):
        row = table[level]
        st = M.allocate_state(w, level)
        assert all(t.dtype == TORCH[row["exp_avg"]] for t in st["exp_avg"]), level
        assert all(t.dtype == TORCH[row["exp_avg_sq"]] for t in st["exp_avg_sq"]), level
        per = M.state_bytes_per_param(level)
        assert per["optimizer_states"] == WIDTH[row["exp_avg"]] + WIDTH[row["exp_avg_sq"]]
        assert per["grad"] == WIDTH[row["weight_grad"]]
        if level == "O3":
            # the FP16 tensor the step updates is the master; the regular
            # weight is the FP8 copy
            assert per["master"] == WIDTH[row["master"]] and per["weight"] == WIDTH[row["weight"]]
            assert all(t.dtype == TORCH[row["weight"]] for t in st["weight_fp8"])
        else:
            assert row["master"] == "none"
            assert per["weight"] == WIDTH[row["weight"]]


def test_oracle_state_layout_matches_the_table():
    table, _ = _load()
    for level in ("O2", "O3"):
        row = table[level]
        st = O.TensorState(np.zeros(33, np.uint16), level)
        assert st.m.dtype == NUMPY[row["exp_avg"]] and st.v.dtype == NUMPY[row["exp_avg_sq"]]
        if level == "O3":
            assert st.w8.dtype == NUMPY[row["weight"]]


def test_printed_savings():
    table, figures = _load()
    full = WIDTH[table["O1"]["exp_avg"]] + WIDTH[table["O1"]["exp_avg_sq"]]
    o2 = WIDTH[table["O2"]["exp_avg"]] + WIDTH[table["O2"]["exp_avg_sq"]]
    assert 100.0 * (1 - o2 / full) == figures["saving_O2_optimizer_states_percent"]
    assert 1 - O.STATE_BYTES_FP8_FP16 / O.STATE_BYTES_FP32_FP32 == 0.625
    assert WIDTH["FP16"] + WIDTH["FP32"] == figures["bytes_half_weight_plus_fp32_master"]
    assert WIDTH["FP8"] + WIDTH["FP32"] == figures["bytes_fp8_weight_plus_fp32_weight"]
