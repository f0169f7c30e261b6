"""Host logic of bench.py (no GPU): kernel-name parsing of rocprofv3 output,
the comment-insensitive kernel-source hash, the counter summary arithmetic
(calibration factors, bytes per launch) on a synthetic rocprofv3 output, and
the one-GPU rule."""
import json
import os
import shutil
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NS = "void msamp::(anonymous namespace)::"


def test_kernel_names_map_to_kinds_and_bytes():
    args = "(msamp::TensorDesc const*, msamp::ChunkRef const*)"
    cases = {
        "k_amax" + args: ("amax", 4),
        "k_quantize<0>" + args: ("quantize_fp8", 5),
        "k_step_pass1<0, false>" + args: ("step_pass1", 2),
        "k_step_pass1<1, true>" + args: ("step_pass1", 4),
        "k_step_pass2<0, false, false, false>" + args: ("o2_pass2", 11),
        "k_step_pass2<0, true, true, false>" + args: ("o3_pass2", 11),
        "k_step_pass2<1, false, false, true>" + args: ("o2_delayed", 11),
        "k_o3_pass3" + args: ("o3_pass3", 3),
        "k_quantize_pass1<0, false>" + args: ("quantize_pass1", 6),
        "k_quantize_pass1<1, true>" + args: ("quantize_pass1", 8),
        "k_quantize_pass1<0, false, 512>" + args: ("quantize_pass1", 6),
        "k_step_pass2<0, false, false, false, 512>" + args: ("o2_pass2", 11),
        "k_step_pass2<0, true, false, false, 512>" + args: ("o3_pass2", 11),
        "k_o3_pass3<512>" + args: ("o3_pass3", 3),
        "k_rmw_probe<512>" + args: ("rmw_probe", 11),
        "k_rmw_probe" + args: ("rmw_probe", 11),
        "k_scaled_v_pass1<0>" + args: ("step_pass1", 4),
        "k_scaled_v_pass2<0>" + args: ("o2_pass2", 11),
    }
    for name, kind in cases.items():
        assert bench._kind_of(NS + name) == kind, name
    assert bench._kind_of("void at::native::vectorized_elementwise_kernel<8>(int)") is None
    assert bench._kind_of(NS + "k_step_finalize(int)") is None


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    csrc = tmp_path / "bit_adamw_optimizer_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "bit_adamw_optimizer_amd", "csrc"), csrc)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    k = csrc / "kernels.hip"
    text = k.read_text()
    k.write_text("// an added comment line\n" + text.replace("namespace msamp {", "namespace msamp {  /* x */", 1))
    assert bench.kernel_source_hash() == h0
    k.write_text(text.replace("kTile", "kTile ", 1).replace("+= kTile", "+= 2 * kTile", 1))
    assert bench.kernel_source_hash() != h0


def _write_counters(path, rows, counter):
    hdr = ("Correlation_Id,Dispatch_Id,Agent_Id,Queue_Id,Process_Id,Thread_Id,Grid_Size,Kernel_Id,"
           "Kernel_Name,Workgroup_Size,LDS_Block_Size,Scratch_Size,VGPR_Count,Accum_VGPR_Count,"
           "SGPR_Count,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n")
    with open(path, "w") as f:
        f.write(hdr)
        for i, (name, value) in enumerate(rows):
            f.write('%d,%d,"Agent 1",1,1,1,256,1,"%s",256,0,0,4,0,16,"%s",%f,0,1\n'
                    % (i + 1, i + 1, name, counter, value))


def test_counter_summary_arithmetic(tmp_path, monkeypatch):
    """Synthetic rocprofv3 output for the 1M-element workload: the copy
    calibration gives the factors, and each kernel's HBM bytes per launch is
    FETCH_SIZE*1024*factor + WRITE_SIZE*1024*factor."""
    shutil.copytree(os.path.join(ROOT, "bit_adamw_optimizer_amd", "csrc"),
                    tmp_path / "bit_adamw_optimizer_amd" / "csrc")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.kernel_source_hash()
    d = {k: tmp_path / k for k in ("trace", "fetch", "write", "cfetch", "cwrite")}
    for p in d.values():
        p.mkdir()
    line = "W0 simple_timer.cpp:55] [rocprofv3] 'python3 /x/bench.py%s' ::     0.0 sec\n"
    bench_line = json.dumps({"kernel_source_hash": h}) + "\n"
    for k in ("trace", "fetch", "write"):
        (d[k] / "bench.log").write_text(line % " --workload single_1m" + bench_line)
    copy_bytes = 1 << 30
    for k in ("cfetch", "cwrite"):
        (d[k] / "bench.log").write_text(line % " --calibrate-copy 1"
                                        + json.dumps({"calibrate_copy_bytes_read": copy_bytes}) + "\n")
    copy_name = "void at::native::copy_kernel(int)"
    # FETCH_SIZE reads half the copied bytes, WRITE_SIZE all of them
    _write_counters(d["cfetch"] / "c_counter_collection.csv", [(copy_name, copy_bytes / 2048.0)], "FETCH_SIZE")
    _write_counters(d["cwrite"] / "c_counter_collection.csv", [(copy_name, copy_bytes / 1024.0)], "WRITE_SIZE")
    p2 = NS + "k_step_pass2<0, false, false, false>(msamp::TensorDesc const*)"
    n = 1 << 20
    _write_counters(d["fetch"] / "f_counter_collection.csv", [(p2, 3 * n / 1024.0)] * 2, "FETCH_SIZE")
    _write_counters(d["write"] / "w_counter_collection.csv", [(p2, 5 * n / 1024.0)] * 2, "WRITE_SIZE")
    (d["trace"] / "t_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"%s",2,2000,1000.0,100,900,1100,1\n' % p2)
    bench.summarize_profiles([str(d[k]) for k in ("trace", "fetch", "write", "cfetch", "cwrite")], "single_1m")
    rec = json.loads((tmp_path / "profiles" / "pmc_o2_pass2_single_1m.json").read_text())
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["hbm_bytes_per_launch"] == 11 * n == rec["algorithmic_bytes"]
    assert rec["kernel_source_hash"] == h
    md = (tmp_path / "profiles" / "path_kernels_single_1m_kernel_trace.md").read_text()
    assert "--workload single_1m" in md and "| o2_pass2 | 2 | 0.0010 |" in md
    assert bench.traffic_from_profiles("o2_pass2", "single_1m", n) == 11 * n


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
