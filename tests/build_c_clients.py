"""Builds the plain-C GPU client of the C ABI (tests/c_abi_gpu.c) into
tests/_bin/, linked against the in-tree libmsamp.so with a relative run
path. Called by __graft_entry__.build(); the GPU test only runs the binary."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BIN = os.path.join(HERE, "_bin", "c_abi_gpu")


def build() -> str:
    os.makedirs(os.path.dirname(BIN), exist_ok=True)
    lib = os.path.join(ROOT, "bit_adamw_optimizer_amd", "_lib")
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           "-isystem", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "c_abi_gpu.c"), "-o", BIN,
           "-L", lib, "-lmsamp", "-Wl,-rpath,$ORIGIN/../../bit_adamw_optimizer_amd/_lib",
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    subprocess.run(cmd, check=True)
    return BIN


if __name__ == "__main__":
    print(build())
