"""Compile tests/c_abi_caller.cpp (a plain C++ caller of the C ABI, test helper) against the
in-tree library: hipcc for the HIP runtime headers, linked to libmoe_plan.so by a relative rpath."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
EXE = os.path.join(HERE, "c_abi_caller")


def build(verbose: bool = False) -> str:
    tmp = EXE + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c_abi_caller.cpp"),
           "-o", tmp, "-L", os.path.join(ROOT, "load_balance_planning_amd"), "-lmoe_plan",
           "-Wl,-rpath,$ORIGIN/../load_balance_planning_amd"]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, EXE)
    return EXE
