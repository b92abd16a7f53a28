"""Compile the CPU oracle (test infrastructure) into oracle/libmoe_oracle.so with g++."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmoe_oracle.so")


def build(verbose: bool = False, sanitize: bool = False, out: str | None = None, src: str | None = None) -> str:
    src = src or os.path.join(HERE, "moe_oracle.cpp")
    target = out or LIB
    tmp = target + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-fno-fast-math", "-Wall", "-Wextra"]
    if sanitize:
        cmd += ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    cmd += ["-I", HERE, "-o", tmp, src]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    print(build(verbose=True))
