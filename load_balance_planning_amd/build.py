"""Compile the HIP kernels and the C ABI into load_balance_planning_amd/libmoe_plan.so (gfx950)."""
import glob
import hashlib
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe_plan.so")
ARCH = os.environ.get("MOE_PLAN_ARCH", "gfx950")


HASH = LIB + ".srchash"


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def source_hash() -> str:
    """SHA-256 of every source the library is built from (kernels, headers, the public header)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(HERE, "csrc", "*"))) + [os.path.join(ROOT, "include", "moe_plan.h")]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def up_to_date() -> bool:
    """The built library exists and was built from the sources now in the tree."""
    if not os.path.exists(LIB) or not os.path.exists(HASH):
        return False
    with open(HASH) as fh:
        return fh.read().strip() == source_hash()


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-result",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           "-o", tmp] + sources()
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature switch; that warning is expected.
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    digest = source_hash()
    os.replace(tmp, LIB)
    with open(HASH + ".tmp", "w") as fh:
        fh.write(digest + "\n")
    os.replace(HASH + ".tmp", HASH)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
