"""Build libpagedkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_120_amd.build
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpagedkv.so")
SOURCES = ["csrc/decode.hip", "csrc/cache_ops.hip", "csrc/probe.hip", "csrc/api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def command(out: str = LIB, extra=()):
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # no packed-fp32 instructions anywhere in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
        *extra,
        *[os.path.join(HERE, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only target feature above
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in r.stdout.splitlines() if noise not in l)
    if msg.strip():
        print(msg, file=sys.stderr)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
