"""Builds libkvq.so (all HIP kernels and the C-ABI host code) for gfx950 with hipcc."""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["kvq_host.cpp", "kvq_api.cpp", "kvq_append.hip", "kvq_decode.hip", "kvq_decode_mfma.hip", "kvq_decode_latent.hip", "kvq_decode_turbo.hip", "kvq_hsi.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source into libkvq.so next to this file (or `out`); returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC] + FLAGS + [f"-D{d}" for d in defines] + ["-o", tmp] + srcs + ["-lamdhip64"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    log = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        sys.stderr.write(log + "\n")
        raise RuntimeError("hipcc failed building libkvq.so")
    if verbose and log.strip():
        print(log)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
