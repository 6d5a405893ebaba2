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

SOURCES = ["kvq_host.cpp", "kvq_api.cpp", "kvq_append.hip", "kvq_decode.hip", "kvq_decode_mfma.hip", "kvq_decode_latent.hip", "kvq_decode_turbo.hip", "kvq_decode_kivi.hip", "kvq_hsi.hip", "kvq_probe.hip", "kvq_static.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    log = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    return res.returncode, log


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source into libkvq.so next to this file (or `out`); returns its path.

    Each translation unit compiles to its own object (in parallel) under
    _build/ next to the output, then hipcc links them."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(os.path.dirname(os.path.abspath(out)), "_build")
    os.makedirs(objdir, exist_ok=True)
    tag = os.path.basename(out).replace(".so", "")
    cflags = [f for f in FLAGS if f != "-shared"] + [f"-D{d}" for d in defines]
    jobs = []
    for s in SOURCES:
        obj = os.path.join(objdir, f"{tag}_{s}.o")
        jobs.append((obj, [HIPCC] + cflags + ["-c", os.path.join(CSRC, s), "-o", obj]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(lambda j: _run(j[1], verbose), jobs))
    failed = False
    for rc, log in results:
        if rc != 0:
            failed = True
            sys.stderr.write(log + "\n")
        elif verbose and log.strip():
            print(log)
    if failed:
        raise RuntimeError("hipcc failed building libkvq.so")
    tmp = out + ".tmp"
    rc, log = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [j[0] for j in jobs]
                   + ["-lamdhip64"], verbose)
    if rc != 0:
        sys.stderr.write(log + "\n")
        raise RuntimeError("hipcc failed linking libkvq.so")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
