"""Builds libhbl.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

Usage: python bit_quantization_amd/build.py [--force]  (run by path: importing
the package loads the library, which need not exist or be current yet)
The library is written next to this file, in-tree, so that it travels with
the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libhbl.so")
PROBE = os.path.join(HERE, "peak_probe")  # stand-alone program: measured device peaks
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["k_quant.hip", "k_ternarize.hip", "k_gemm.hip", "k_gemm_mx.hip", "k_kvquant.hip", "hbl_noalloc.hip",
           "hbl_api.cpp"]
HEADERS = [os.path.join(CSRC, "hbl_internal.h"), os.path.join(CSRC, "k_dot.h"), os.path.join(ROOT, "include", "hbl.h")]

# -ffp-contract=off: no fused multiply-adds, so every product and sum is
# rounded as written.  Packed fp32 instructions are disabled.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
]


def _stale(target: str, deps: list[str]) -> bool:
    if not os.path.exists(target):
        return True
    t = os.path.getmtime(target)
    return any(os.path.getmtime(d) > t for d in deps)


def build(force: bool = False, verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(OBJ, src + ".o")
        objs.append(obj)
        if force or _stale(obj, [path] + HEADERS):
            cmd = [HIPCC, *FLAGS, "-c", path, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the gfx950 feature name: harmless
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, text))
        elif text.strip() and verbose:
            print(text)
    if failed:
        msg = "\n".join(f"--- {s} ---\n{t}" for s, t in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    if force or procs or _stale(LIB, objs):
        tmp = LIB + ".tmp"
        subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
        os.replace(tmp, LIB)
    probe_src = os.path.join(CSRC, "peak_probe.hip")
    if force or _stale(PROBE, [probe_src]):
        cmd = [HIPCC, *[f for f in FLAGS if f != "-fPIC"], probe_src, "-o", PROBE + ".tmp"]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed on peak_probe.hip:\n" + r.stdout.decode(errors="replace"))
        os.replace(PROBE + ".tmp", PROBE)
    return LIB


if __name__ == "__main__":
    build(force="--force" in sys.argv, verbose=True)
    print(LIB)
