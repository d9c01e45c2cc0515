"""Build libep.so (HIP kernels for gfx950 + host driver) in-tree with hipcc.

Each translation unit is compiled in its own hipcc process (in parallel), then linked."""

from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(OUT_DIR, "libep.so")
UNITS = ["ep_kernels.hip"] + [f"ep_decode_{d}{k}.hip" for d in ("bf16", "fp16", "fp8", "int8", "fp32")
                              for k in ("", "_k128")] + [
    "ep_decode_mm_bf16.hip", "ep_decode_mm_fp16.hip", "ep_decode_trace.hip", "ep_encode.hip",
    "ep_rate.hip",
    "ep_host.cpp"]
SOURCES = [os.path.join(CSRC, u) for u in UNITS]
HEADERS = [os.path.join(ROOT, "include", "ep.h")] + [
    os.path.join(CSRC, h) for h in ("ep_internal.h", "ep_device.h", "ep_load.h", "ep_decode.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # every product and sum in the E8 quantiser and the row sums is rounded on its own
    "-ffp-contract=off",
    # packed fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the decoder's phase loop must unroll fully (its fields live in registers indexed by phase)
    "-mllvm", "-pragma-unroll-threshold=1000000",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    incs = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        procs.append((src, subprocess.Popen([HIPCC, *FLAGS, *incs, "-c", "-o", obj, src],
                                            stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
    errors = []
    for src, p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            errors.append(f"{src}:\n{out}{err}")
        elif verbose and err.strip():
            print(err)
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    tmp = LIB + ".tmp"
    res = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
                          "-lpthread"], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
