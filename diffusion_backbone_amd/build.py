"""Builds libdig.so (the C-ABI HIP library) in-tree for gfx950 with hipcc.

    python -m diffusion_backbone_amd.build        # or build() from Python
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdig.so")
PROBE_LIB = os.path.join(HERE, "libdig_probe.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["dig_api.cpp", "gla_fwd.hip", "gla_fwd_bf16.hip", "gla_fwd_f32.hip",
           "gla_fwd_bf16_lr.hip", "gla_bwd.hip", "gla_bwd_bf16.hip", "gla_bwd_f32.hip",
           "gla_bwd_bf16_lr.hip", "gla_beta.hip", "srem.hip", "linear.hip", "block.hip"]
HEADERS = ["dig_device.h", "dig_internal.h", "gla_fwd_kernel.h", "gla_bwd_kernel.h"]

ARCH = "gfx950"
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    # packed fp32 arithmetic stays off (scalar and float2 code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def _stale(obj: str, src: str) -> bool:
    if not os.path.exists(obj):
        return True
    deps = [src] + [os.path.join(CSRC, h) for h in HEADERS] + [os.path.join(ROOT, "include", "dig.h")]
    return any(os.path.getmtime(d) > os.path.getmtime(obj) for d in deps)


def build(verbose: bool = False, force: bool = True) -> str:
    """Compiles every source (force=True) or only stale objects, then links libdig.so."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        objs.append(obj)
        if not force and not _stale(obj, os.path.join(CSRC, src)):
            continue
        cmd = [hipcc] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd = [hipcc] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                  stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, cmd, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l
                        and "not a recognized feature" not in l)
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out)
    if failed:
        msg = "\n".join("--- %s\n%s" % f for f in failed)
        raise RuntimeError("hipcc failed:\n" + msg)
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    build_probe(hipcc)
    return LIB


def build_probe(hipcc: str) -> str:
    """libdig_probe.so: the measurement kernels bench.py times (contraction microbenchmark,
    streaming copy); not part of libdig.so."""
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc] + FLAGS + ["-shared", "-o", tmp, os.path.join(CSRC, "probe.hip")],
                          stderr=subprocess.DEVNULL)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, force="--incremental" not in sys.argv))
