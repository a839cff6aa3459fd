"""Build libqsa.so (gfx950) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with floating-point contraction
off (the rotary recipe is a sequence of separately rounded fp32 operations) and
packed-fp32 instruction selection disabled.  The host rotary-table source is
compiled with -fno-builtin so libm cos/sin are called as written.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqsa.so")
PROBE_LIB = os.path.join(PKG, "libqsa_probe.so")     # benchmark-only gather probe, not the QSA boundary
ARCH = "gfx950"

HIP_SOURCES = ["qsa_api.hip", "k_prologue.hip", "k_indexer.hip", "k_select.hip", "k_attend.hip", "k_decode.hip", "k_gdn.hip",
               "k_train.hip", "k_dense.hip"]
CPP_SOURCES = ["qsa_tables.cpp"]
PROBE_SOURCES = ["probe_gather.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Werror", "-Wno-unused-function", "-Wno-unused-variable",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
CPP_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fno-builtin", "-ffp-contract=off", "-Wall", "-Werror"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libqsa.so.  Always recompiles."""
    os.makedirs(OBJ, exist_ok=True)
    jobs_list = []
    for src in HIP_SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        jobs_list.append(([HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj], obj))
    for src in CPP_SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        jobs_list.append((["g++"] + CPP_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj], obj))
    probe_jobs = []
    for src in PROBE_SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        probe_jobs.append(([HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj], obj))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        outs = list(ex.map(lambda j: _run(j[0]), jobs_list + probe_jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [o for _, o in jobs_list])
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [o for _, o in probe_jobs])
    os.replace(tmp, PROBE_LIB)
    return LIB


ASAN_DIR = os.path.join(OBJ, "asan")
ASAN_RUNTIME = "/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"


def build_asan(jobs: int = 8) -> str:
    """libqsa.so with its host code built under AddressSanitizer (device code
    as usual), into _build/asan/.  Host-only checking: the library's argument
    checks, workspace sizing and table construction run instrumented; load it
    with the ASan runtime preloaded (ASAN_RUNTIME) and no GPU."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    jobs_list = []
    for src in HIP_SOURCES:
        obj = os.path.join(ASAN_DIR, src + ".o")
        jobs_list.append(([HIPCC] + HIP_FLAGS + san + ["-c", os.path.join(CSRC, src), "-o", obj], obj))
    clangxx = os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin", "clang++")
    for src in CPP_SOURCES:
        obj = os.path.join(ASAN_DIR, src + ".o")
        jobs_list.append(([clangxx] + CPP_FLAGS + ["-fsanitize=address", "-fno-omit-frame-pointer", "-c",
                                                   os.path.join(CSRC, src), "-o", obj], obj))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda j: _run(j[0]), jobs_list))
    lib = os.path.join(ASAN_DIR, "libqsa.so")
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host", "-fsanitize=address",
          "-shared-libsan", "-o", lib] + [o for _, o in jobs_list])
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
