"""Builds libconvverify.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: python -m causal_conv1d_verify_amd.build   (or __graft_entry__.build())
"""

from __future__ import annotations

import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libconvverify.so")
# The write-count build (tests only): every global store also counts into registered
# ranges (conv_verify_debug_count).  Its verify objects cover bf16 x and state only.
LIB_WC = os.path.join(PKG, "libconvverify_wc.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 instructions are kept out of every kernel: hipcc would otherwise form
# v_pk_{add,mul,fma}_f32 from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # the token loop is unrolled over its compile-time bucket (up to 32) so
                # every register index is static; allow that size
                "-mllvm", "-pragma-unroll-threshold=1000000"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra", "-Wno-unused-parameter",
          f"-I{INCLUDE}", f"-I{CSRC}"]

# The verify kernel source is compiled once per (x bytes, state bytes, variant:
# 0 dense, 1 rows, 2 time-major rows, 3 tree; conv_state layout: 0 channel-major,
# 1 time-major); those objects, the restore / prefill / L2 kernels and the C ABI build
# in parallel.
SOURCES = [
    ("cv_kernels.hip", f"cv_kernels_{xb}_{sb}_{v}_{tm}",
     [f"--offload-arch={ARCH}", *DEVICE_FLAGS, f"-DCV_XB={xb}", f"-DCV_SB={sb}",
      f"-DCV_VARIANT={v}", f"-DCV_TM={tm}"])
    for tm in (0, 1) for xb, sb in ((4, 4), (2, 2), (2, 4)) for v in (0, 1, 2, 3)
] + [("cv_aux_kernels.hip", "cv_aux_kernels", [f"--offload-arch={ARCH}", *DEVICE_FLAGS]),
     ("cv_api.cpp", "cv_api", [])]
SOURCES_WC = [
    ("cv_kernels.hip", f"wc/cv_kernels_2_2_{v}_{tm}",
     [f"--offload-arch={ARCH}", *DEVICE_FLAGS, "-DCV_XB=2", "-DCV_SB=2", f"-DCV_VARIANT={v}",
      f"-DCV_TM={tm}", "-DCV_WRITE_COUNT"])
    for tm in (0, 1) for v in (0, 1, 2, 3)
] + [("cv_aux_kernels.hip", "wc/cv_aux_kernels", [f"--offload-arch={ARCH}", *DEVICE_FLAGS, "-DCV_WRITE_COUNT"]),
     ("cv_api.cpp", "wc/cv_api", ["-DCV_WRITE_COUNT"])]
MAX_JOBS = max(1, min(len(SOURCES) + len(SOURCES_WC), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}):\n{' '.join(cmd)}\n"
                           f"{res.stdout}\n{res.stderr}")
    return res


def build(verbose: bool = True) -> str:
    """Builds libconvverify.so and the write-count test library libconvverify_wc.so."""
    os.makedirs(os.path.join(BUILD, "wc"), exist_ok=True)
    t0 = time.time()
    pending = []
    libs = []
    for sources, lib in ((SOURCES, LIB), (SOURCES_WC, LIB_WC)):
        objs = []
        for src, stem, extra in sources:
            obj = os.path.join(BUILD, stem + ".o")
            pending.append([HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        libs.append((lib, objs))
    running = []

    def reap(cmd, p):
        out, err = p.communicate()
        if p.returncode != 0:
            for _, q in running:
                q.kill()
            raise RuntimeError(f"build step failed ({p.returncode}):\n{' '.join(cmd)}\n{out}\n{err}")
        noise = [ln for ln in err.splitlines()
                 if ln.strip() and "packed-fp32-ops' is not a recognized feature" not in ln]
        if verbose and noise:
            print("\n".join(noise), file=sys.stderr)

    while pending or running:
        while pending and len(running) < MAX_JOBS:
            cmd = pending.pop(0)
            running.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                  stderr=subprocess.PIPE, text=True)))
        cmd, p = running.pop(0)
        reap(cmd, p)
    for lib, objs in libs:
        tmp = lib + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
        os.replace(tmp, lib)
    if verbose:
        print(f"built {LIB} and {LIB_WC} in {time.time() - t0:.1f}s", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
