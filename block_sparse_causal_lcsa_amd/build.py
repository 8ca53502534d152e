"""Builds liblcsa.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m block_sparse_causal_lcsa_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblcsa.so")
ARCH = "gfx950"

KERNELS = ["pool.hip", "score_select.hip", "attn_fwd.hip", "attn_fwd_block.hip", "attn_bwd.hip", "stream.hip",
           "rope.hip", "probe.hip"]
HOST = ["lcsa_host.cpp"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# Packed fp32 VALU ops are kept out of every device build.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]
# Per-unit extra flags. The block-granular attention variants run 7% faster under the iterative ILP
# machine scheduler (LDS operand reads spread between the MFMAs); the other units are no faster with
# it, and the token-window attention variant spills more registers.
EXTRA = {"attn_fwd_block.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OUT, exist_ok=True)
    jobs = []
    for src in KERNELS:
        obj = os.path.join(OUT, src.replace(".hip", ".o"))
        jobs.append(["hipcc", *COMMON, *DEVICE, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST:
        obj = os.path.join(OUT, src.replace(".cpp", ".o"))
        # host only; fp64 keep-ratio rule evaluated without contraction
        jobs.append(["hipcc", *COMMON, "-ffp-contract=off", "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


# Build of every source whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer
# (each -fsanitize= applies to the host pass only, -Xarch_host): the validation, geometry and
# stream-state code that runs before any launch, checked on the CPU. Device code is built as usual.
SAN_LIB = os.path.join(OUT, "hostsan", "liblcsa_hostsan.so")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_sanitized() -> str:
    out = os.path.dirname(SAN_LIB)
    os.makedirs(out, exist_ok=True)
    base = [*COMMON, "-Xarch_host", "-g"]
    jobs = []
    for src in KERNELS:
        jobs.append(["hipcc", *base, *DEVICE, *EXTRA.get(src, []), *SAN, "-c",
                     os.path.join(CSRC, src), "-o", os.path.join(out, src.replace(".hip", ".o"))])
    for src in HOST:
        jobs.append(["hipcc", *base, "-ffp-contract=off", *SAN, "-c", os.path.join(CSRC, src), "-o",
                     os.path.join(out, src.replace(".cpp", ".o"))])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(_run, jobs))
    tmp = SAN_LIB + ".tmp"
    _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN, "-o", tmp, *[j[-1] for j in jobs]])
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def sanitizer_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (to LD_PRELOAD into a Python that loads
    the sanitized library)."""
    r = subprocess.run(["hipcc", "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                       stderr=subprocess.DEVNULL, text=True)
    return r.stdout.strip()


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized())
    else:
        print(build(verbose="-v" in sys.argv))
