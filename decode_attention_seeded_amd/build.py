"""Builds libtq.so (HIP for gfx950) in-tree.

    python -m decode_attention_seeded_amd.build

Objects go to decode_attention_seeded_amd/_build/, the library to
decode_attention_seeded_amd/libtq.so. The split-K decode and the encode
kernels are compiled once per (head dim, key bits) pair in parallel processes.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtq.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 vector ops stay off in all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]

DECODE_VARIANTS = [(d, bk) for d in (128, 256) for bk in (2, 3, 4, 16)]
ENCODE_VARIANTS = [(d, bk) for d in (128, 256) for bk in (2, 3, 4)]


def _jobs():
    jobs = [
        ("tq_host.o", ["g++", "-O2", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__",
                       "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
                       "-c", os.path.join(CSRC, "tq_host.cpp")]),
        ("tq_api.o", [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "tq_api.hip")]),
        ("tq_affine.o", [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "tq_affine.hip")]),
    ]
    for d, bk in DECODE_VARIANTS:
        jobs.append((f"tq_decode_d{d}_k{bk}.o",
                     [HIPCC, *HIP_FLAGS, f"-DTQ_D={d}", f"-DTQ_BK={bk}",
                      "-c", os.path.join(CSRC, "tq_inst_decode.hip")]))
    for d in (128, 256):
        jobs.append((f"tq_prefill_d{d}.o",
                     [HIPCC, *HIP_FLAGS, f"-DTQ_D={d}",
                      "-c", os.path.join(CSRC, "tq_inst_prefill.hip")]))
    for d, bk in ENCODE_VARIANTS:
        jobs.append((f"tq_encode_d{d}_k{bk}.o",
                     [HIPCC, *HIP_FLAGS, f"-DTQ_D={d}", f"-DTQ_BK={bk}",
                      "-c", os.path.join(CSRC, "tq_inst_encode.hip")]))
    return jobs


def _run(name, cmd, verbose):
    out = os.path.join(OUT, name)
    full = cmd + ["-o", out]
    if verbose:
        print(" ".join(full), flush=True)
    r = subprocess.run(full, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {name} failed:\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source for gfx950 and link libtq.so; returns its path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(OUT, exist_ok=True)
    n = jobs or min(8, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(n) as ex:
        futs = [ex.submit(_run, name, cmd, verbose) for name, cmd in _jobs()]
        objs = [f.result() for f in futs]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
