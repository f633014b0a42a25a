"""Build libkvq.so for gfx950 with hipcc, in-tree.

    python -m quantized_kv_cache_02_amd.build        # or build() from Python

The split-decode kernel source is compiled once per (cache dtype, K scale
mode, V scales per row or static), plus once for the unquantized bf16 cache,
so its variants build in parallel translation units.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvq.so")
# the streaming-read probe benchmarks compare the decode with: a library of its own
PROBE_LIB = os.path.join(PKG, "libkvq_probe.so")
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops stay off (plain fp32 and packed fp16 only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _units():
    units = [
        ("kvq_host.o", os.path.join(CSRC, "kvq_host.cpp"), []),
        ("kvq_append.o", os.path.join(CSRC, "kvq_append.hip"), []),
        ("kvq_combine.o", os.path.join(CSRC, "kvq_combine.hip"), []),
    ]
    # one unit per (dtype, K scale mode, V scales per row or static).  The MFMA
    # accumulators stay in ordinary VGPRs: the variants built for one wavefront
    # per SIMD then keep what exceeds 256 registers in the accumulation
    # registers (one-cycle copies), where the default form put the accumulators
    # there and copied all of them around every rescale test.
    vf = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    for dt in (1, 2, 3):
        for md in (1, 2, 3):
            for vr in (0, 1):
                units.append((f"kvq_split_{dt}_{md}_{vr}.o", os.path.join(CSRC, "kvq_split.hip"),
                              [f"-DKVQ_DTYPE={dt}", f"-DKVQ_MODE={md}", f"-DKVQ_VROW={vr}", *vf]))
    # the unquantized bf16 cache: no scales
    units.append(("kvq_split_4_0_0.o", os.path.join(CSRC, "kvq_split.hip"),
                  ["-DKVQ_DTYPE=4", "-DKVQ_MODE=0", "-DKVQ_VROW=0", *vf]))
    # the wide-row-set variants (one wavefront per SIMD), in units of their own
    # built in the default MFMA form: their accumulators (up to 192 registers)
    # live in the accumulation registers, which the MFMAs read and write
    # directly, and everything else in the ordinary ones
    for dt, md, vr in [(d, m, v) for d in (1, 2, 3) for m in (1, 2, 3) for v in (0, 1)] + [(4, 0, 0)]:
        units.append((f"kvq_split_wide_{dt}_{md}_{vr}.o", os.path.join(CSRC, "kvq_split.hip"),
                      [f"-DKVQ_DTYPE={dt}", f"-DKVQ_MODE={md}", f"-DKVQ_VROW={vr}", "-DKVQ_WIDE=1"]))
    # the chunked-prefill kernel, split the same way.  Its accumulators stay in
    # ordinary vector registers: left to itself the backend parks them in the
    # accumulation registers and copies all of them in and out on every tile
    # (160 copies per tile at D 256).
    pf = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    for dt in (1, 2, 3):
        for md in (1, 2, 3):
            for vr in (0, 1):
                units.append((f"kvq_prefill_{dt}_{md}_{vr}.o", os.path.join(CSRC, "kvq_prefill.hip"),
                              [f"-DKVQ_DTYPE={dt}", f"-DKVQ_MODE={md}", f"-DKVQ_VROW={vr}", *pf]))
    units.append(("kvq_prefill_4_0_0.o", os.path.join(CSRC, "kvq_prefill.hip"),
                  ["-DKVQ_DTYPE=4", "-DKVQ_MODE=0", "-DKVQ_VROW=0", *pf]))
    return units


def _compile(obj, src, extra):
    out = os.path.join(BUILD, obj)
    cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", out]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *COMMON, "-x", "hip", *extra, "-c", src, "-o", out]
    t0 = time.time()
    p = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(ln for ln in (p.stdout + p.stderr).splitlines()
                     if "packed-fp32-ops" not in ln)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {obj}:\n{' '.join(cmd)}\n{msgs}")
    return obj, time.time() - t0, msgs


def build(verbose: bool = True, jobs: int | None = None) -> str:
    """Compile every HIP translation unit for gfx950 and link libkvq.so."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    units = _units()
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_compile, *u) for u in units]
        for f in cf.as_completed(futs):
            obj, dt, msgs = f.result()
            if verbose:
                print(f"[kvq build] {obj} {dt:.1f}s", flush=True)
                if msgs.strip():
                    print(msgs, flush=True)
    tmp = LIB + ".tmp"
    objs = [os.path.join(BUILD, u[0]) for u in units]
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stdout}\n{p.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"[kvq build] linked {LIB}", flush=True)
    obj, _, msgs = _compile("kvq_probe.o", os.path.join(CSRC, "kvq_probe.hip"), [])
    tmp = PROBE_LIB + ".tmp"
    p = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
                        os.path.join(BUILD, obj)], capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stdout}\n{p.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"[kvq build] linked {PROBE_LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
