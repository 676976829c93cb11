"""Build libnomas_attn.so in-tree with hipcc for gfx950.

    python -m segment_causal_masked_amd.build

HIP sources (*.hip) are compiled for the device and host; C++ sources are
compiled as host code against the HIP runtime headers; everything is linked
into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnomas_attn.so")
# the MFMA throughput probe the benchmark reports beside its roofline (a
# measuring instrument, built as its own library)
PROBE_SRC = os.path.join(PKG, "probe", "mfma_peak.hip")
PROBE_LIB = os.path.join(PKG, "libnomas_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
# Packed fp32 VALU forms are kept out of the device code on purpose.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-ffp-contract=fast", "-munsafe-fp-atomics"]
# Per-file additions (later flags win): the video-block score is defined with
# separately rounded products and adds, so nothing in that file is fused.
DEVICE_EXTRA = {"select.hip": ["-ffp-contract=off"]}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for f in sources():
        src = os.path.join(CSRC, f)
        obj = os.path.join(BUILD, f + ".o")
        if f.endswith(".hip"):
            cmd = [HIPCC, *COMMON, *DEVICE, *DEVICE_EXTRA.get(f, []), "-c", src, "-o", obj]
        else:
            cmd = [HIPCC, *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c", src, "-o", obj]
        jobs.append((cmd, obj))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for r in ex.map(lambda j: _run(j[0]), jobs):
            if verbose and r.stderr:
                print(r.stderr, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *[o for _, o in jobs]])
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    _run([HIPCC, *COMMON, *DEVICE, "-shared", PROBE_SRC, "-o", tmp])
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
