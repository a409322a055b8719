"""Build libvit.so (the HIP kernels + C ABI) for gfx950, in-tree.

    python -m quantized_kv_cache_append_amd.build

Compiles every source with hipcc (in parallel) into ``_build/`` and links
``libvit.so`` next to this file.  Flags that matter for correctness:
  * ``-ffp-contract=off`` on the append kernels: the codec encoders' fp32
    operation order is part of the bit-exact format;
  * no fast-math anywhere (IEEE division, denormals kept);
  * ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed fp32 VALU
    instructions are generated.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libvit.so")
ARCH = os.environ.get("VIT_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]
SOURCES = {
    "append.hip": ["-ffp-contract=off"],
    "decode_k0.hip": [],
    "decode_k1.hip": [],
    "decode_k2.hip": [],
    "decode_k3.hip": [],
    "decode_k4.hip": [],
    "reduce.hip": [],
    "noalloc.hip": [],
    "probe.hip": [],
    "vit_host.cpp": [],
}


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def _compile(src, extra):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [_hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
