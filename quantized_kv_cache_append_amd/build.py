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
import json
import re
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
          "-Wno-unused-command-line-argument",
          "-Rpass-analysis=kernel-resource-usage"]  # per-kernel registers, scratch, LDS (kept below)
RESOURCES = os.path.join(BUILD, "kernel_resources.json")
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                     r"LDS Size \[bytes/block\]|VGPRs Spill|SGPRs Spill):\s+(\S+)")
_KEYS = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "waves_per_simd",
         "LDS Size [bytes/block]": "lds", "VGPRs Spill": "vgpr_spill", "SGPRs Spill": "sgpr_spill"}
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


def _resources(stderr):
    """{kernel: {vgpr, agpr, scratch, ...}} from the compiler's resource remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(stderr):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[_KEYS[key]] = int(val) if val.isdigit() else val
    return out


def _compile(src, extra):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [_hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and "remark:" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj, _resources(r.stderr)


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(jobs) as ex:
        done = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    objs = [o for o, _ in done]
    res = {}
    for _, r in done:
        res.update(r)
    with open(RESOURCES, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
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
