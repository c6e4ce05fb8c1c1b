"""Build libgptq_mi355x.so (gfx950) in-tree with hipcc.

    python -m post_weight_quantization_17_amd.build

Every HIP source in csrc/ is compiled for gfx950 and linked into
``post_weight_quantization_17_amd/libgptq_mi355x.so``. Packed-fp32 VALU
instructions are disabled for the device code.

The compiler's per-kernel resource report (registers, LDS, occupancy,
scratch) is written to ``_build/kernel_resources.txt``; the build fails if
any kernel needs scratch memory (register spills or a dynamic stack): every
kernel of the library is designed to run from registers and LDS alone.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgptq_mi355x.so")
ARCH = os.environ.get("GPTQ_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang",
    "-target-feature",
    "-Xclang",
    "-packed-fp32-ops",
    "-Rpass-analysis=kernel-resource-usage",
]
RESOURCES = os.path.join(BUILD, "kernel_resources.txt")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def kernel_resources(remarks: str) -> dict:
    """{kernel: {field: value}} from the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z /\[\]]+?): (\S+) \[-Rpass-analysis", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return out


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj, kernel_resources(r.stderr)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(len(srcs), os.cpu_count() or 4)) as pool:
        done = list(pool.map(_compile, srcs))
    objs = [o for o, _ in done]
    res = {k: v for _, r in done for k, v in r.items()}
    with open(RESOURCES, "w") as f:
        f.write("kernel VGPRs AGPRs SGPRs scratch_bytes_per_lane dynamic_stack occupancy_waves_per_simd lds_bytes\n")
        for k in sorted(res):
            v = res[k]
            f.write(" ".join([k] + [v.get(x, "?") for x in ("VGPRs", "AGPRs", "TotalSGPRs", "ScratchSize [bytes/lane]",
                                                             "Dynamic Stack", "Occupancy [waves/SIMD]",
                                                             "LDS Size [bytes/block]")]) + "\n")
    if not res:
        raise RuntimeError("no kernel resource report from hipcc")
    spill = [k for k, v in res.items() if v.get("ScratchSize [bytes/lane]") != "0" or v.get("Dynamic Stack") != "False"]
    if spill:
        raise RuntimeError(f"kernels that need scratch memory (see {RESOURCES}): {spill}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources for {ARCH}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
