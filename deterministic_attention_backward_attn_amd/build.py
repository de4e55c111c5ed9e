"""Build the C-ABI shared library libdash_attn.so in-tree with hipcc for gfx950.

Usage: python -m deterministic_attention_backward_attn_amd.build   (or build())

Objects go to _build/ next to this file; the library to
deterministic_attention_backward_attn_amd/libdash_attn.so.  Every call
recompiles every source (a cross-compile for gfx950 works without a GPU).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdash_attn.so")

SOURCES = [
    "host/abi.cpp",
    "host/schedule.cpp",
    "host/dag.cpp",
    "kernels/attn_bwd.hip",
    "kernels/attn_bwd_pair.hip",
    "kernels/attn_bwd_pipe.hip",
    "kernels/attn_fwd.hip",
    "kernels/elementwise.hip",
    "kernels/noalloc.hip",
]

ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
          f"-I{os.path.join(ROOT, 'include')}"]
# Device flags: packed-fp32 instructions off (they are formed from plain
# float code otherwise); hardware fp32 atomics for the dQ adds.
DEVICE = [f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Forward: MFMA results in vector registers (the softmax reads the scores
# with VALU instructions, which cannot take the accumulation registers, so
# otherwise every read is a copy): 16K causal forward 3.19 -> 2.69 ms.  The
# backward measured slower with it (10.5 -> 11.3 ms) and keeps the default.
MFMA_VGPR = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
PER_FILE = {
    "kernels/attn_fwd.hip": MFMA_VGPR,
}


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(src: str, verbose: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src.replace("/", "_") + ".o")
    hip = src.endswith(".hip")
    cmd = [_hipcc(), *COMMON, "-c", path, "-o", obj]
    if hip:
        cmd[1:1] = ["-x", "hip", *DEVICE, *PER_FILE.get(src, [])]
    else:
        # host translation units include HIP runtime headers only
        cmd[1:1] = ["-D__HIP_PLATFORM_AMD__"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{res.stdout}\n{res.stderr}")
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise and verbose:
        print("\n".join(noise), file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int = 6) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
