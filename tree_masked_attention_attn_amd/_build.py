"""Compile the HIP library in-tree with hipcc for gfx950.

Produces ``tree_masked_attention_attn_amd/libtree_attn.so``. Objects go to
``tree_masked_attention_attn_amd/_build/``. Every call recompiles.

Flags: ``-O3 --offload-arch=gfx950`` and the packed-fp32 feature switched off
for device code (``-Xclang -target-feature -Xclang -packed-fp32-ops``); the
host pass warns that it does not know that feature, which is harmless.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtree_attn.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I" + os.path.join(ROOT, "include")]
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SOURCES = [("plan.cpp", False), ("api.cpp", False),
           ("tree_attn_kernel.hip", True), ("kv_reroot_kernel.hip", True),
           ("tree_verify_kernel.hip", True), ("tree_expand_kernel.hip", True), ("noalloc.hip", True)]


def _compile(src, device):
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + (DEVICE if device else ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include")]) + \
        ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj, err


def build(verbose=False):
    os.makedirs(OUT_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(*s), SOURCES))
    for obj, err in results:
        if err and verbose:
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
