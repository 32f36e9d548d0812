"""Builds libmla.so (the MLA kernels + C ABI) and libmla_inputs.so (the device
input generator) in-tree for gfx950 with hipcc.  ``python -m
mla_latent_kv_dkv_amd.build`` or ``build()``."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build", "obj")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# packed-fp32 instructions are disabled for every device compile
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]

LIBS = {
    "libmla.so": ["mla_api.cpp", "errword.hip", "kernels_generic.hip", "kernels_fast.hip",
                  "gemm_fast.hip", "fp8_cache.hip"],
    "libmla_inputs.so": ["fill_inputs.hip"],
}


def _compile(src: str, verbose: bool) -> str:
    os.makedirs(OBJ, exist_ok=True)
    out = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    return out


def build(verbose: bool = False) -> list:
    """Compile every source and link both libraries; returns their paths.  Any
    previously built library is removed first, so a failed build never leaves a
    stale one behind."""
    for lib in LIBS:
        if os.path.exists(os.path.join(HERE, lib)):
            os.remove(os.path.join(HERE, lib))
    srcs = sorted({s for v in LIBS.values() for s in v})
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    built = []
    for lib, parts in LIBS.items():
        out = os.path.join(HERE, lib)
        tmp = out + ".tmp"
        cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + [objs[s] for s in parts]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link of {lib} failed:\n{r.stdout}{r.stderr}")
        os.replace(tmp, out)
        built.append(out)
    return built


if __name__ == "__main__":
    for p in build(verbose=True):
        print(p)
