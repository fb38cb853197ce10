"""Build the HIP shared libraries in-tree for gfx950.

    python quantized_moe_expert_lds_amd/build.py

produces ``quantized_moe_expert_lds_amd/lib/libmoe_ffn.so`` (the MoE FFN
library behind ``include/moe_ffn.h``) and ``moe_inputs/lib/libmoe_inputs.so``
(the GPU twin of the seeded weight generator).  Every call recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions anywhere (they are avoided on this platform)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result",
]


def _hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj: str) -> None:
    cmd = [_hipcc(), *HIP_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noisy = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noisy:
        sys.stderr.write("\n".join(noisy) + "\n")


def _link(objs, out: str) -> None:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build_library(srcdir: str, builddir: str, out: str, jobs: int = 8) -> str:
    os.makedirs(builddir, exist_ok=True)
    srcs = sorted(os.path.join(srcdir, f) for f in os.listdir(srcdir) if f.endswith(".hip"))
    objs = [os.path.join(builddir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _compile(*so), zip(srcs, objs)))
    _link(objs, out)
    return out


def build_all() -> None:
    build_library(os.path.join(PKG, "csrc"), os.path.join(PKG, "_build"),
                  os.path.join(PKG, "lib", "libmoe_ffn.so"))
    gen = os.path.join(ROOT, "moe_inputs")
    build_library(os.path.join(gen, "csrc"), os.path.join(gen, "_build"),
                  os.path.join(gen, "lib", "libmoe_inputs.so"))


if __name__ == "__main__":
    build_all()
    print("built")
