"""Build the gfx950 shared library (C ABI) in-tree with hipcc.

Each source compiles to its own object (in parallel, under `_build/`), then
one link step makes `libmoe_prerouter.so`.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_prerouter.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["moe_api.hip", "kernels_decode.hip", "kernels_dec2.hip", "kernels_deca.hip", "kernels_prefill.hip",
           "kernels_shared.hip", "kernels_stage.hip", "kernels_stack.hip", "host_plan.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wno-unused-result",
]
# per-source extras: the prefill GEMMs keep their MFMA results in ordinary
# VGPRs (no copies between the matrix and vector register files around the
# per-group scaling, measured 15-20 % faster on the 64-token gate/up kernel)
EXTRA: dict[str, list[str]] = {
    "kernels_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _filtered(r: subprocess.CompletedProcess) -> str:
    return "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)


def compile_cmds(csrc: str = CSRC, objdir: str = OBJDIR, include: str | None = None):
    include = include or os.path.join(HERE, "..", "include")
    out = []
    for s in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(s)[0] + ".o")
        out.append((obj, [HIPCC, *FLAGS, *EXTRA.get(s, []), "-I", include, "-c", os.path.join(csrc, s), "-o", obj]))
    return out


def build(verbose: bool = False, csrc: str = CSRC, lib: str = LIB, objdir: str = OBJDIR) -> str:
    os.makedirs(objdir, exist_ok=True)
    cmds = compile_cmds(csrc, objdir)
    if verbose:
        for _, c in cmds:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda c: subprocess.run(c[1], capture_output=True, text=True), cmds))
    for (obj, _), r in zip(cmds, results):
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(obj)} ({r.returncode}):\n{_filtered(r)}")
        if verbose and _filtered(r).strip():
            print(_filtered(r))
    tmp = lib + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-fno-gpu-rdc", *[o for o, _ in cmds], "-o", tmp]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed ({r.returncode}):\n{_filtered(r)}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
