"""Build liblattn.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblattn.so")
SOURCES = [os.path.join(CSRC, n) for n in ("lattn_kernels.hip", "lattn_gated.hip", "lattn_noalloc.hip", "lattn_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off (hipcc's host pass warns it does not know the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs: the register budget fits, and it avoids
    # moving every accumulator between AGPRs and VGPRs for the VALU steps
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if errs.strip() and verbose:
        print(errs, file=sys.stderr)


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every source into ``out`` (always recompiles; one hipcc per source, in
    parallel, then one link)."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(os.path.dirname(out), "_build")
    os.makedirs(objdir, exist_ok=True)
    stem = os.path.basename(out)
    objs = [os.path.join(objdir, f"{stem}.{os.path.basename(src)}.o") for src in SOURCES]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    cmds = [[HIPCC] + compile_flags + list(extra or []) + ["-c", src, "-o", obj] for src, obj in zip(SOURCES, objs)]
    with ThreadPoolExecutor(len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", out + ".tmp"], verbose)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
