"""Build libmla.so (HIP for gfx950) in-tree with hipcc.

    python -m mla_latent_kv_05_amd.build            # build
    python -m mla_latent_kv_05_amd.build --asm      # also dump device assembly

Every source under csrc/ is compiled for gfx950 only.  Packed fp32 VALU
instructions are disabled (-packed-fp32-ops)."""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla.so)")


def common_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "--amdgpu-mfma-vgpr-form=1",
            "-Wno-unused-command-line-argument"]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-c", src, "-o", obj] + common_flags()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-o", tmp] + objs + [f"--offload-arch={ARCH}", "-fPIC"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def dump_asm(out_dir: str) -> None:
    os.makedirs(out_dir, exist_ok=True)
    for src in sources():
        out = os.path.join(out_dir, os.path.basename(src) + ".s")
        cmd = [hipcc(), "-S", "--cuda-device-only", src, "-o", out] + common_flags()
        subprocess.run(cmd, check=True, capture_output=True)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", metavar="DIR", help="also write device assembly to DIR")
    args = ap.parse_args(argv)
    build(verbose=True)
    if args.asm:
        dump_asm(args.asm)
    return 0


if __name__ == "__main__":
    sys.exit(main())
