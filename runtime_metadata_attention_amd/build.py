"""Build libcompilemask.so (host C++ + HIP kernels for gfx950) in-tree.

    python -m runtime_metadata_attention_amd.build [--jobs N] [--debug]

Every .cpp and .hip file under csrc/ is compiled by hipcc for gfx950 and
linked into runtime_metadata_attention_amd/lib/libcompilemask.so.  Objects go
to _build/ at the repository root.  Packed fp32 instructions are disabled for
all device code.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libcompilemask.so")
BUILD = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-result"]


# Per-file options.  The backward kernels consume most MFMA results with VALU
# code; asking for VGPR-form MFMAs there avoids AGPR<->VGPR copies of every
# score tile.
FILE_FLAGS = {"attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.cpp")) + glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, opt: list, extra: list) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *opt, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature; drop that warning
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(jobs: int = 8, debug: bool = False, extra=None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    opt = ["-O1", "-g"] if debug else ["-O3"]
    extra = list(extra or [])
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, opt, extra), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # a kernel whose host-side launch stub was not emitted leaves an undefined
    # symbol that would only surface when the library is loaded
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        raise RuntimeError("kernel launch stubs missing from the library: " + ", ".join(missing))
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--debug", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.debug))


if __name__ == "__main__":
    main()
