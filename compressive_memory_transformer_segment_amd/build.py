"""Build ``libinfini_attn.so`` (the C-ABI library of HIP kernels) for gfx950, in-tree.

Every HIP source under ``csrc/`` is compiled with hipcc for gfx950 and linked into one
shared library next to this file.  Packed-fp32 instruction selection is turned off for
all device code.  Nothing here is needed at run time: the binding only loads the built
library.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG_DIR), "include")
LIB_NAME = "libinfini_attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["api.hip", "state_pass.hip", "chain.hip", "attention.hip", "gemm.hip", "decode.hip", "backward.hip", "attention_bwd.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        "-Wall", "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}",
    ]


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc(), *common_flags(), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the device-only feature flag
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)


PROBES = {"ceilings.hip": "ceilings"}   # hardware-ceiling probe (measurement only, not linked)


def build_probes(verbose: bool = True) -> None:
    """Compile the measurement probes under probes/ into executables next to their sources."""
    pdir = os.path.join(PKG_DIR, "probes")
    for src, exe in PROBES.items():
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               os.path.join(pdir, src), "-o", os.path.join(pdir, exe)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for probes/{src}:\n{res.stdout}\n{res.stderr}")
        if verbose:
            print(f"built {os.path.join(pdir, exe)}")


def build(verbose: bool = True) -> str:
    """Compile all sources (in parallel) and link the shared library; returns its path."""
    obj_dir = os.path.join(PKG_DIR, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    objs = [os.path.join(obj_dir, s.replace(".hip", ".o")) for s in SOURCES]
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_compile, [os.path.join(CSRC, s) for s in SOURCES], objs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    build_probes(verbose)
    return LIB_PATH


if __name__ == "__main__":
    build()
