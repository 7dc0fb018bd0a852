"""Build libkvq.so in-tree with hipcc for gfx950.

Run as a script (python quantized_decode_attention_amd/_build.py) or load it by
path (load_build_module()): importing it through the package would first load
the library being rebuilt.

Every HIP source is compiled with packed-FP32 instruction selection disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); the quantisation sources
also with -ffp-contract=off so binary32 arithmetic rounds exactly as written.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvq.so")
BUILD_DIR = os.path.join(PKG, "_build")

# source -> extra flags
SOURCES = {
    "kvq_api.cpp": [],
    "quant_write.hip": ["-ffp-contract=off"],
    "kvarn_write.hip": ["-ffp-contract=off"],
    "dequant.hip": ["-ffp-contract=off"],
    "decode_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "kvarn_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "decode_scratch.hip": [],
}

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libkvq")


def _compile(src: str, flags: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source (always; the caller asked for a build) and link
    libkvq.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = {s: f for s, f in SOURCES.items() if os.path.exists(os.path.join(CSRC, s))}
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), srcs.items()))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libkvq.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


READ_PROBE_SRC = os.path.join(CSRC, "read_probe.hip")
READ_PROBE_LIB = os.path.join(PKG, "libkvq_probe.so")


def build_read_probe() -> str:
    """The benchmark's measurement helper (libkvq_probe.so, not part of
    libkvq): the decode's access pattern with no arithmetic."""
    tmp = READ_PROBE_LIB + ".tmp"
    cmd = [hipcc(), *COMMON, "-shared", READ_PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the read probe failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, READ_PROBE_LIB)
    return READ_PROBE_LIB


PROBE_SRC = os.path.join(ROOT, "tests", "gpu_probes", "probes.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "gpu_probes", "libkvq_probes.so")


def build_probes() -> str:
    """Test-only library of conversion-builtin probes (not part of libkvq)."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc(), *COMMON, "-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the probes failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    build(verbose=True)
    build_read_probe()
    build_probes()
