"""Build liblinattn.so (HIP, gfx950) in-tree with hipcc.

Every source is compiled for gfx950 only, with packed-fp32 instructions
disabled, and linked into ``kernelized_linear_attention_la_amd/_lib/liblinattn.so``.
Only the ``la_*`` C entry points are exported.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_DIR = os.path.join(PKG, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "liblinattn.so")
SOURCES = ["la_api.hip", "la_generic.hip", "la_decode.hip", "la_mfma.hip", "la_mfma_seg.hip", "la_backward.hip", "la_backward_mfma.hip",
           "la_gated.hip", "la_gla_chunk.hip", "la_favor.hip", "la_delta_chunk.hip", "la_f32mma.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblinattn)")


def compile_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + compile_flags() + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def device_asm(src: str, extra=()) -> str:
    """The gfx950 assembly text of one source, compiled with the library's flags."""
    cmd = [hipcc()] + compile_flags() + list(extra) + ["--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{' '.join(cmd)}\n{r.stderr}")
    return r.stdout


def build(extra_flags=(), verbose: bool = False) -> str:
    """Compile all sources and link liblinattn.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra_flags), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH



# The sources that decide each kernel family's code and launch plan: its own
# file, the shared device helpers and argument structs, and the host code that
# sizes its grid and segments.
KERNEL_SOURCES = {
    "k_mfma": ("la_mfma.hip", "la_mfma_ops.h", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_favor": ("la_favor.hip", "la_mfma_ops.h", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_seg": ("la_mfma_seg.hip", "la_mfma_ops.h", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_generic": ("la_generic.hip", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_f32mma": ("la_f32mma.hip", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_scan": ("la_generic.hip", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_decode": ("la_decode.hip", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_bwd_dq": ("la_backward.hip", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_bwd_rscan": ("la_backward.hip", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_bwd_dkv": ("la_backward.hip", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_delta_prep": ("la_delta_chunk.hip", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_delta_scan": ("la_delta_chunk.hip", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_delta_out": ("la_delta_chunk.hip", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_gated": ("la_gated.hip", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_gla_chunk": ("la_gla_chunk.hip", "la_gated.hip", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_gla_prep": ("la_gla_chunk.hip", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_gla_chain": ("la_gla_chunk.hip", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_gla_out": ("la_gla_chunk.hip", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_bwd_dq_mfma": ("la_backward_mfma.hip", "la_device.h", "la_internal.h", "la_api.hip"),
    "k_bwd_dkv_mfma": ("la_backward_mfma.hip", "la_device.h", "la_internal.h", "la_api.hip"),
}


def source_hash(kernel: str | None = None) -> str:
    """sha256 over the HIP sources behind one kernel family (all sources when
    `kernel` is None or not a known family); identifies a kernel build."""
    import hashlib
    h = hashlib.sha256()
    fam = None if kernel is None else kernel.split("<")[0]
    if fam in KERNEL_SOURCES:
        files = sorted(KERNEL_SOURCES[fam])
    else:
        files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))
    for f in files:
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    if fam not in KERNEL_SOURCES:
        with open(os.path.join(INCLUDE, "liblinattn.h"), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    build(sys.argv[1:], verbose=True)
