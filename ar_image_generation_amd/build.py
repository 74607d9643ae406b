"""Builds libdiagattn.so (HIP for gfx950) in-tree with hipcc.

    python -m ar_image_generation_amd.build
    python -m ar_image_generation_amd.build --host-asan DIR

Every call recompiles all sources; objects go to ``_build/`` next to this
file and the shared library to ``libdiagattn.so`` beside it.  With
``--host-asan DIR`` the library is built into DIR instead, its host code
(argument checks, sizing, the batch schedule, the residency tables)
instrumented with AddressSanitizer and the device code unchanged; run the
CPU tests against it with ``DIAGATTN_LIB=DIR/libdiagattn.so`` and the
sanitizer runtime preloaded (``LD_PRELOAD``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdiagattn.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "keepset.hip", "decode.hip", "probe.hip", "prefill.hip", "residency.hip",
           "schedule.hip"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    # the first kernel arguments arrive preloaded in SGPRs (gfx950 kernel-
    # argument preloading); kernels read the rest from the argument block
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libdiagattn)")


# Per-source additions.  decode.hip: matrix-core accumulators in ordinary
# VGPRs (the decode kernel rescales them with vector instructions; held in
# AGPRs they were copied back and forth every block and took a wave a SIMD).
EXTRA_FLAGS = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


# host-only AddressSanitizer: each -fsanitize= applies to the host pass alone
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def build(verbose: bool = False, host_asan_dir: str = None) -> str:
    out_dir, lib = (BUILD, LIB) if host_asan_dir is None else (host_asan_dir, os.path.join(host_asan_dir, "libdiagattn.so"))
    os.makedirs(out_dir, exist_ok=True)
    extra = [] if host_asan_dir is None else ["-O1", "-g"] + HOST_ASAN

    def comp(src):
        if host_asan_dir is None:
            return _compile(src)
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *[f for f in FLAGS if f != "-O3"], *extra, *EXTRA_FLAGS.get(src, []), "-c",
               os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(comp, SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *([] if host_asan_dir is None else HOST_ASAN[:2]),
           *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--host-asan":
        build(verbose=True, host_asan_dir=os.path.abspath(sys.argv[2]))
    else:
        build(verbose=True)
    sys.exit(0)
