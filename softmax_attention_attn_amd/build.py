"""Build libattn.so (the gfx950 HIP kernels + C ABI) in the package directory.

    python -m softmax_attention_attn_amd.build

Every source is compiled with hipcc for gfx950 only, with packed-FP32
instruction generation switched off, and linked into one shared library next
to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["attn_api.cpp", "prefill_bf16.hip", "prefill_bf16_band.hip", "prefill_f32.hip", "decode_bf16.hip", "decode_f32.hip", "stream_cache.hip", "backward_bf16.hip", "backward_f32.hip", "socket_bf16.hip", "probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def common_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, build_dir: str, defines: tuple) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    # Kernel sources never produce or test for NaN (masked logits are -inf and every
    # -inf - -inf case is guarded), so max/min need no NaN canonicalisation there.
    # The host API keeps IEEE semantics: it checks scale/gamma with isfinite().
    extra = ["-fno-honor-nans"] if src.endswith(".hip") else []
    cmd = [hipcc()] + common_flags() + extra + [f"-D{d}" for d in defines] + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB, defines: tuple = ()) -> str:
    """Compile every source and link the library (default: libattn.so here); returns its path.

    `defines` are extra preprocessor definitions (NAME or NAME=VALUE), e.g. to pin a kernel
    variant in an A/B build written to another path."""
    build_dir = BUILD_DIR if not defines else BUILD_DIR + "_" + "_".join(d.replace("=", "") for d in defines)
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, tuple(defines)), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
