"""Build the gfx950 HIP library ``libpagedattn.so`` in-tree with hipcc.

Every kernel source is compiled for gfx950 only. Packed FP32 instructions are
disabled in the device pass (``-Xclang -target-feature -Xclang
-packed-fp32-ops``); hipcc's host pass warns that it does not know the feature.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD_DIR = PKG / "_build"
LIB_PATH = PKG / "libpagedattn.so"
SOURCES = ["api.hip", "kv_append.hip", "decode.hip", "decode_mfma.hip", "decode_quant.hip", "decode_multi.hip", "prefill.hip", "attn_f32.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMPILE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", str(ROOT / "include"), "-I", str(CSRC),
]


def _compile(src: str) -> Path:
    obj = BUILD_DIR / (Path(src).stem + ".o")
    cmd = [HIPCC, *COMPILE_FLAGS, "-c", str(CSRC / src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> Path:
    """Compile every source and link the shared library; always rebuilds."""
    BUILD_DIR.mkdir(exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH.with_suffix(".so.tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
