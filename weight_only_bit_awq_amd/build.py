"""Builds the gfx950 HIP library ``libawq_mi355x.so`` in-tree with hipcc.

Usage: ``python -m weight_only_bit_awq_amd.build`` (or ``__graft_entry__.build()``).
Every source is compiled for gfx950 only; packed-fp32 instruction selection is
disabled (its forms are avoided on this target) and no fast-math flag is used,
so fp16 subnormals and IEEE rounding are kept.
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
LIB_NAME = "libawq_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["awq_api.cpp", "awq_pack.hip", "awq_decode.hip", "awq_prefill.hip", "awq_probe.hip", "awq_quant.hip",
           "awq_attention.hip", "awq_w4a8.hip"]

ARCH = "gfx950"
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc",
    # code object v5: loadable by the HIP runtime PyTorch ships as well as ROCm 7.2's
    "-mcode-object-version=5",
]
# Per-source device flags. The decode kernels keep their MFMA results in
# ordinary VGPRs instead of accumulation registers: the per-group scale is
# applied to every group's result right after its MFMAs, so accumulation
# registers only add a move per result register (four per 128-row band and
# column tile) and registers (the staged kernel with four waves, as run on
# the one-row gate+up layer: 72 -> 66; the streamed kernel for 16 and 32
# rows with four tiles: 160 -> 138 and 244 -> 190). The instructions are
# otherwise the same, and so are the results, bit for bit. The prefill GEMMs
# hold 256x256 fp32 accumulator tiles and need the accumulation registers.
SOURCE_FLAGS = {
    "awq_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build the library")
    return path


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON_FLAGS
    if src.endswith(".hip"):
        cmd += DEVICE_FLAGS + SOURCE_FLAGS.get(src, []) + ["-x", "hip"]
    else:
        cmd += ["-D__HIP_PLATFORM_AMD__"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    # the host pass of hipcc does not know the packed-fp32 feature: drop that note
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l and l.strip())
    if err and verbose:
        print(err, file=sys.stderr)
    return obj


def _check_no_undefined_kernels(lib: str) -> None:
    """The host pass of hipcc can drop a kernel's launch stub without an error
    (a diagnostic it defers inside a template); the library then links but
    cannot be loaded. Catch that here, naming the missing symbols."""
    nm = shutil.which("nm") or shutil.which("llvm-nm") or "/opt/rocm/llvm/bin/llvm-nm"
    res = subprocess.run([nm, "-D", "--undefined-only", lib], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"nm failed on {lib}:\n{res.stderr}")
    missing = [l.split()[-1] for l in res.stdout.splitlines() if "_ZN3awq" in l]
    if missing:
        raise RuntimeError("library has undefined kernel symbols (host stub not emitted):\n" + "\n".join(missing))


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source for gfx950 and link ``libawq_mi355x.so`` next to
    this file. Always recompiles. Returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fno-gpu-rdc", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking {LIB_NAME} failed:\n{res.stdout}\n{res.stderr}")
    _check_no_undefined_kernels(tmp)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
