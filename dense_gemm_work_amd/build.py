"""Compile the gfx950 GEMM library in-tree: ``dense_gemm_work_amd/libdgw_gemm.so``.

Every HIP source is built for gfx950 only, with packed-fp32 instructions
disabled for the device pass (``-Xclang -target-feature -Xclang -packed-fp32-ops``;
the host pass warns that it does not know the feature, which is harmless) and
hardware fp32 atomics enabled (``-munsafe-fp-atomics``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libdgw_gemm.so"
SOURCES = ["gemm_kernels.hip", "gemm_api.hip", "plan.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def command(out: Path) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-munsafe-fp-atomics",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        *[str(CSRC / s) for s in SOURCES],
        "-o", str(out),
    ]


def build(verbose: bool = False) -> Path:
    """Always recompiles (the driver's build check), then atomically replaces the library."""
    tmp = LIB.with_name(LIB.name + f".tmp{os.getpid()}")
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, cwd=str(PKG))
    if res.returncode != 0:
        raise RuntimeError(f"HIP build failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stderr[-8000:]}")
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if verbose and noise:
        print("\n".join(noise[-40:]))
    os.replace(tmp, LIB)
    build_example(verbose)
    return LIB


EXAMPLE_SRC = PKG / "examples" / "gemm_c_api.c"
EXAMPLE_BIN = PKG / "examples" / "gemm_c_api"


def build_example(verbose: bool = False) -> Path:
    """The plain-C usage example, linked against the in-tree library (host code
    only; the platform macro is what the HIP runtime headers ask of C code)."""
    rocm_include = Path(hipcc()).resolve().parent.parent / "include"
    cmd = [hipcc(), "-x", "c", "-O2", "-D__HIP_PLATFORM_AMD__", f"-I{rocm_include}", str(EXAMPLE_SRC), f"-L{PKG}",
           "-ldgw_gemm",
           "-Wl,-rpath,$ORIGIN/..", "-o", str(EXAMPLE_BIN)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, cwd=str(PKG))
    if res.returncode != 0:
        raise RuntimeError(f"example build failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stderr[-4000:]}")
    return EXAMPLE_BIN


def is_stale() -> bool:
    if not LIB.exists():
        return True
    t = LIB.stat().st_mtime
    srcs = [CSRC / s for s in SOURCES] + list(CSRC.glob("*.h")) + [PKG.parent / "include" / "gemm.h"]
    return any(p.stat().st_mtime > t for p in srcs if p.exists())


if __name__ == "__main__":
    print(build(verbose=True))
