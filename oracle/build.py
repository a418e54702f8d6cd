"""Build the fp64 reference GEMM (``ref_gemm.c``) into a shared library with gcc.

Test infrastructure: the library this produces is loaded only by tests, the
smoke check and the benchmark's CPU-baseline leg.

``build(mutation=0)`` compiles the real oracle into ``oracle/_build/``.  A
nonzero ``mutation`` compiles a copy with one planted mistake into a separate
file (used by the tests that prove the pins can fail).
"""
from __future__ import annotations

import os
import subprocess
from pathlib import Path

HERE = Path(__file__).resolve().parent
SRC = HERE / "ref_gemm.c"
OUT_DIR = HERE / "_build"


def lib_path(mutation: int = 0, out_dir: Path | None = None) -> Path:
    d = Path(out_dir) if out_dir is not None else OUT_DIR
    return d / ("libref_gemm.so" if mutation == 0 else f"libref_gemm_mut{mutation}.so")


def build(mutation: int = 0, out_dir: Path | None = None, quiet: bool = True) -> Path:
    out = lib_path(mutation, out_dir)
    out.parent.mkdir(parents=True, exist_ok=True)
    tmp = out.with_suffix(f".so.tmp{os.getpid()}")
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        # keep every product and sum separately rounded, in source order
        "-ffp-contract=off", "-fno-fast-math",
        f"-DORACLE_MUTATION={int(mutation)}",
        str(SRC), "-o", str(tmp), "-lm",
    ]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, out)
    if not quiet:
        print(" ".join(cmd))
    return out


if __name__ == "__main__":
    print(build(quiet=False))
