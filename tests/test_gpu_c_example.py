"""The plain-C usage example (dense_gemm_work_amd/examples/gemm_c_api.c, built
by the package build) runs on the GPU in a process of its own: the C ABI with
device buffers from the HIP runtime only, no Python and no torch."""
import subprocess
from pathlib import Path

import pytest

pytestmark = pytest.mark.gpu

EXAMPLE = Path(__file__).resolve().parent.parent / "dense_gemm_work_amd" / "examples" / "gemm_c_api"


def test_c_example_runs():
    assert EXAMPLE.exists(), f"{EXAMPLE} is not built (the package build makes it)"
    out = subprocess.run([str(EXAMPLE)], capture_output=True, text=True, timeout=120)
    print(out.stdout, out.stderr[-2000:], flush=True)
    assert out.returncode == 0
    assert out.stdout.strip().splitlines()[-1] == "ok"
