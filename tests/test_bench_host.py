"""Host-side contract of bench.py (no GPU): the one-GPU refusal, the comment-
insensitive kernel code digest, and the gating of the measured HBM traffic on
that digest."""
import json
import subprocess
import sys
from pathlib import Path

import bench

ROOT = Path(__file__).resolve().parent.parent


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=str(ROOT), timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line is printed


def test_code_digest_ignores_comments_only(tmp_path):
    src = "int f(int x) {\n    return x + 1;   // one more\n}\n/* a block\n   comment */\n"
    a = tmp_path / "a.hip"
    a.write_text(src)
    b = tmp_path / "b.hip"
    b.write_text("// a new header line\n" + src.replace("// one more", "// changed note").replace("    ", "\t"))
    c = tmp_path / "c.hip"
    c.write_text(src.replace("x + 1", "x + 2"))
    assert bench.kernel_code_digest(a) == bench.kernel_code_digest(b)
    assert bench.kernel_code_digest(a) != bench.kernel_code_digest(c)


def test_traffic_is_reported_only_for_the_profiled_code(monkeypatch):
    entries = json.loads((ROOT / "profiles" / "traffic.json").read_text())
    name, entry = next(iter(entries.items()))
    monkeypatch.setattr(bench, "kernel_code_digest", lambda path=None: entry["code_sha256"])
    assert bench.measured_traffic(name) == int(entry["bytes"])
    assert bench.measured_traffic("no_such_profile") is None
    monkeypatch.setattr(bench, "kernel_code_digest", lambda path=None: "0" * 64)
    assert bench.measured_traffic(name) is None


def test_profile_key_names_the_launch():
    class P:   # the plan fields profile_key reads
        decision, atomic, bm, bn, tiles_m, tiles_n, tiles = 3, 0, 128, 128, 16, 17, 272

    class DG:
        GEMM_DP, GEMM_SPLITK, GEMM_STREAMK = 1, 2, 3

        @staticmethod
        def gemm_num_cus():
            return 256

    from workloads import WORKLOADS
    w = WORKLOADS["c3_wavequant"]
    assert bench.profile_key(DG, P, w) == "gemm_streamk_bf16_kn_2048x2176x4096"
    P.bm = 256
    assert bench.profile_key(DG, P, w) == "gemm_streamk_bf16_kn_2048x2176x4096_256x128"


    # a grouped launch: the key of the committed grouped profile
    from workloads import GROUPED
    P.bm = 128
    key = bench.grouped_profile_key(DG, P, GROUPED["x4_grouped"])
    assert key == "gemm_streamk_grouped_bf16_nk_8_problems_2048x2048x4096"
    assert (ROOT / "profiles" / (key + ".md")).exists()


def test_compulsory_bytes():
    import bench
    from workloads import WORKLOADS

    w = WORKLOADS["c2a_m96_s8"]
    assert bench.compulsory_bytes(w) == 96 * 2048 * 2 + 2048 * 512 * 2 + 96 * 512 * 4
    x2 = WORKLOADS["x2_batched"]
    assert bench.compulsory_bytes(x2) == 5 * (1024 * 2048 * 2 * 2 + 1024 * 1024 * 4)
