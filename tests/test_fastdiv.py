"""The kernels' division by launch constants (dense_gemm_work_amd/csrc/fastdiv.h):
the host's constants, put through the quotient the kernels evaluate in 32-bit
arithmetic, give floor(n / d) for every numerator below 2^31.  Compiled with the
host compiler alone (no GPU, no HIP)."""
import subprocess
from pathlib import Path

ROOT = Path(__file__).resolve().parent.parent

PROGRAM = r"""
#include "fastdiv.h"
#include <cstdio>
#include <cstdint>
#include <initializer_list>

// the kernels' form: (umulhi(n, m') + n) >> s, all in 32 bits
static uint32_t quotient(uint32_t n, dgw::FastDiv f) {
    const uint32_t hi = (uint32_t)(((uint64_t)n * f.m) >> 32);
    return (hi + n) >> f.s;
}

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next31() {   // splitmix64, top 31 bits
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) >> 33);
}

static long bad = 0, checked = 0;
static void check(uint32_t n, uint32_t d, dgw::FastDiv f) {
    ++checked;
    if (quotient(n, f) != n / d && bad++ < 5) std::printf("d=%u n=%u: %u, not %u\n", d, n, quotient(n, f), n / d);
}

int main() {
    const uint32_t top = 0x7FFFFFFFu;
    // every divisor up to 2048: every numerator below 2^15, the last 2^12 below
    // 2^31 and the multiples of d (and their neighbours) below 2^31 sampled
    for (uint32_t d = 1; d <= 2048; ++d) {
        const dgw::FastDiv f = dgw::fast_div(d);
        for (uint32_t n = 0; n < (1u << 15); ++n) check(n, d, f);
        for (uint32_t n = top - 4095; n <= top && n >= top - 4095; ++n) check(n, d, f);
        for (int i = 0; i < 256; ++i) {
            const uint32_t k = next31() / d;
            for (int e = -1; e <= 1; ++e) {
                const int64_t n = (int64_t)k * d + e;
                if (n >= 0 && n <= top) check((uint32_t)n, d, f);
            }
        }
    }
    // divisors across the whole range (powers of two and their neighbours
    // included), each with random numerators, multiples and the largest index
    for (int i = 0; i < 200000; ++i) {
        uint32_t d;
        if (i < 31 * 3) {
            const int p = i / 3;
            d = (uint32_t)((1ull << p) + (i % 3) - 1);
            if (d == 0) d = 1;
        } else {
            d = next31() >> (next31() % 31);
            if (d == 0) d = 1;
        }
        const dgw::FastDiv f = dgw::fast_div(d);
        check(top, d, f);
        check(next31(), d, f);
        const uint32_t k = next31() / d;
        for (int e = -1; e <= 1; ++e) {
            const int64_t n = (int64_t)k * d + e;
            if (n >= 0 && n <= top) check((uint32_t)n, d, f);
        }
    }
    // d = 2^31, the largest divisor
    const dgw::FastDiv f = dgw::fast_div(int64_t(1) << 31);
    for (uint32_t n : {0u, 1u, top - 1, top}) check(n, 0x80000000u, f);
    // a divisor below 1 is taken as 1
    const dgw::FastDiv one = dgw::fast_div(0);
    for (uint32_t n : {0u, 7u, top}) check(n, 1u, one);
    std::printf("checked %ld, wrong %ld\n", checked, bad);
    return bad != 0;
}
"""


def test_fast_division_is_exact(tmp_path):
    src = tmp_path / "fastdiv_check.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "fastdiv_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", str(ROOT / "dense_gemm_work_amd" / "csrc"), str(src), "-o",
                    str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "wrong 0" in out.stdout


def test_the_check_catches_a_wrong_constant(tmp_path):
    # the same program with the rounding of m taken down instead of up must fail
    src = tmp_path / "fastdiv_bad.cpp"
    header = (ROOT / "dense_gemm_work_amd" / "csrc" / "fastdiv.h").read_text()
    planted = header.replace("+ uint64_t(d) - 1) / uint64_t(d)", ") / uint64_t(d)")
    assert planted != header
    (tmp_path / "fastdiv.h").write_text(planted)
    src.write_text(PROGRAM)
    exe = tmp_path / "fastdiv_bad"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", str(tmp_path), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode != 0
