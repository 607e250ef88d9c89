"""The kernels' division by invariant integers (csrc/gdn_divide.hpp: the
round-up method of Granlund and Montgomery, "Division by Invariant Integers
using Multiplication", PLDI 1994) against the native division, on the CPU:
every dividend below 3000 and near multiples of the divisor for every divisor
up to 5000, the extreme dividends, divisors near powers of two and near 2^32,
and random pairs. The workgroup-id decode of verify, commit and the native
copy divides by the head and row counts this way."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_deltanet_speculative_gdn_amd", "csrc")

CHECK = r"""
#include "gdn_divide.hpp"
#include <cstdio>
#include <random>
static unsigned long long n = 0;
static bool check(uint32_t x, uint32_t d, gdn::Divider v) {
    ++n;
    if (gdn::udiv(x, v) == x / d) return true;
    std::printf("x=%u d=%u: %u instead of %u\n", x, d, gdn::udiv(x, v), x / d);
    return false;
}
int main() {
    std::mt19937_64 g(20260);
    for (uint32_t d = 1; d <= 5000; ++d) {
        const gdn::Divider v = gdn::make_divider(d);
        for (uint32_t x = 0; x < 3000; ++x) if (!check(x, d, v)) return 1;
        for (int k = 0; k < 64; ++k) {
            const unsigned long long x = (unsigned long long)d * (g() % 800000);
            for (int o = -1; o <= 1; ++o)
                if (x + o < (1ull << 32) && !check((uint32_t)(x + o), d, v)) return 1;
        }
        if (!check(0xffffffffu, d, v) || !check(0xfffffffeu, d, v) || !check(1u << 31, d, v)) return 1;
    }
    const uint32_t ds[] = {1u, 2u, 3u, 7u, 4095u, 4096u, 4097u, 65535u, 65536u, 65537u,
                           0x7fffffffu, 0x80000000u, 0x80000001u, 0xfffffffeu, 0xffffffffu};
    for (uint32_t d : ds) {
        const gdn::Divider v = gdn::make_divider(d);
        for (int i = 0; i < 20000; ++i) if (!check((uint32_t)g(), d, v)) return 1;
        if (!check(0xffffffffu, d, v) || !check(0u, d, v) || !check(d, d, v)) return 1;
    }
    for (int i = 0; i < 500000; ++i) {
        uint32_t d = (uint32_t)(g() >> (g() % 63));
        if (d == 0) d = 1;
        if (!check((uint32_t)g(), d, gdn::make_divider(d))) return 1;
    }
    if (gdn::udiv(12345u, gdn::make_divider(0)) != 12345u) return 1;   // 0 is taken as 1
    std::printf("%llu divisions exact\n", n);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_invariant_division_is_exact(tmp_path):
    src = tmp_path / "check.cpp"
    src.write_text(CHECK)
    exe = tmp_path / "check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "divisions exact" in r.stdout
