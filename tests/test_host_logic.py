"""Host-side logic of the library checked on the CPU (no kernel runs).

* The magic-number division the convolution kernels use to turn a wavefront index into
  (row, tile) and a row into its channel: ``make_fastdiv`` from the kernels' header, compiled
  for the host, must agree with true division for every divisor it can be given and dividends
  up to 2^31 - 1 (checked over all divisors below 4096, powers of two and their neighbours, and
  dividends at the edges and at random).
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_26_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <cstdint>
#include <random>
#include <vector>
#include "msel_kernels.hpp"
static uint32_t div_by(uint32_t n, const msel::FastDiv& f) {
    return static_cast<uint32_t>(((uint64_t(n) * f.m) >> 32) + n) >> f.l;
}
int main() {
    std::mt19937 rng(12345);
    std::vector<uint32_t> ds;
    for (uint32_t d = 1; d < 4096; ++d) ds.push_back(d);
    for (int b = 12; b < 31; ++b) {
        ds.push_back((1u << b) - 1); ds.push_back(1u << b); ds.push_back((1u << b) + 1);
    }
    for (int i = 0; i < 2000; ++i) ds.push_back(1 + rng() % 0x7fffffffu);
    long bad = 0, checked = 0;
    for (uint32_t d : ds) {
        const msel::FastDiv f = msel::make_fastdiv(d);
        uint32_t ns[] = {0, 1, d - 1, d, d + 1, 2 * d - 1, 0x7fffffffu, 0x7ffffffeu,
                         0x7fffffffu - 0x7fffffffu % d, 0x7fffffffu - 0x7fffffffu % d - 1};
        for (uint32_t n : ns) {
            if (n > 0x7fffffffu) continue;
            ++checked; if (div_by(n, f) != n / d) ++bad;
        }
        for (int i = 0; i < 200; ++i) {
            uint32_t n = rng() & 0x7fffffffu;
            ++checked; if (div_by(n, f) != n / d) ++bad;
        }
    }
    std::printf("%ld %ld\n", checked, bad);
    return bad != 0;
}
"""


def test_fastdiv_matches_division(tmp_path):
    src = tmp_path / "fastdiv.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "fastdiv"
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    # host-only build of the header (it includes the HIP runtime header for its types)
    rocm = os.path.dirname(os.path.dirname(hipcc))
    subprocess.run([hipcc, "-std=c++17", "-O2", "-D__HIP_PLATFORM_AMD__", "-I",
                    os.path.join(rocm, "include"), "-I", CSRC, "-x", "c++", str(src), "-o",
                    str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    checked, bad = map(int, out.stdout.split())
    assert checked > 1_000_000 and bad == 0, out.stdout
