"""The plan-time division helper of the fast kernel (make_fastdiv_u31 / fastdiv_u31 in
fused_proj_kernels.h), checked on the CPU: a host program built from the header divides
by many divisors (all small ones, powers of two and their neighbours, the largest, random
ones) and compares every quotient with the hardware division. The dividends cover the
edges of each quotient step, the largest dividend 2^31 - 1 and random values; small
divisors are checked on every dividend below 2^20."""
import os
import subprocess

from ff_input_projection_amd import build as fpbuild

PROGRAM = r"""
#include "fused_proj_kernels.h"
#include <cstdio>
#include <cstdint>
#include <vector>

static uint64_t state = 0x9e3779b97f4a7c15ull;
static uint32_t rnd31() {   // splitmix64, top 31 bits
    uint64_t z = (state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return (uint32_t)((z ^ (z >> 31)) >> 33);
}

int main() {
    const uint32_t nmax = 0x7fffffffu;
    std::vector<uint32_t> ds;
    for (uint32_t d = 1; d <= 4096; ++d) ds.push_back(d);
    for (int k = 1; k <= 31; ++k) {
        const uint64_t p = uint64_t(1) << k;
        for (int64_t e = -1; e <= 1; ++e)
            if (p + e >= 1 && p + e <= nmax) ds.push_back((uint32_t)(p + e));
    }
    for (int i = 0; i < 20000; ++i) ds.push_back(rnd31() | 1u);
    long long checks = 0, bad = 0;
    for (uint32_t d : ds) {
        const fp::FastDivU31 f = fp::make_fastdiv_u31(d);
        std::vector<uint32_t> ns = {0u, 1u, nmax, nmax - 1u};
        for (uint64_t k : {uint64_t(1), uint64_t(2), uint64_t(3), uint64_t(nmax / d), uint64_t(nmax / d / 2 + 1)}) {
            for (int64_t e = -1; e <= 1; ++e) {
                const int64_t n = (int64_t)(k * d) + e;
                if (n >= 0 && n <= nmax) ns.push_back((uint32_t)n);
            }
        }
        for (int i = 0; i < 64; ++i) ns.push_back(rnd31());
        if (d <= 64)
            for (uint32_t n = 0; n < (1u << 20); ++n) ns.push_back(n);
        for (uint32_t n : ns) {
            ++checks;
            if (fp::fastdiv_u31(n, f) != n / d) {
                if (bad < 10) std::printf("MISMATCH d=%u n=%u got=%u want=%u\n", d, n, fp::fastdiv_u31(n, f), n / d);
                ++bad;
            }
        }
    }
    std::printf("checks=%lld bad=%lld divisors=%zu\n", checks, bad, ds.size());
    return bad != 0;
}
"""


def test_fastdiv_matches_integer_division(tmp_path):
    src = os.path.join(tmp_path, "fastdiv.cpp")
    exe = os.path.join(tmp_path, "fastdiv")
    with open(src, "w") as f:
        f.write(PROGRAM)
    # host code only: the header's __host__ __device__ helpers compile for the CPU and the
    # program makes no HIP runtime call
    cmd = [fpbuild.HIPCC, "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", "-I", fpbuild.CSRC, src, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "bad=0" in r.stdout
