"""The tile scheduler's division by invariant counts (a multiply-high and
two shifts, the constants prepared on the host) against plain integer
division, over every numerator a launch can give it (program ids below
2^31): all divisors up to 5000 and those around each power of two and at
the top of the range, each at its edge numerators and random ones, and
every numerator for a few divisors.  The header is compiled host-only with
g++, the same source the kernels include."""
import os
import subprocess
import tempfile

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "dense_gemm_10_amd", "csrc")

CHECK = r'''
#include <stdio.h>
#include <stdint.h>
#include <random>
#include <vector>
#include "scheduler.hpp"
using namespace dg;

static long bad = 0;
static void check(uint32_t n, uint32_t d, const FastDiv &f)
{
    if (fastdiv(n, f) != n / d && bad++ < 10)
        printf("FAIL n=%u d=%u got %u want %u\n", n, d, fastdiv(n, f), n / d);
}

int main()
{
    const uint32_t top = 0x7fffffffu;               // largest program id + 1
    std::mt19937 rng(12345);
    std::vector<uint32_t> divs;
    for (uint32_t d = 1; d <= 5000; ++d)
        divs.push_back(d);
    for (int k = 1; k <= 31; ++k) {
        const uint64_t p = 1ull << k;
        for (int64_t e = -3; e <= 3; ++e)
            if ((int64_t)p + e >= 1 && (uint64_t)((int64_t)p + e) <= top)
                divs.push_back((uint32_t)((int64_t)p + e));
    }
    for (int i = 0; i < 2000; ++i)
        divs.push_back(1 + rng() % top);
    long cases = 0;
    for (uint32_t d : divs) {
        const FastDiv f = fastdiv_make(d);
        std::vector<uint32_t> ns = {0, 1, 2, top - 1, top - 2, top - d % top};
        for (uint64_t k : {(uint64_t)1, (uint64_t)2, (uint64_t)3, (uint64_t)1000, (uint64_t)(top / d)})
            for (int64_t e = -1; e <= 1; ++e) {
                const int64_t n = (int64_t)(k * d) + e;
                if (n >= 0 && n < top)
                    ns.push_back((uint32_t)n);
            }
        for (int i = 0; i < 300; ++i)
            ns.push_back(rng() % top);
        for (uint32_t n : ns) {
            check(n, d, f);
            ++cases;
        }
    }
    // every numerator for divisors of each kind (7 and 641 need the
    // shift-and-add form; 3 * 5 * 17 * 257 = 65535; 136 = 8 x 17 tiles, a
    // band of the tile grid)
    for (uint32_t d : {7u, 641u, 65535u, 136u}) {
        const FastDiv f = fastdiv_make(d);
        for (uint32_t n = 0; n < top; ++n)
            check(n, d, f);
        cases += top;
    }
    printf("%ld cases, %ld failures\n", cases, bad);
    return bad != 0;
}
'''


def test_fastdiv_matches_integer_division():
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "check.cpp")
        exe = os.path.join(tmp, "check")
        with open(src, "w") as fh:
            fh.write(CHECK)
        r = subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, src, "-o", exe],
                           capture_output=True, text=True)
        if r.returncode != 0:
            pytest.fail(r.stderr[-3000:])
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stdout[-3000:]
        assert " 0 failures" in r.stdout
