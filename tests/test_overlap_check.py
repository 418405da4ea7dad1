"""Host-side check of the carry overlap test that decides when the prefill copies its carry in to
the workspace before the main kernel (ccq_overlap.hpp), compiled with g++ on the CPU.

With more than one segment per chain, segment 0 reads the caller's carry in while the chain's
last segment writes the carry out in the same launch; any overlap between the two must be seen.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "curvature_conditioned_query_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include <cstdint>
#include "ccq_overlap.hpp"
using ccq::CarryRanges;
static char buf[1 << 24];
int main() {
  const size_t chains = 4, d = 64;
  const size_t S = chains * d * d * 4, C = chains * d * d * 4, Cp = chains * d * (d + 1) / 2 * 4;
  const size_t m = chains * d * 4, n = chains * 8;
  char* p = buf;
  // carry in laid out back to back, carry out after it
  CarryRanges in{p, p + S, p + S + C, p + S + C + m};
  char* q = p + S + C + m + n;
  CarryRanges out{q, q + S, q + S + C, q + S + C + m};
  printf("%d\n", (int)ccq::carry_ranges_overlap(in, out, chains, d, false));          // 0 disjoint
  printf("%d\n", (int)ccq::carry_ranges_overlap(in, in, chains, d, false));           // 1 alias
  CarryRanges sh{p + 4, q + S, q + S + C, q + S + C + m};                              // S out shifted into S in
  printf("%d\n", (int)ccq::carry_ranges_overlap(in, sh, chains, d, false));           // 1
  CarryRanges nn{q, q + S, q + S + C, p + S + C + m + n - 8};                          // n out = last n in
  printf("%d\n", (int)ccq::carry_ranges_overlap(in, nn, chains, d, false));           // 1
  CarryRanges touch{p + S + C + m + n, q + S, q + S + C, q + S + C + m};               // S out starts where n in ends
  printf("%d\n", (int)ccq::carry_ranges_overlap(in, touch, chains, d, false));        // 0
  // C out starts right after a packed C in, inside a full one; everything else far apart
  char* far = p + (1 << 22);
  CarryRanges in2{p, p + S, p + (1 << 23), p + (1 << 23) + m};
  CarryRanges cx{far, p + S + Cp, far + S + C, far + S + C + m};
  printf("%d\n", (int)ccq::carry_ranges_overlap(in2, cx, chains, d, true));           // 0 packed
  printf("%d\n", (int)ccq::carry_ranges_overlap(in2, cx, chains, d, false));          // 1 full
  CarryRanges none{nullptr, nullptr, nullptr, nullptr};
  printf("%d\n", (int)ccq::carry_ranges_overlap(none, in, chains, d, false));         // 0 no carry in
  printf("%d\n", (int)ccq::carry_ranges_overlap(in, none, chains, d, false));         // 0 no carry out
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_carry_overlap_cases(tmp_path):
    src = tmp_path / "overlap.cpp"
    exe = tmp_path / "overlap"
    src.write_text(DRIVER)
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    assert out == ["0", "1", "1", "1", "0", "0", "1", "0", "0"]
