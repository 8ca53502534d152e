"""The attention kernels' workgroup order (`xcd_work_order` in csrc/lcsa_geom.h) must be a permutation
of the workgroups for every size, or query blocks would be skipped or computed twice. Compiled for the
host with g++ and checked over many grid sizes, blocks per head and both walk directions."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_causal_lcsa_amd", "csrc")

PROGRAM = r"""
#include "lcsa_geom.h"
#include <stdio.h>
#include <vector>
int main() {
  long bad = 0, cases = 0;
  const int nqbs[] = {1, 2, 3, 5, 7, 64, 65, 66, 252, 264, 858};
  for (int nrows = 1; nrows <= 1200; ++nrows)
    for (int rpw = 1; rpw <= 2; ++rpw)
      for (int nqb : nqbs)
        for (int desc = 0; desc < 2; ++desc) {
          const int nwg = (nrows + rpw - 1) / rpw;
          std::vector<int> seen(nwg, 0);
          for (int n = 0; n < nwg; ++n) {
            const int w = lcsa::xcd_work_order(n, nwg, rpw, nqb, desc != 0);
            if (w < 0 || w >= nwg || seen[w]++) { ++bad; break; }
          }
          ++cases;
        }
  // the 768x1408 chunk (12 heads x 66 query blocks, two per workgroup, 49.5 workgroups per XCD):
  // at least 31 of every XCD's first 32 workgroups come from the head of its first one
  const int nwg = 396, nqb = 66;
  for (int x = 0; x < 8; ++x) {
    const int h = (2 * lcsa::xcd_work_order(x, nwg, 2, nqb, false)) / nqb;
    int same = 0;
    for (int l = 0; l < 32; ++l) same += (2 * lcsa::xcd_work_order(8 * l + x, nwg, 2, nqb, false)) / nqb == h;
    if (same < 31) ++bad;
  }
  printf("%ld cases, %ld failures\n", cases, bad);
  return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_work_order_is_a_permutation(tmp_path):
    src = tmp_path / "order.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "order"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
