"""The decode's XCD-aware launch order (csrc/xcd_order.hpp), on the CPU.

The launch order is a scheduling choice of this library, not a step of the
pages' method: it must hand every work unit to exactly one workgroup, keep
each XCD's units in the schedule's order (longest first), and give the odd
XCDs 10 units for every 11 on the even ones.  The header's functions use no
HIP API, so a host build of it is checked here with g++.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR_DIR = os.path.join(ROOT, "paged_kv_cache_write_amd", "csrc")

PROGRAM = r'''
#include "xcd_order.hpp"
#include <cstdio>
#include <vector>
using namespace pa;
int main() {
  long bad_bijection = 0, bad_order = 0, bad_positions = 0;
  long even_units = 0, odd_units = 0;
  const int sizes[] = {1, 2, 7, 8, 9, 15, 16, 17, 83, 84, 85, 167, 168, 169, 1000, 2040, 4060,
                       12720, 123457};
  for (int offset = 0; offset < 16; ++offset) {
    for (int N : sizes) {
      const long P = xcd_order_positions(N, offset);
      std::vector<int> seen(N, 0);
      std::vector<int> last(8, -1);
      long maxpos = -1;
      for (long p = 0; p < P + 64; ++p) {
        const int u = xcd_order_unit(int(p), offset);
        if (u < 0) { ++bad_bijection; continue; }
        if (u >= N) continue;
        if (p >= P) { ++bad_positions; continue; }
        if (seen[u]++) ++bad_bijection;
        if (xcd_order_position(u, offset) != p) ++bad_bijection;
        const int x = int((offset + p) % 8);
        if (u <= last[x]) ++bad_order;   // each XCD takes its units in order
        last[x] = u;
        maxpos = p > maxpos ? p : maxpos;
        if (N == 123457 && offset == 0) { if (x % 2) ++odd_units; else ++even_units; }
      }
      for (int u = 0; u < N; ++u) if (!seen[u]) ++bad_bijection;
      if (maxpos + 1 != P) ++bad_positions;
    }
  }
  printf("%ld %ld %ld %ld %ld\n", bad_bijection, bad_order, bad_positions, even_units, odd_units);
  return 0;
}
'''


@pytest.fixture(scope="module")
def order_run(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    d = tmp_path_factory.mktemp("xcd_order")
    src, exe = d / "t.cpp", d / "t"
    src.write_text(PROGRAM)
    subprocess.run([gxx, "-O2", "-std=c++17", "-D__host__=", "-D__device__=", "-I", HDR_DIR,
                    str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    return [int(x) for x in out]


def test_every_unit_once(order_run):
    """Every unit runs on exactly one workgroup, for 16 region offsets and sizes
    from 1 to 123457, and position and unit invert each other."""
    assert order_run[0] == 0


def test_each_xcd_keeps_the_schedule_order(order_run):
    """On each XCD the units come in increasing index (the schedule lists them
    longest first), so a launch of several rounds starts with its longest work."""
    assert order_run[1] == 0


def test_position_count_is_tight(order_run):
    """The launch size (positions) ends at the last unit's position: no unit is
    placed past it and no trailing position is empty."""
    assert order_run[2] == 0


def test_odd_xcds_take_ten_for_eleven(order_run):
    """Over a long launch the odd XCDs take 10 units for every 11 on the even ones."""
    even, odd = order_run[3], order_run[4]
    assert abs(odd / even - 10 / 11) < 1e-3
