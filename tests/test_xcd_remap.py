"""The work-group index remaps of the attention and score kernels (common.h: one contiguous
range of logical tiles per XCD, or runs of C tiles per XCD in turn) must be bijections on
[0, n) for every grid size n: a remap that maps two work-groups to one tile would leave another
tile uncomputed, silently. Checked exhaustively on the host (CPU, hipcc), for every grid size
up to 5000 and around the sizes the workloads launch."""
import os
import subprocess

import pytest

from block_sparse_attention_top_amd import build as B

PROG = r"""
#include <stdio.h>
#include <vector>
#include "common.h"
using namespace recap;

template <class F>
static int check(const char* name, F f, int n) {
  std::vector<char> seen(n, 0);
  for (int wg = 0; wg < n; ++wg) {
    const int t = f(wg, n);
    if (t < 0 || t >= n || seen[t]) {
      printf("%s: n=%d wg=%d -> %d is not a bijection\n", name, n, wg, t);
      return 1;
    }
    seen[t] = 1;
  }
  return 0;
}

int main() {
  std::vector<int> sizes;
  for (int n = 1; n <= 5000; ++n) sizes.push_back(n);
  // grids of the workloads: 40 heads x 591 pairs (720p), 24 x 929, 40 x 256, 12 x 256,
  // 40 x 591 dense tiles, and a few large ones
  const int big[] = {23640, 22296, 10240, 3072, 23639, 23641, 65536, 65537, 1 << 20};
  for (int n : big) sizes.push_back(n);
  int bad = 0;
  for (int n : sizes) {
    bad |= check("xcd_remap", [](int w, int m) { return xcd_remap(w, m); }, n);
    bad |= check("xcd_runs<64>", [](int w, int m) { return xcd_runs<64>(w, m); }, n);
    bad |= check("xcd_runs<16>", [](int w, int m) { return xcd_runs<16>(w, m); }, n);
    bad |= check("xcd_runs<8>", [](int w, int m) { return xcd_runs<8>(w, m); }, n);
    bad |= check("xcd_runs<1>", [](int w, int m) { return xcd_runs<1>(w, m); }, n);
  }
  printf(bad ? "FAIL\n" : "OK\n");
  return bad;
}
"""


def test_remaps_are_bijections(tmp_path):
    src = tmp_path / "remap_check.hip"
    src.write_text(PROG)
    exe = tmp_path / "remap_check"
    cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", "-O2", "-std=c++17", f"-I{B.CSRC}",
           str(src), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        pytest.fail(res.stderr[-2000:])
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0 and run.stdout.strip().endswith("OK"), run.stdout[-2000:]
