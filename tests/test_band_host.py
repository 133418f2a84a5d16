"""The interval form of the band mask (Band::key_range / query_range, used
per element by the kernels) agrees with the plain rule (Band::hidden) for
every (row, key) pair over many shapes, offsets and windows.  Host code:
compiled with hipcc, no GPU needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_05_amd", "csrc")

PROGRAM = r"""
#include "fa_internal.hpp"
#include <cstdio>
int main() {
  long bad = 0, checked = 0;
  const int offs[] = {0, 1, -1, 7, -7, 31, -40, 100, -100, 513};
  const int wins[] = {-1, 0, 1, 3, 16, 50, 200};
  for (int n_q : {1, 5, 33, 70})
    for (int n_k : {1, 4, 40, 71})
      for (int off : offs)
        for (int w : wins)
          for (int c = 0; c < 2; ++c) {
            fa::Band b{n_q, n_k, off, w, c == 1};
            for (int q = 0; q < n_q + 3; ++q) {
              int lo, span;
              b.key_range(q, lo, span);
              for (int key = 0; key < n_k + 3; ++key) {
                const bool vis = !b.hidden(q, key);
                if (fa::Band::in_range(key, lo, span) != vis) ++bad;
                ++checked;
              }
            }
            for (int key = 0; key < n_k + 3; ++key) {
              int lo, span;
              b.query_range(key, lo, span);
              for (int q = 0; q < n_q + 3; ++q) {
                const bool vis = q < n_q && !b.hidden(q, key);
                if (fa::Band::in_range(q, lo, span) != vis) ++bad;
                ++checked;
              }
            }
          }
  std::printf("%ld %ld\n", checked, bad);
  return bad != 0;
}
"""


def test_interval_form_matches_the_rule(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    src = tmp_path / "band.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "band"
    r = subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17", f"-I{CSRC}",
                        f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    checked, bad = map(int, out.stdout.split())
    assert checked > 100000 and bad == 0, out.stdout
