"""LDS tile addressing (fa_tiles.hpp) checked on the host: the per-lane XOR
form of TileLane gives the same byte offsets as the swizzled Tile::offset for
every lane, row block, chunk and head dimension; offsets stay inside the tile
and the swizzle is a permutation of each row's 16-byte chunks; the direct
copies of 2, 4 or 8 waves put every 16-byte chunk where the offsets say; and the two
operand reads are free of LDS bank conflicts (16 lanes of a row read cover 16
distinct 16-byte bank groups, 32 lanes of a transposing read 32 distinct
8-byte bank pairs).  Compiled with hipcc, no GPU needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_05_amd", "csrc")

PROGRAM = r"""
#include "fa_tiles.hpp"
#include <cstdio>
#include <set>

static long bad = 0, checked = 0;
#define EXPECT(c) do { ++checked; if (!(c)) { if (bad < 10) std::printf("fail: %s (D=%d ROWS=%d)\n", #c, D, ROWS); ++bad; } } while (0)

template <int D, int ROWS>
void check() {
  using T = fa::Tile<D, ROWS>;
  // the swizzle permutes each row's chunks; offsets tile the buffer exactly
  std::set<int> all;
  for (int r = 0; r < ROWS; ++r) {
    std::set<int> row;
    for (int c = 0; c < T::kChunks; ++c) {
      const int o = T::offset(r, c);
      EXPECT(o >= r * T::kRowBytes && o < (r + 1) * T::kRowBytes && o % 16 == 0);
      row.insert(o);
      all.insert(o);
    }
    EXPECT((int)row.size() == T::kChunks);
  }
  EXPECT((int)all.size() == ROWS * T::kChunks);
  for (int lane = 0; lane < 64; ++lane) {
    fa::TileLane<D, ROWS> tl;
    tl.init(lane);
    for (int row0 = 0; row0 < ROWS; row0 += 32)
      for (int c = 0; c < D / 16; ++c) {
        const int o = T::rows_offset(row0, c, lane);
        EXPECT(tl.rows_at(row0, c) == o);
        EXPECT(o >= 0 && o + 16 <= T::kBytes && o % 16 == 0);
      }
    for (int r0 = 0; r0 < ROWS; r0 += 16)
      for (int col0 = 0; col0 < D; col0 += 32)
        for (int half = 0; half < 2; ++half) {
          const int o = T::tr_offset(r0, col0, lane, half);
          EXPECT(tl.tr_at(r0, col0, half) == o);
          EXPECT(o >= 0 && o + 8 <= T::kBytes && o % 8 == 0);
        }
  }
  // bank groups: a 16-byte access covers banks 4k..4k+3 with k = (addr/16) % 16
  for (int row0 = 0; row0 < ROWS; row0 += 32)
    for (int c = 0; c < D / 16; ++c)
      for (int g = 0; g < 4; ++g) {
        std::set<int> banks;
        for (int lane = 16 * g; lane < 16 * g + 16; ++lane) banks.insert((T::rows_offset(row0, c, lane) / 16) % 16);
        EXPECT(banks.size() == 16);
      }
  // an 8-byte access covers banks 2k, 2k+1 with k = (addr/8) % 32
  for (int r0 = 0; r0 < ROWS; r0 += 16)
    for (int col0 = 0; col0 < D; col0 += 32)
      for (int half = 0; half < 2; ++half)
        for (int g = 0; g < 2; ++g) {
          std::set<int> banks;
          for (int lane = 32 * g; lane < 32 * g + 32; ++lane) banks.insert((T::tr_offset(r0, col0, lane, half) / 8) % 32);
          EXPECT(banks.size() == 32);
        }
}

// Direct tile copies: the 16 bytes a lane's copy i fetches (row, chunk) land
// at the byte the lane writes (KiB block L, lane position), which must be
// Tile::offset(row, chunk); together the waves fill every byte once.
template <int D, int ROWS, int WAVES>
void check_dma() {
  using T = fa::Tile<D, ROWS>;
  using M = fa::TileDma<D, ROWS, WAVES>;
  std::set<int> dst;
  for (int w = 0; w < WAVES; ++w)
    for (int lane = 0; lane < 64; ++lane) {
      M m;
      m.init(w, lane);
      for (int i = 0; i < M::kMine; ++i) {
        const int L = w + i * WAVES;
        if (!(T::kKiB % WAVES == 0 || L < T::kKiB)) continue;
        const int row = m.row0 + i * M::kRowStep;
        const int chunk = m.col_bytes[M::kSamePhase ? 0 : i] / 16;
        EXPECT(row < ROWS && T::offset(row, chunk) == L * 1024 + 16 * lane);
        dst.insert(L * 1024 + 16 * lane);
      }
    }
  EXPECT((int)dst.size() == T::kBytes / 16);
}

int main() {
  check<32, 32>(); check<32, 64>();
  check<64, 32>(); check<64, 64>();
  check<128, 32>(); check<128, 64>();
  check_dma<32, 64, 2>(); check_dma<32, 64, 4>(); check_dma<32, 64, 8>();
  check_dma<64, 64, 2>(); check_dma<64, 64, 4>(); check_dma<64, 64, 8>();
  check_dma<128, 64, 2>(); check_dma<128, 64, 4>(); check_dma<128, 64, 8>();
  std::printf("%ld %ld\n", checked, bad);
  return bad != 0;
}
"""


def test_tile_addressing(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    src = tmp_path / "tiles.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "tiles"
    r = subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17", f"-I{CSRC}",
                        f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    checked, bad = map(int, r.stdout.split()[-2:])
    assert checked > 10000
    assert r.returncode == 0 and bad == 0, r.stdout[-2000:]
