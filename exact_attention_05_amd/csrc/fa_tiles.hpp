// LDS tiles of bf16 rows (K, V, Q or dO blocks) for the gfx950 kernels:
// layout, direct global -> LDS filling, and the two operand reads the matrix
// cores need.
//
// Layout: a tile is ROWS rows of D bf16 values, unpadded (2*D bytes per
// row).  The 16-byte chunk c of row r is stored at chunk position c ^ f(r).
// The LDS serves 256 bytes (64 banks x 4 bytes) per clock: 16 lanes of a
// 16-byte row read, 32 lanes of an 8-byte transposing read.  f keeps both
// reads free of bank conflicts:
//  * row read: 16 consecutive rows, one logical chunk each, must occupy
//    distinct banks;
//  * transposing read: two 16-lane groups read the same 4 aligned rows, the
//    first the chunk pair {b, b+1}, the second {b+2, b+3} (b a multiple of
//    4); the 8 (row, pair) combinations must occupy distinct banks.
// For D = 128 (one 256-byte row spans all banks) f(r) = 4 (r mod 4) +
// (r/4 mod 4): a permutation over any 16 aligned rows, and 4 aligned rows
// differ in chunk bits 2-3 while sharing bits 0-1.  For D = 64 two rows
// share the banks and f(r) = 4 (r/2 mod 2) + (r/4 mod 4); for D = 32 four
// rows share them and f(r) = r/4 mod 4.
// Filling: the tile is copied with global_load_lds_dwordx4, 1 KiB per wave
// instruction (lane j writes bytes [16 j, 16 j + 16) of its KiB).  Wave w of
// a WAVES-wave workgroup issues KiB number w, w + WAVES, ...  Rows past the
// last valid row repeat the last valid row, so nothing outside the tensor is
// read; callers mask those rows.
#pragma once

#include "fa_device.hpp"

namespace fa {

template <int D, int ROWS>
struct Tile {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = D / 8;            // 16-byte chunks per row
  static constexpr int kBytes = ROWS * kRowBytes;
  static constexpr int kKiB = kBytes / 1024;
  static_assert(kKiB * 1024 == kBytes, "a tile is a whole number of KiB");

  // Chunk permutation of row `row` (see the layout note above).
  __host__ __device__ static __forceinline__ int swizzle(int row) {
    if constexpr (D == 128) return 4 * (row & 3) + ((row >> 2) & 3);
    else if constexpr (D == 64) return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
    else return (row >> 2) & 3;
  }

  // Byte offset of (row, 16-byte logical chunk) within the tile.
  __host__ __device__ static __forceinline__ int offset(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swizzle(row)) << 4);
  }

  // A-operand read for v_mfma_f32_32x32x16_bf16 from rows row0 .. row0+31:
  // lane l gets row row0 + l%32, columns 16c + 8(l/32) .. +7.
  __host__ __device__ static __forceinline__ int rows_offset(int row0, int c, int lane) {
    return offset(row0 + (lane & 31), 2 * c + (lane >> 5));
  }
  __device__ static __forceinline__ bf16x8 read_rows(const char* tile, int row0, int c, int lane) {
    return *reinterpret_cast<const bf16x8*>(tile + rows_offset(row0, c, lane));
  }

  // A-operand read of the TRANSPOSED tile for v_mfma_f32_32x32x16_bf16:
  // operand rows are tile columns col0 .. col0+31, operand k-slots are tile
  // rows.  Lane l gets columns col0 + l%32 of tile rows
  //   r0 + 4(l/32) + 0..3  and  r0 + 8 + 4(l/32) + 0..3,
  // i.e. the 16-row chunk r0 .. r0+15 in the order the 32x32 accumulator
  // layout lists its rows (element i of lane l is row 8(i/4) + 4(l/32) + i%4),
  // so an accumulator converted to bf16 can be the matching B operand.
  // Byte offset of the lane's 8-byte piece `half` (0: rows r0 + 4(l/32) +
  // 0..3, 1: the same rows + 8) of that read; the transposing read takes
  // 4 columns of 4 consecutive rows from each lane group of 4.
  __host__ __device__ static __forceinline__ int tr_offset(int r0, int col0, int lane, int half) {
    const int row = r0 + 4 * (lane >> 5) + ((lane & 15) >> 2) + 8 * half;
    const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    return offset(row, col >> 3) + 2 * (col & 7);
  }
  __device__ static __forceinline__ bf16x8 read_cols_tr(const char* tile, int r0, int col0, int lane) {
    const bf16x4 a = lds_read_tr16(reinterpret_cast<const __bf16*>(tile + tr_offset(r0, col0, lane, 0)));
    const bf16x4 b = lds_read_tr16(reinterpret_cast<const __bf16*>(tile + tr_offset(r0, col0, lane, 1)));
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
};

// The same two operand reads with the lane's part of the address computed
// once.  The swizzle XORs chunk bits that lie below one row, so
//   offset(row, chunk) = (row * kRowBytes + 16 chunk) ^ (16 swizzle(row)),
// and for a row block starting at a multiple of 16 rows (the swizzle period)
// and a chunk split into a lane part and a multiple of the lane part's range,
// the address is the block's row offset plus (lane constant ^ chunk part):
// one XOR per read instead of a per-read register or recomputation.
template <int D, int ROWS>
struct TileLane {
  using T = Tile<D, ROWS>;
  int rows;   // read_rows: lane part for row0 = 0, c = 0
  int tr0;    // read_cols_tr, first 8 bytes: lane part for r0 = 0, col0 = 0
  int tr1;    // second 8 bytes (rows + 8)

  __host__ __device__ __forceinline__ void init(int lane) {
    rows = T::rows_offset(0, 0, lane);
    tr0 = T::tr_offset(0, 0, lane, 0);
    tr1 = T::tr_offset(0, 0, lane, 1);
  }
  // T::rows_offset(row0, c, lane) for row0 a multiple of 32.
  __host__ __device__ __forceinline__ int rows_at(int row0, int c) const {
    return row0 * T::kRowBytes + (rows ^ (32 * c));
  }
  // T::tr_offset(r0, col0, lane, half) for r0 a multiple of 16 and col0 a
  // multiple of 32.
  __host__ __device__ __forceinline__ int tr_at(int r0, int col0, int half) const {
    return r0 * T::kRowBytes + ((half ? tr1 : tr0) ^ (2 * col0));
  }
  __device__ __forceinline__ bf16x8 read_rows(const char* tile, int row0, int c) const {
    return *reinterpret_cast<const bf16x8*>(tile + rows_at(row0, c));
  }
  __device__ __forceinline__ bf16x8 read_cols_tr(const char* tile, int r0, int col0) const {
    const bf16x4 a = lds_read_tr16(reinterpret_cast<const __bf16*>(tile + tr_at(r0, col0, 0)));
    const bf16x4 b = lds_read_tr16(reinterpret_cast<const __bf16*>(tile + tr_at(r0, col0, 1)));
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
};

// Per-lane state for filling Tile<D, ROWS> tiles by direct copies.  The
// KiB blocks of one wave lie WAVES KiB apart.  When that is a whole number of
// 16-row swizzle periods every copy of a lane uses the same chunk position
// and only its row advances; otherwise (two waves) each copy keeps its own.
template <int D, int ROWS, int WAVES>
struct TileDma {
  using T = Tile<D, ROWS>;
  static constexpr int kMine = (T::kKiB + WAVES - 1) / WAVES;  // KiB copies per wave
  static constexpr int kRowStep = WAVES * 1024 / T::kRowBytes;  // rows between a lane's copies
  static constexpr bool kSamePhase = kRowStep % 16 == 0;
  // Every wave issues kMine copies per tile, or none (so that a count of
  // outstanding copies is the same for every wave that has any).
  static_assert(T::kKiB % WAVES == 0 || T::kKiB < WAVES, "uneven copies per wave");
  int row0;                                // tile row of the lane's first copy
  int col_bytes[kSamePhase ? 1 : kMine];   // byte offset of its 16-byte chunk (swizzled)
  int wave;

  __host__ __device__ __forceinline__ void init(int wave_, int lane) {
    wave = wave_;
    const int off = wave * 1024 + 16 * lane;
    row0 = off / T::kRowBytes;
#pragma unroll
    for (int i = 0; i < (kSamePhase ? 1 : kMine); ++i)
      col_bytes[i] = (((off % T::kRowBytes) >> 4) ^ T::swizzle(row0 + i * kRowStep)) * 16;
  }

  // Copy rows [0, ROWS) starting at `src` (row 0 of the tile in global
  // memory, rows of D bf16) into the tile at LDS byte address `lds`.  Rows at
  // or past `valid` repeat row valid - 1 (valid >= 1).
  __device__ __forceinline__ void load(const __bf16* src, int valid, uint32_t lds) const {
#pragma unroll
    for (int i = 0; i < kMine; ++i) {
      const int L = wave + i * WAVES;
      if (T::kKiB % WAVES == 0 || L < T::kKiB) {
        const uint32_t voff =
            (uint32_t)(min(row0 + i * kRowStep, valid - 1) * T::kRowBytes + col_bytes[kSamePhase ? 0 : i]);
        lds_dma16(lds + L * 1024, src, voff);
      }
    }
  }

  // The same for a tile whose ROWS rows all exist: the per-lane offsets do
  // not depend on the tile.
  __device__ __forceinline__ void load_full(const __bf16* src, uint32_t lds) const {
#pragma unroll
    for (int i = 0; i < kMine; ++i) {
      const int L = wave + i * WAVES;
      if (T::kKiB % WAVES == 0 || L < T::kKiB) {
        const uint32_t voff = (uint32_t)((row0 + i * kRowStep) * T::kRowBytes + col_bytes[kSamePhase ? 0 : i]);
        lds_dma16(lds + L * 1024, src, voff);
      }
    }
  }
};

}  // namespace fa
