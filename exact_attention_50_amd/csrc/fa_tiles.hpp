// LDS tiles of bf16 rows shared by the attention kernels (gfx950).
//
// A tile holds ROWS consecutive rows of a [S, D] bf16 tensor, row r at byte
// r * 2D.  Its 16-byte chunks are permuted inside each row,
//     chunk c of row r lives at chunk position c ^ f(r),
// with f(r) = 4 (r & 3) + ((r >> 2) & 3)          for D = 128 (16 chunks/row),
//      f(r) = 4 ((r >> 1) & 1) + ((r >> 2) & 3)   for D = 64  (8 chunks/row),
// which makes both ways the kernels read a tile free of LDS bank conflicts:
//   * row reads (MFMA A operand with rows = tile rows, k = D): 32 rows at one
//     chunk, 16 bytes per lane (ds_read_b128);
//   * transposed reads (A operand with rows = D, k = tile rows): 4 rows x 4
//     chunks per 32 lanes, 8 bytes per lane (ds_read_b64_tr_b16).
// The same tile can therefore serve as K and as K^T, V and V^T, Q and Q^T.
//
// Addressing.  With this permutation every operand read is a per-lane base
// XOR a small constant plus a constant (an immediate of the LDS instruction):
//   row read, rows 32 kb + r, dims 16 kc + 8 g .. +8:
//       (row_lane ^ 32 kc) + 32 kb * RowBytes
//   transposed read, dims 32 db .. +32, rows 16 ks + 8 jh + (4 g + s / 4),
//   s = lane % 16:
//       ((tr_lane ^ 32 jh) ^ 64 db) + (16 ks + 8 jh) RowBytes
// and the 16 rows of step ks arrive in the MFMA accumulator's row order (slot
// 8 g + j holds row 8 (j / 4) + 4 g + j % 4), so an accumulator rounded to
// bf16 is directly the matching B operand.
#pragma once

#include "fa_device.hpp"

namespace fa {

template <int D>
struct TileGeom {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;               // 16-byte chunks per row
  static constexpr int kRowsPerLoad = 64 / kChunks;   // rows of one wave-wide 16-byte load
};

template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  return D == 128 ? (4 * (r & 3) + ((r >> 2) & 3)) : (4 * ((r >> 1) & 1) + ((r >> 2) & 3));
}

template <int D>
__device__ __forceinline__ int row_lane_offset(int lane) {
  const int r = lane & 31, g = lane >> 5;
  const int x = tile_swz<D>(r);
  return r * TileGeom<D>::kRowBytes + 32 * (x >> 1) + 16 * (g ^ (x & 1));
}

template <int D>
__device__ __forceinline__ int tr_lane_offset(int lane) {
  const int s16 = lane & 15, g = lane >> 5;
  const int w = D == 128 ? ((s16 >> 2) & 3) : ((s16 >> 3) & 1);
  const int part = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
  return (4 * g + (s16 >> 2)) * TileGeom<D>::kRowBytes + 64 * w + 16 * (part ^ g) + 8 * (s16 & 1);
}

// A operand, rows 32 kb .. +32 of the tile, dims 16 kc + 8 g .. +8.
template <int D>
__device__ __forceinline__ bf16x8 read_rows(const char* tile, int row_lane, int kb, int kc) {
  return *reinterpret_cast<const bf16x8*>(tile + (row_lane ^ (32 * kc)) + 32 * kb * TileGeom<D>::kRowBytes);
}

// A operand with rows = dims 32 db .. +32 and k = the 16 tile rows of step ks,
// in accumulator row order (two ds_read_b64_tr_b16 of 4 rows x 16 dims).
template <int D>
__device__ __forceinline__ bf16x8 read_cols(const char* tile, int tr_lane, int ks, int db) {
  constexpr int RB = TileGeom<D>::kRowBytes;
  const bf16x4_t lo = lds_read_tr16(tile + (tr_lane ^ (64 * db)) + 16 * ks * RB);
  const bf16x4_t hi = lds_read_tr16(tile + ((tr_lane ^ 32) ^ (64 * db)) + (16 * ks + 8) * RB);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// A tile's share (ROWS rows split over NW waves; wave `wave` handles loads
// i = 0 .. kLoads-1, the rows of load i NW + wave) loaded straight from
// memory into LDS with the chunk permutation (gfx950's 16-byte
// buffer_load ... lds).  One such load writes 64 x 16 contiguous LDS bytes,
// lane i at the uniform base + 16 i, i.e. RowsPerLoad whole rows; so lane i
// fetches the global chunk that belongs at its LDS position: chunk
// (i % Chunks) ^ f(row) of the row.  Rows at or past the descriptor's end
// are written as zeros.  The writes complete with the wave's vector-memory
// counter: wait for vmcnt, then a barrier, before other waves read them.
template <int D, int ROWS, int NW>
struct TileDMA {
  static constexpr int kLoads = ROWS / TileGeom<D>::kRowsPerLoad / NW;
  static_assert(kLoads >= 1, "tile too small for the workgroup");

  // load i (0 <= i < kLoads) of this wave
  __device__ __forceinline__ static void load_one(__amdgpu_buffer_rsrc_t src, int row0, char* tile, int wave, int lane,
                                                  int i) {
    constexpr int RPL = TileGeom<D>::kRowsPerLoad;
    constexpr int C = TileGeom<D>::kChunks;
    const int blk = i * NW + wave;   // wave-uniform
    const int row = blk * RPL + lane / C;
    const unsigned off = (unsigned)(row0 + row) * TileGeom<D>::kRowBytes + ((lane % C) ^ tile_swz<D>(row)) * 16;
    lds_dma16(src, off, tile + blk * RPL * TileGeom<D>::kRowBytes);
  }
  __device__ __forceinline__ static void load(__amdgpu_buffer_rsrc_t src, int row0, char* tile, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) load_one(src, row0, tile, wave, lane, i);
  }
};

// Output of a wave's 32 x D accumulator block as bf16 rows.  In the MFMA C
// layout of X^T a lane holds 8-byte pieces of one row of X (acc[db][i] is
// X[r][32 db + 8 (i / 4) + 4 g + i % 4] for lane r + 32 g), so storing from
// registers touches 32 rows per instruction.  The block, times mul (per lane,
// i.e. per row), is staged in `stage` (kBytes of LDS private to the wave, rows
// padded by 16 bytes so the 8-byte writes meet every bank once per 16 rows)
// and stored 16 bytes per lane over consecutive rows: rows row0 .. row0 + 31
// of out (row pitch D elements), skipping rows >= n_rows.  With swap23 the
// lane's row is r with bits 2 and 3 exchanged (lane r + 32 g holds row
// (r & 19) | (r & 4) << 1 | (r & 8) >> 1): the row order of an accumulator
// whose columns came from a transposed read of rows stored in that order.
template <int D>
struct RowStore {
  static constexpr int kPitch = D * 2 + 16;
  static constexpr int kBytes = 32 * kPitch;

  __device__ __forceinline__ static void store(char* stage, const f32x16* acc, float mul, bf16* out, int row0,
                                               int n_rows, int lane, bool swap23 = false) {
    const int r = lane & 31, g = lane >> 5;
    const int sr = swap23 ? ((r & 19) | ((r & 4) << 1) | ((r & 8) >> 1)) : r;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 v = {acc[db][4 * i4 + 0] * mul, acc[db][4 * i4 + 1] * mul, acc[db][4 * i4 + 2] * mul,
                         acc[db][4 * i4 + 3] * mul};
        *reinterpret_cast<bf16x4*>(stage + sr * kPitch + (db * 32 + 8 * i4 + 4 * g) * 2) =
            __builtin_convertvector(v, bf16x4);
      }
    constexpr int kChunks = D / 8;   // 16-byte chunks per row
    constexpr int kRowsPerStore = 64 / kChunks;
    const int c = lane % kChunks;
#pragma unroll
    for (int j = 0; j < 32 / kRowsPerStore; ++j) {
      const int row = j * kRowsPerStore + lane / kChunks;
      const u32x4 val = *reinterpret_cast<const u32x4*>(stage + row * kPitch + c * 16);
      if (row0 + row < n_rows) *reinterpret_cast<u32x4*>(out + (size_t)(row0 + row) * D + c * 8) = val;
    }
  }
};

}  // namespace fa
