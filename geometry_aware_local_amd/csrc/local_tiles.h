// Plane-tile geometry shared by the bf16 local-attention kernels (forward
// and backward): the 1 x TY x TX query tile, its patches and the LDS layout
// of a z-plane's K / V rows (tile plus a 3-cell halo).
#pragma once

#include "pack3d_device.h"

namespace pack3d {
namespace lb {

constexpr int kHalo = 3;     // largest supported y/x radius
constexpr int kKx = 8;       // key slots per row: patch width 2 + 2 * halo

template <int G> struct Shape;   // patch PY x 2 cells, tile TY x TX cells
template <> struct Shape<4> { static constexpr int PY = 4, TY = 8, TX = 8; };
template <> struct Shape<8> { static constexpr int PY = 2, TY = 8, TX = 4; };
template <> struct Shape<16> { static constexpr int PY = 1, TY = 4, TX = 4; };

template <int G>
struct Cfg {
  static constexpr int PY = Shape<G>::PY, PX = 2, TY = Shape<G>::TY, TX = Shape<G>::TX;
  static constexpr int KY = PY + 2 * kHalo;                 // key rows per plane
  static constexpr int NKB = (KY * kKx + 31) / 32;          // 32-key blocks per plane
  static constexpr int RX = TX - PX + kKx;                  // region width (cells)
  static constexpr int RY = TY + 2 * kHalo;
  static constexpr int RC = RX * RY;                        // region cells
  static constexpr int RCP = (RC + 7) / 8 * 8;              // padded to 1 KB pieces
  // key blocks round a patch's key rows up to 4*NKB: the last patch row
  // reaches region row TY - PY + 4*NKB - 1, so the slot holds that many rows
  // (the rows past RY are zero, never copied, and always masked)
  static constexpr int RYA = TY - PY + 4 * NKB > RY ? TY - PY + 4 * NKB : RY;
  static constexpr int RCA = RYA * RX > RCP ? RYA * RX : RCP;   // cells per slot
  static constexpr int W = TY * TX / (PY * PX);             // waves = patches
  static_assert(PY * PX * G == 32, "a patch is one MFMA column block");
  static_assert(W <= 16, "at most 1024 threads");
  static_assert(NKB * 4 >= KY, "key rows fit the key blocks");
  static_assert(RX % 2 == 0, "a cell's bank half is the parity of its column");
};

// 16-byte chunk positions in a cell's 128-byte LDS row, for the K and the V
// tiles alike (both are read as rows and, in the backward, transposed).
// gfx950 LDS has 64 four-byte banks; it serves a 128-bit read 16 lanes at a
// time and the 8-byte transposing read 32 lanes at a time.  A cell (y, x) of
// the region sits in bank half x & 1 (RX is even).  A row read takes 8
// consecutive columns of 2 consecutive region rows per 16 lanes: within a
// bank half, 4 consecutive values of x >> 1 times 2 row parities need
// distinct positions.  A transposing read takes 4 consecutive cells of one
// region row times 4 aligned chunks per 32 lanes: the cells x and x + 2 (one
// bank half) need their chunks in different 4-chunk halves.
// sw = 4 ((x >> 1) & 1) + ((x >> 2) & 1) + 2 (y & 1) does both: 4
// consecutive x >> 1 give distinct (bit 0, bit 1) pairs, and x + 2 flips
// bit 0 of x >> 1, hence bit 2 of sw.
__device__ __forceinline__ int kv_swz(int y, int x, int chunk) {
  return chunk ^ (4 * ((x >> 1) & 1) + ((x >> 2) & 1) + 2 * (y & 1));
}

typedef __attribute__((address_space(3))) void* lds_ptr;

}  // namespace lb
}  // namespace pack3d
