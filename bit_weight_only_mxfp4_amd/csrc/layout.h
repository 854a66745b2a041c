// layout.h -- the private tiled layout of packed weights, shared by the host
// packers (pack.cpp) and the kernels (*.hip).
//
// Both formats are laid out in *tiles* of 16 rows.  A tile is a contiguous
// byte range; tiles follow each other at a fixed stride.  Inside a tile the
// reduction dimension K is cut into *units*: 4 consecutive 32-element pieces
// per row (128 elements).  One unit of one tile is 16 rows x 4 pieces x 16
// bytes = 1 KiB, stored so that lane l of a 64-wide wavefront loads bytes
// [16 l, 16 l + 16) -- piece q = l / 16 of row r = l % 16, i.e. 32 FP4/INT4
// elements in their canonical nibble order.  One 16-byte load per lane
// therefore streams 1 KiB of contiguous weights per wave instruction.
//
// MXFP4 tile (K % 32 == 0, nb = K / 32 blocks; a piece is one block):
//   [codes]  units U = ceil(nb / 4); unit kk at byte 1024 kk; the last unit
//            holds only qv_last = nb - 4 (U - 1) pieces (256 qv_last bytes).
//   [scales] ceil(U / 4) groups of 256 bytes: in group j, lane l's dword
//            holds the E8M0 byte of its piece in units 4j .. 4j+3 (byte t for
//            unit 4j + t).  Pieces past the row end read scale 127 (1.0).
//   [trailer] 128 bytes: 16 fp32 row postscales, then 64 reserved bytes.
//   The gate/up pack puts gate rows 8t..8t+7 in tile rows 0..7 and the up
//   rows of the same output features in tile rows 8..15.
//
// INT4 tile (group 128 = one unit; K even, padded to 32 with zero nibbles):
//   [codes]  nq = ceil(K / 32) pieces, U = ceil(nq / 4) units, as above.
//   [s|z]    ceil(U / 4) groups of 256 bytes: in group j, row r owns 16
//            bytes = 4 dwords (s | z << 16) for units 4j .. 4j+3.
//
// Rows past N in the last tile are zero codes with scale 127 (value 0).
//
// FP8 E4M3 tile (row-scaled matvec; down projections have few rows and a
// long K, so these tiles are 8 rows high to give twice as many workgroups):
//   [codes]  units U = ceil(K / 128); one unit is 8 rows x 8 pieces x 16
//            bytes = 1 KiB, lane l loading piece q = l / 8 (16 consecutive k)
//            of row r = l % 8.  Codes past K and rows past N are 0.
//   [scales] 64 bytes: 8 fp32 row scales, then 32 reserved bytes.
#pragma once

#include <stdint.h>

// The geometry helpers run on the host (packers, launch set-up) and in the
// kernels (which derive a tile's offsets from its block count).
#ifdef __HIPCC__
#define TT_GEOM __host__ __device__ inline
#else
#define TT_GEOM inline
#endif

namespace tt {

constexpr int kTileRows = 16;
constexpr int kUnitBytes = 1024;
constexpr int kGroupBytes = 256;
constexpr int kTrailerBytes = 128;
constexpr uint8_t kPadScale = 127;

struct MxGeom {
    int64_t k;         // columns
    int64_t nb;        // 32-element blocks per row
    int64_t units;     // units per tile row-band
    int64_t qv_last;   // valid pieces in the last unit (1..4)
    int64_t groups;    // 256-byte scale groups
    int64_t scale_off; // byte offset of the scale groups in a tile
    int64_t ps_off;    // byte offset of the postscale trailer
    int64_t stride;    // bytes per tile
};

TT_GEOM MxGeom mx_geom(int64_t k) {
    MxGeom g;
    g.k = k;
    g.nb = k / 32;
    g.units = (g.nb + 3) / 4;
    g.qv_last = g.nb - 4 * (g.units - 1);
    g.groups = (g.units + 3) / 4;
    g.scale_off = 256 * g.nb;  // 16 rows x nb blocks x 16 bytes
    g.ps_off = g.scale_off + kGroupBytes * g.groups;
    g.stride = g.ps_off + kTrailerBytes;
    return g;
}

struct I4Geom {
    int64_t k;
    int64_t nq;        // 32-element pieces per row (K padded to 32)
    int64_t units;
    int64_t qv_last;
    int64_t groups;
    int64_t sz_off;
    int64_t stride;
};

TT_GEOM I4Geom i4_geom(int64_t k) {
    I4Geom g;
    g.k = k;
    g.nq = (k + 31) / 32;
    g.units = (g.nq + 3) / 4;
    g.qv_last = g.nq - 4 * (g.units - 1);
    g.groups = (g.units + 3) / 4;
    g.sz_off = 256 * g.nq;
    g.stride = g.sz_off + kGroupBytes * g.groups;
    return g;
}

constexpr int kF8TileRows = 8;
constexpr int kF8UnitK = 128;
constexpr int kF8TrailerBytes = 64;

struct F8Geom {
    int64_t k;
    int64_t units;     // 128-element units per row
    int64_t scale_off; // byte offset of the row scales
    int64_t stride;    // bytes per tile
};

TT_GEOM F8Geom f8_geom(int64_t k) {
    F8Geom g;
    g.k = k;
    g.units = (k + kF8UnitK - 1) / kF8UnitK;
    g.scale_off = 1024 * g.units;
    g.stride = g.scale_off + kF8TrailerBytes;
    return g;
}

TT_GEOM int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace tt
