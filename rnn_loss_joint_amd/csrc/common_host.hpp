// Plan records as seen by host code that is compiled without HIP (their
// layout is identical to rnnt::Tile / rnnt::Group in common.hpp, checked by
// static_asserts in api.hip), and the layout of the lattice arrays.
#pragma once

#include <stdint.h>

namespace rnnt {

struct TileH {
  int32_t b, t0, u0, ht, wu, htp, row0, strip0;
};

struct GroupH {
  int32_t b, start, len, first, count, pad0, pad1, pad2;
};

// Lattice arrays (lse, phi, psi, alpha, beta) are stored per sample in
// groups of four anti-diagonals: cell (t, u) of sample b, on diagonal
// d = t + u, is entry ((b * NQ + d / 4) * US + u) * 4 + d % 4, with
// NQ = ceil((T + U1 - 1) / 4) groups and US = U1 rounded up to 32 rows. The
// four diagonals 4q .. 4q + 3 of row u form one aligned 16-byte piece and
// the pieces of consecutive rows are adjacent, so the forward-backward sweep
// (one row per lane, diagonal after diagonal) moves four diagonals of a row
// with one 16-byte access, and a group of a diagonal's rows is contiguous.
// (constexpr: usable from host and device code)
constexpr int lat_us(int U1) { return (U1 + 31) & ~31; }
constexpr int lat_nq(int T, int U1) { return (T + U1 - 1 + 3) / 4; }
constexpr int64_t lat_sample(int T, int U1) { return (int64_t)lat_nq(T, U1) * lat_us(U1) * 4; }
constexpr int64_t lat_cells(int B, int T, int U1) { return (int64_t)B * lat_sample(T, U1); }
constexpr int64_t lat_ix(int b, int t, int u, int T, int U1) {
  return (((int64_t)b * lat_nq(T, U1) + ((t + u) >> 2)) * lat_us(U1) + u) * 4 + ((t + u) & 3);
}

}  // namespace rnnt
