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

// That layout with every sample's block cut to its own lattice ("packed", the
// layout inside `saved`): sample b's block holds lat_nq(T_b, U_b + 1) groups
// of lat_us(U_b + 1) rows and starts at entry off[b], the prefix sum of the
// blocks before it, so padding frames and padding labels take no space.
// The padded layout above is the packed one with every sample at T_b = T,
// U_b = U. A block is a multiple of 4 entries, so every block stays 16-byte
// aligned.
struct LatGeo {
  int64_t base;  // first entry of the sample's block
  int us;        // rows per group of four diagonals
};
constexpr int64_t lat_block(int Tb, int Ub) { return lat_sample(Tb, Ub + 1); }
constexpr LatGeo lat_geo_padded(int b, int T, int U1) { return LatGeo{(int64_t)b * lat_sample(T, U1), lat_us(U1)}; }
constexpr LatGeo lat_geo_packed(int64_t base, int Ub) { return LatGeo{base, lat_us(Ub + 1)}; }
constexpr int64_t lat_at(const LatGeo& g, int t, int u) {
  return g.base + ((int64_t)((t + u) >> 2) * g.us + u) * 4 + ((t + u) & 3);
}

}  // namespace rnnt
