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

// Lattice arrays (lse, phi, psi, alpha, beta) are stored diagonal-major per
// sample: cell (t, u) of sample b is entry (b * ND + t + u) * US + u, with
// ND = T + U1 - 1 diagonals and the diagonal stride US = U1 rounded up to 32
// entries (128 bytes). A diagonal is then one contiguous, aligned vector
// over u, which is what the forward-backward sweep reads and writes; the
// neighbours (t + 1, u) and (t, u + 1) sit US and US + 1 entries further.
// (constexpr: usable from host and device code)
constexpr int lat_us(int U1) { return (U1 + 31) & ~31; }
constexpr int lat_nd(int T, int U1) { return T + U1 - 1; }
constexpr int64_t lat_cells(int B, int T, int U1) { return (int64_t)B * lat_nd(T, U1) * lat_us(U1); }
constexpr int64_t lat_ix(int b, int t, int u, int T, int U1) {
  return ((int64_t)b * lat_nd(T, U1) + t + u) * lat_us(U1) + u;
}

}  // namespace rnnt
