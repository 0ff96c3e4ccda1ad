// Plan records as seen by host code that is compiled without HIP. Their
// layout is identical to rnnt::Tile / rnnt::Group in common.hpp (checked by
// static_asserts in api.hip).
#pragma once

#include <stdint.h>

namespace rnnt {

struct TileH {
  int32_t b, t0, u0, ht, wu, htp, row0, strip0;
};

struct GroupH {
  int32_t b, start, len, first, count, pad0, pad1, pad2;
};

}  // namespace rnnt
