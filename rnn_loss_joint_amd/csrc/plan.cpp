// Host-side tile plan and buffer layout. See plan.hpp.
#include "plan.hpp"

#include <algorithm>
#include <cstring>
#include <map>
#include <utility>

namespace rnnt {

namespace {

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

int joint_ks_for(int H) {
  int hp = (H + 63) / 64 * 64;
  int ks = hp / 16;
  static const int ok[] = {8, 16, 24, 32, 40, 48};  // even stage count per V chunk
  for (int v : ok)
    if (v >= ks) return v;
  return -1;
}

bool check_plan(const Plan& p, std::string& err) {
  // row and strip numbers, wave row ranges and the 128-row rounding of the
  // wave buffers are 32-bit in the plan records and the kernels
  if (p.total_rows > kMaxPlanRows) {
    err = "the tile plan has " + std::to_string(p.total_rows) + " rows, more than " + std::to_string(kMaxPlanRows) +
          " (each tile holds tile_u columns of t rows padded to a multiple of 32: small tile_t values "
          "multiply the rows)";
    return false;
  }
  return true;
}

bool persistent_scores(const Plan& p) { return p.d.fp8 || (p.d.bf16 && p.H_pad / 64 >= 8); }

bool check_dims(const Dims& d, std::string& err, int& status) {
  status = -1;  // RNNT_E_INVALID
  if (d.B <= 0 || d.T <= 0 || d.U < 0 || d.V < 2 || d.HA <= 0 || d.HL <= 0 || d.H <= 0) {
    err = "dimensions must satisfy B,T,HA,HL,H > 0, U >= 0, V >= 2";
    return false;
  }
  if (d.blank < 0 || d.blank >= d.V) {
    err = "blank must lie in [0, V)";
    return false;
  }
  if (d.tile_t <= 0 || d.tile_u <= 0) {
    err = "tile_t and tile_u must be positive";
    return false;
  }
  if (d.tiles_per_wave < 0) {
    err = "tiles_per_wave must be >= 0";
    return false;
  }
  status = -4;  // RNNT_E_UNSUPPORTED
  if (d.fp8 && (!d.bf16 || d.untiled)) {
    err = "the fp8 output layer runs in tiled mode only";
    return false;
  }
  if (d.H % 8 || d.HA % 8 || d.HL % 8) {
    err = "this library needs H, HA and HL to be multiples of 8";
    return false;
  }
  if (d.H > 768) {
    err = "this library supports H <= 768";
    return false;
  }
  if (d.U + 1 > 1024) {
    err = "this library supports U + 1 <= 1024";
    return false;
  }
  if (d.V > 65536) {
    err = "this library supports V <= 65536";
    return false;
  }
  // the lattice arrays: B * 4 NQ * US entries in all, and each sample's block
  // addressable with 32-bit byte offsets
  if (lat_cells(d.B, d.T, d.U + 1) > ((int64_t)1 << 30) || lat_sample(d.T, d.U + 1) > ((int64_t)1 << 29)) {
    err = "the lattice arrays exceed B*4*NQ*US <= 2^30 entries or 4*NQ*US <= 2^29 per sample "
          "(NQ = ceil((T+U)/4), US = U+1 rounded up to 32)";
    return false;
  }
  status = 0;
  return true;
}

bool check_lengths(const Dims& d, const int32_t* T_len, const int32_t* U_len, std::string& err) {
  if (!T_len || !U_len) {
    err = "length arrays must not be null";
    return false;
  }
  for (int b = 0; b < d.B; ++b) {
    if (T_len[b] < 1 || T_len[b] > d.T) {
      err = "T_len[" + std::to_string(b) + "] must lie in [1, T]";
      return false;
    }
    if (U_len[b] < 0 || U_len[b] > d.U) {
      err = "U_len[" + std::to_string(b) + "] must lie in [0, U]";
      return false;
    }
  }
  return true;
}

bool check_band(const Dims& d, const int32_t* T_len, const int32_t* U_len, const Band& band, std::string& err) {
  if (!band.lo) {
    err = "band lo array must not be null";
    return false;
  }
  if (band.S < 1) {
    err = "band width must be >= 1";
    return false;
  }
  for (int b = 0; b < d.B; ++b) {
    const int32_t* lo = band.lo + (size_t)b * d.T;
    const int Tb = T_len[b], Ub = U_len[b];
    auto bad = [&](int t, const char* what) {
      err = "band of sample " + std::to_string(b) + ", frame " + std::to_string(t) + ": " + what;
      return false;
    };
    if (lo[0] != 0) return bad(0, "lo must be 0 at the first frame");
    for (int t = 0; t < Tb; ++t) {
      if (lo[t] < 0 || lo[t] > Ub) return bad(t, "lo must lie in [0, U_b]");
      if (t + 1 < Tb && (lo[t + 1] < lo[t] || lo[t + 1] > lo[t] + band.S - 1))
        return bad(t, "lo must not decrease and must step by at most S - 1");
    }
    if ((int64_t)lo[Tb - 1] + band.S - 1 < Ub) return bad(Tb - 1, "the last frame's band must reach U_b");
  }
  return true;
}

void build_plan(const Dims& d, const int32_t* T_len, const int32_t* U_len, int H_pad, Plan& p, const Band& band) {
  p = Plan{};
  p.d = d;
  if (band.lo) {
    p.band_lo.assign(band.lo, band.lo + (size_t)d.B * d.T);
    p.band_S = band.S;
  }
  p.U1 = d.U + 1;
  p.H_pad = H_pad;
  // bf16: whole 256-score tiles (the score kernels write every column of dh)
  p.V_pad = d.bf16 ? (int)cdiv(d.V, 256) * 256 : (int)cdiv(d.V, 64) * 64;
  p.KS = H_pad / 16;
  // fp8: the score kernels take 128 k per stage and at least five stages per item
  p.H8 = d.fp8 ? std::max(640, (int)cdiv(H_pad, 128) * 128) : 0;
  p.tile_tp = (int)cdiv(d.tile_t, 32) * 32;

  // per-sample tile grids
  std::vector<int> nt(d.B), nu(d.B);
  int max_tiles = 0;
  for (int b = 0; b < d.B; ++b) {
    nt[b] = (int)cdiv(T_len[b], d.tile_t);
    nu[b] = (int)cdiv(U_len[b] + 1, d.tile_u);
    max_tiles = std::max(max_tiles, nt[b] * nu[b]);
  }
  auto make_tile = [&](int b, int k) {
    int it = k / nu[b], iu = k % nu[b];
    TileH t{};
    t.b = b;
    t.t0 = it * d.tile_t;
    t.u0 = iu * d.tile_u;
    t.ht = std::min(d.tile_t, T_len[b] - t.t0);
    t.wu = std::min(d.tile_u, U_len[b] + 1 - t.u0);
    t.htp = (int)cdiv(t.ht, 32) * 32;
    return t;
  };
  // A pruned lattice keeps a tile iff some frame's band meets its u range:
  // consecutive bands overlap or touch (steps of at most S - 1), so the
  // bands of the tile's frames cover [lo(t0), lo(t_last) + S - 1] without gaps.
  auto kept = [&](const TileH& t) {
    if (p.band_lo.empty()) return true;
    const int32_t* lo = p.band_lo.data() + (size_t)t.b * d.T;
    return lo[t.t0] <= t.u0 + t.wu - 1 && (int64_t)lo[t.t0 + t.ht - 1] + p.band_S - 1 >= t.u0;
  };
  // per sample, its kept tiles in (t, u) order
  std::vector<std::vector<TileH>> per(d.B);
  for (int b = 0; b < d.B; ++b)
    for (int k = 0; k < nt[b] * nu[b]; ++k) {
      const TileH t = make_tile(b, k);
      if (kept(t)) per[b].push_back(t);
    }
  max_tiles = 0;
  for (int b = 0; b < d.B; ++b) max_tiles = std::max(max_tiles, (int)per[b].size());
  if (d.untiled) {
    // one wave holding every tile, sample by sample
    for (int b = 0; b < d.B; ++b)
      for (const TileH& t : per[b]) p.tiles.push_back(t);
  } else {
    // round robin over samples, so consecutive tiles belong to different samples
    for (int k = 0; k < max_tiles; ++k)
      for (int b = 0; b < d.B; ++b)
        if (k < (int)per[b].size()) p.tiles.push_back(per[b][k]);
  }
  // packed lattice blocks: sample b's block is cut to its own T_b x (U_b + 1)
  p.lat_off.assign(d.B + 1, 0);
  for (int b = 0; b < d.B; ++b) p.lat_off[b + 1] = p.lat_off[b] + lat_block(T_len[b], U_len[b]);
  // lattice sweep pairing: the j-th longest sample's alpha with the j-th
  // shortest's beta (longest first by T_b - 1 + U_b, ties by index)
  {
    std::vector<int32_t> order(d.B);
    for (int b = 0; b < d.B; ++b) order[b] = b;
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
      return T_len[x] + U_len[x] > T_len[y] + U_len[y];
    });
    p.lat_pair.assign(2 * (size_t)d.B, 0);
    for (int j = 0; j < d.B; ++j) {
      p.lat_pair[2 * j] = order[j];
      p.lat_pair[2 * j + 1] = order[d.B - 1 - j];
    }
  }
  int64_t row = 0, strip = 0;
  for (auto& t : p.tiles) {
    t.row0 = (int32_t)row;
    t.strip0 = (int32_t)strip;
    row += (int64_t)t.wu * t.htp;
    strip += t.htp / 32;
  }
  p.total_rows = row;

  const int n = (int)p.tiles.size();
  int tpw = d.tiles_per_wave;
  if (tpw <= 0) {
    // enough rows per wave to fill the GPU: at least B tiles and ~128K rows
    int64_t area = (int64_t)p.tile_tp * d.tile_u;
    tpw = (int)std::max<int64_t>(d.B, cdiv(131072, area));
  }
  if (d.untiled) tpw = std::max(n, 1);
  p.tpw = tpw;

  for (int w0 = 0; w0 < n; w0 += tpw) {
    WaveInfo wv{};
    wv.tile_begin = w0;
    wv.tile_end = std::min(n, w0 + tpw);
    const TileH& first = p.tiles[wv.tile_begin];
    const TileH& last = p.tiles[wv.tile_end - 1];
    wv.row_begin = first.row0;
    wv.row_end = last.row0 + last.wu * last.htp;
    wv.strip_begin = first.strip0;
    wv.strip_end = last.strip0 + last.htp / 32;
    // gA groups: tiles of this wave sharing (b, t0); gL groups: sharing (b, u0)
    std::map<std::pair<int, int>, std::vector<int>> ga, gl;
    for (int i = wv.tile_begin; i < wv.tile_end; ++i) {
      ga[{p.tiles[i].b, p.tiles[i].t0}].push_back(i);
      gl[{p.tiles[i].b, p.tiles[i].u0}].push_back(i);
    }
    auto emit = [&](const std::map<std::pair<int, int>, std::vector<int>>& m, bool is_a, int& mx) {
      for (const auto& kv : m) {
        GroupH g{};
        g.b = kv.first.first;
        g.start = kv.first.second;
        const TileH& t = p.tiles[kv.second[0]];
        g.len = is_a ? t.ht : t.wu;
        g.first = (int)p.gidx.size();
        g.count = (int)kv.second.size();
        for (int id : kv.second) p.gidx.push_back(id);
        mx = std::max(mx, g.len);
        p.groups.push_back(g);
      }
    };
    wv.gA_begin = (int)p.groups.size();
    emit(ga, true, wv.maxA_len);
    wv.gA_end = (int)p.groups.size();
    wv.gL_begin = (int)p.groups.size();
    emit(gl, false, wv.maxL_len);
    wv.gL_end = (int)p.groups.size();
    p.waves.push_back(wv);
    p.max_wave_rows = std::max(p.max_wave_rows, wv.row_end - wv.row_begin);
    p.max_wave_tiles = std::max(p.max_wave_tiles, wv.tile_end - wv.tile_begin);
  }

  // Tiled mode sizes the wave buffers by the tile bound, not by the largest
  // wave actually planned, so the working set depends on the tile size and
  // tiles_per_wave only (min'd with the tile count for small problems).
  if (!d.untiled) {
    int64_t bound_tiles = std::min<int64_t>(tpw, n);
    p.max_wave_rows = (int)std::max<int64_t>(p.max_wave_rows, bound_tiles * p.tile_tp * d.tile_u);
    p.max_wave_tiles = (int)std::max<int64_t>(p.max_wave_tiles, bound_tiles);
  }
  // split-K counts: dW^O ~1024 workgroups of 128 x 128 (fp32 path); in the
  // bf16 path all output tiles of one split run on one XCD (32 CUs, the
  // split's dh and z rows shared in its L2), as many whole splits per XCD as
  // fit, one round (the dz workgroups of the same launch fill the rest);
  // dW^A / dW^L ~512
  p.nvt = (int)cdiv(d.V, 256);
  if (d.bf16) {
    int64_t tiles_vh = cdiv(d.V, 256) * cdiv(d.H + 1, 256);
    int64_t per_xcd = std::max<int64_t>(1, 32 / tiles_vh);
    p.s6 = (int)std::max<int64_t>(1, std::min<int64_t>(8 * per_xcd, p.max_wave_rows / 4096));
  } else {
    int64_t tiles_vh = cdiv(d.V, 128) * cdiv(d.H, 128);
    p.s6 = (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(1024, tiles_vh), p.max_wave_rows / 2048));
  }
  int64_t tiles_ha = cdiv(d.H, 128) * cdiv(d.HA, 128);
  int64_t tiles_hl = cdiv(d.H, 128) * cdiv(d.HL, 128);
  p.s7a = (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(512, tiles_ha), cdiv((int64_t)d.B * d.T, 64)));
  p.s7l = (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(512, tiles_hl), cdiv((int64_t)d.B * p.U1, 64)));
}

Layout make_layout(const Plan& p) {
  const Dims& d = p.d;
  Layout L{};
  const size_t ct = d.bf16 ? 2 : 4;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  L.off_status = take(2 * sizeof(int32_t));
  L.off_Tlen = take(sizeof(int32_t) * d.B);
  L.off_Ulen = take(sizeof(int32_t) * d.B);
  L.off_tiles = take(sizeof(TileH) * p.tiles.size());
  L.off_groups = take(sizeof(GroupH) * p.groups.size());
  L.off_gidx = take(sizeof(int32_t) * p.gidx.size());
  L.off_latoff = take(sizeof(int64_t) * p.lat_off.size());
  L.off_latpair = take(sizeof(int32_t) * p.lat_pair.size());
  L.off_band = p.band_lo.empty() ? 0 : take(sizeof(int32_t) * p.band_lo.size());
  L.plan_bytes = o;
  L.off_labels = take(sizeof(int32_t) * (size_t)d.B * p.U1);
  const size_t cells = (size_t)p.lat_off[d.B];
  L.lat_entries = cells;
  L.off_a = take(sizeof(float) * (size_t)d.B * d.T * p.H_pad);
  L.off_l = take(sizeof(float) * (size_t)d.B * p.U1 * p.H_pad);
  L.off_lse = take(sizeof(float) * cells);
  L.off_phi = take(sizeof(float) * cells);
  L.off_psi = take(sizeof(float) * cells);
  // fp32 mode keeps the forward-backward variables in fp64: in fp32 their
  // magnitude (thousands of nats on long lattices) would limit the
  // occupancies exp(alpha + beta - ln P) to about 1e-4 relative
  L.lat64 = !d.bf16;
  const size_t lat_el = L.lat64 ? sizeof(double) : sizeof(float);
  L.off_alpha = take(lat_el * cells);
  L.off_beta = take(lat_el * cells);
  L.off_lnP = take(lat_el * d.B);
  L.off_logits = L.off_z = 0;
  if (d.untiled) {
    L.off_logits = take(ct * (size_t)p.total_rows * p.V_pad);
    // bf16: z rows, with the rows up to the next multiple of 128 and 128 more
    // as padding that the score kernels' last cell tile reads (never used)
    const size_t zrows = d.bf16 ? (size_t)(p.total_rows + 255) / 128 * 128 : (size_t)p.total_rows;
    L.off_z = take(ct * zrows * p.H_pad);
  }
  L.saved_bytes = o;

  o = 0;
  L.w_dh = L.w_z = 0;
  // wave buffers hold whole 128-row cell tiles (rows past the wave are scratch)
  const size_t wrows = (size_t)cdiv(p.max_wave_rows, 128) * 128;
  if (!d.untiled) {
    L.w_dh = take(ct * wrows * p.V_pad);
    L.w_z = take(ct * wrows * p.H_pad);  // bf16: z rows; fp32: z^T [H_pad, max_wave_rows]
  }
  L.w_gA = take(sizeof(float) * (size_t)d.B * d.T * d.H);
  L.w_gL = take(sizeof(float) * (size_t)d.B * p.U1 * d.H);
  L.w_PA = take(sizeof(float) * (size_t)p.max_wave_tiles * p.tile_tp * d.H);
  L.w_PL = take(sizeof(float) * (size_t)p.max_wave_tiles * (p.tile_tp / 32) * d.tile_u * d.H);
  L.w_PW = take(sizeof(float) * (size_t)p.s6 * d.V * d.H);
  L.w_PB = take(sizeof(float) * (size_t)p.s6 * d.V);
  L.w_PWA = take(sizeof(float) * (size_t)p.s7a * d.H * d.HA);
  L.w_PBZ = take(sizeof(float) * (size_t)p.s7a * d.H);
  L.w_PWL = take(sizeof(float) * (size_t)p.s7l * d.H * d.HL);
  L.w_WOT = take(ct * (size_t)d.H * p.V_pad);
  // bf16 forward buffers, one wave of rows (wave-relative, whole cell tiles)
  L.w_zf = 0;  // the tiled forward's z rows reuse the backward's z buffer (w_z)
  L.w_stats = d.bf16 ? take(8 * wrows * p.nvt) : 0;
  L.w_hb = d.bf16 ? take(4 * wrows) : 0;
  L.w_hy = d.bf16 ? take(4 * wrows) : 0;
  // persistent score kernels: padded W^O, bias table; bf16 backward
  // coefficients per wave row (persistent score kernels, untiled mode)
  L.w_WOp = L.w_bl = L.w_coefA = L.w_coefB = 0;
  const bool s3 = persistent_scores(p);
  if (s3 && !d.fp8) L.w_WOp = take(2 * (size_t)p.nvt * 256 * p.H_pad);
  if (s3 || (d.bf16 && d.untiled)) L.w_bl = take(4 * (size_t)p.nvt * 256);  // untiled: dh_logits reads it
  if (d.bf16 && (s3 || d.untiled)) {
    L.w_coefA = take(8 * wrows);
    L.w_coefB = take(16 * wrows);
  }
  L.w_WO8 = L.w_z8 = L.w_ew = 0;
  if (d.fp8) {
    L.w_WO8 = take((size_t)p.nvt * 256 * p.H8);
    L.w_z8 = take(wrows * p.H8);
    L.w_ew = take(sizeof(int32_t));
  }
  // bf16: gA and gL rounded to bf16 for the encoder-side products, in the
  // wave buffers (dh then z, contiguous, dead after the last wave) when they fit
  L.w_gb = 0;
  if (d.bf16) {
    const size_t gb = 2 * ((size_t)d.B * d.T + (size_t)d.B * p.U1) * d.H;
    const size_t wave_bytes = d.untiled ? 0 : ct * wrows * (size_t)(p.V_pad + p.H_pad);
    L.w_gb = gb <= wave_bytes ? L.w_dh : take(gb);
  }
  // bf16: the encodings with their padding rows zeroed (operands of dW^A and
  // dW^L), after the rounded gA, gL in the dead wave buffers when both fit
  L.w_hs = 0;
  if (d.bf16) {
    const size_t gb = 2 * ((size_t)d.B * d.T + (size_t)d.B * p.U1) * d.H;
    const size_t hs = 2 * ((size_t)d.B * d.T * d.HA + (size_t)d.B * p.U1 * d.HL);
    const size_t wave_bytes = d.untiled ? 0 : ct * wrows * (size_t)(p.V_pad + p.H_pad);
    L.w_hs = L.w_gb == L.w_dh && gb + hs <= wave_bytes ? L.w_dh + (gb + 255) / 256 * 256 : take(hs);
  }
  L.w_WAT = d.bf16 ? take(2 * (size_t)d.HA * d.H) : 0;
  L.w_WLT = d.bf16 ? take(2 * (size_t)d.HL * d.H) : 0;
  L.workspace_bytes = o;
  return L;
}

Layout make_forward_layout(const Plan& p) {
  const Dims& d = p.d;
  Layout L = make_layout(p);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  const size_t wrows = (size_t)cdiv(p.max_wave_rows, 128) * 128;
  L.w_dh = L.w_gA = L.w_gL = L.w_PA = L.w_PL = L.w_PW = L.w_PB = L.w_PWA = L.w_PBZ = L.w_PWL = L.w_WOT = 0;
  L.w_coefA = L.w_coefB = L.w_gb = L.w_hs = L.w_WAT = L.w_WLT = 0;
  L.w_z = L.w_stats = L.w_hb = L.w_hy = L.w_WOp = L.w_bl = L.w_WO8 = L.w_z8 = L.w_ew = 0;
  if (d.bf16) {
    if (!d.untiled && !d.fp8) L.w_z = take(2 * wrows * p.H_pad);  // fp8: the forward needs no bf16 z
    L.w_stats = take(8 * wrows * p.nvt);
    L.w_hb = take(4 * wrows);
    L.w_hy = take(4 * wrows);
    if (persistent_scores(p)) {
      if (!d.fp8) L.w_WOp = take(2 * (size_t)p.nvt * 256 * p.H_pad);  // fp8: the E4M3 rows instead
      L.w_bl = take(4 * (size_t)p.nvt * 256);
    }
    if (d.fp8) {
      L.w_WO8 = take((size_t)p.nvt * 256 * p.H8);
      L.w_z8 = take(wrows * p.H8);
      L.w_ew = take(sizeof(int32_t));
    }
  }
  L.workspace_bytes = o;
  return L;
}

void serialize_plan(const Plan& p, const Layout& L, const int32_t* T_len, const int32_t* U_len,
                    std::vector<char>& out) {
  out.assign(L.plan_bytes, 0);
  const int B = p.d.B;
  std::memcpy(out.data() + L.off_Tlen, T_len, sizeof(int32_t) * B);
  std::memcpy(out.data() + L.off_Ulen, U_len, sizeof(int32_t) * B);
  if (!p.tiles.empty()) std::memcpy(out.data() + L.off_tiles, p.tiles.data(), sizeof(TileH) * p.tiles.size());
  if (!p.groups.empty()) std::memcpy(out.data() + L.off_groups, p.groups.data(), sizeof(GroupH) * p.groups.size());
  if (!p.gidx.empty()) std::memcpy(out.data() + L.off_gidx, p.gidx.data(), sizeof(int32_t) * p.gidx.size());
  std::memcpy(out.data() + L.off_latoff, p.lat_off.data(), sizeof(int64_t) * p.lat_off.size());
  if (!p.lat_pair.empty())
    std::memcpy(out.data() + L.off_latpair, p.lat_pair.data(), sizeof(int32_t) * p.lat_pair.size());
  if (!p.band_lo.empty()) std::memcpy(out.data() + L.off_band, p.band_lo.data(), sizeof(int32_t) * p.band_lo.size());
}

}  // namespace rnnt
