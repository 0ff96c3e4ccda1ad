// Host-side tile plan and buffer layout (plain C++, no HIP calls).
//
// The lattice of sample b (t < T_b, u <= U_b) is cut into tiles of at most
// tile_t x tile_u cells ("Flash RNN-T", section "Compute it, use it, make
// room": grid positions are grouped into tiles, and the working space of the
// joint intermediates depends on the tile size, not the recording length).
// Tiles are grouped into waves of at most tiles_per_wave tiles; only one
// wave's scores and z exist at a time in the backward. Padded cells are never
// part of any tile ("Neural transducer training ...", Introduction and
// Conclusion: padding removal).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "common_host.hpp"

namespace rnnt {

struct Dims {
  int B, T, U, V, HA, HL, H, blank;
  bool bf16;
  bool untiled;
  bool fp8;  // bf16 inputs, output-layer product of the score kernels on E4M3 operands (tiled only)
  int tile_t, tile_u, tiles_per_wave;
};

struct WaveInfo {
  int tile_begin, tile_end;
  int row_begin, row_end;      // global rows
  int strip_begin, strip_end;  // global strips
  int gA_begin, gA_end;        // group ranges
  int gL_begin, gL_end;
  int maxA_len, maxL_len;
};

// Pruned lattice: frame t of sample b keeps the label positions
// lo[b*T + t] <= u < lo[b*T + t] + S (host array; null lo = no pruning).
struct Band {
  const int32_t* lo = nullptr;
  int S = 0;
};

struct Plan {
  Dims d;
  std::vector<int32_t> band_lo;  // [B * T] copy of the caller's bands (empty: not pruned)
  int band_S = 0;
  int U1, H_pad, V_pad, KS, tile_tp, tpw;
  std::vector<TileH> tiles;
  std::vector<WaveInfo> waves;
  std::vector<GroupH> groups;
  std::vector<int32_t> gidx;
  std::vector<int64_t> lat_off;  // [B + 1] packed lattice block offsets (entries)
  // [2 B] lattice sweep pairing: samples by T_b - 1 + U_b, longest first
  // (ties by index); workgroup j sweeps alpha of the j-th longest and beta of
  // the j-th shortest
  std::vector<int32_t> lat_pair;
  int64_t total_rows = 0;
  int max_wave_rows = 0, max_wave_tiles = 0;
  int s6 = 1, s7a = 1, s7l = 1;  // split-K counts
  int nvt = 1;                   // 256-score tiles of the vocabulary (bf16 path)
  int H8 = 0;                    // fp8: bytes per row of the E4M3 operands (>= H_pad, >= 640; 0 otherwise)
};

// Byte offsets inside `saved` and `workspace` (all 256-byte aligned).
struct Layout {
  size_t plan_bytes;  // status + lengths + tiles + groups + gidx (one host->device copy)
  size_t off_status;  // int32 [2]: labels out of range, flat index of the first (-1 if none)
  size_t off_Tlen, off_Ulen, off_tiles, off_groups, off_gidx;
  size_t off_labels;  // int32 [B, U+1]: the labels the kernels read (range-checked copy)
  size_t off_latoff;  // int64 [B + 1]: packed lattice block offsets (part of the plan copy)
  size_t off_latpair; // int32 [2 B]: lattice sweep pairing (part of the plan copy)
  size_t off_band;    // int32 [B, T]: the bands of a pruned lattice (part of the plan copy; 0 if none)
  size_t lat_entries; // entries of each lattice array (lat_off[B])
  size_t off_a, off_l, off_lse, off_phi, off_psi, off_alpha, off_beta, off_lnP;
  bool lat64;  // alpha, beta, ln P held in fp64 (fp32 mode), else fp32
  // untiled only: the scores [total_rows, V_pad] (bf16 mode: scaled by log2 e,
  // bias included) and z (bf16: rows [total_rows + 128 rows of padding, H_pad],
  // the padding read by the last 128-row cell tile; fp32: z^T [H_pad, total_rows])
  size_t off_logits, off_z;
  size_t saved_bytes;
  size_t w_dh, w_z, w_gA, w_gL, w_PA, w_PL, w_PW, w_PB, w_PWA, w_PBZ, w_PWL, w_WOT;
  size_t w_zf, w_stats, w_hb, w_hy;  // bf16 forward: z rows, V-tile statistics, blank/label scores
  size_t w_WOp, w_bl;        // persistent score kernels: padded W^O, bias table
  size_t w_coefA, w_coefB;   // bf16 backward coefficients per wave row (persistent kernels, untiled mode)
  size_t w_WO8, w_z8, w_ew;              // fp8: E4M3 W^O rows, z rows, W^O scale exponent (int)
  size_t w_gb;  // bf16: rounded gA, gL for the encoder-side products (may alias w_dh)
  size_t w_WAT, w_WLT;  // bf16: W^A^T [HA, H], W^L^T [HL, H] for dh^A, dh^L
  size_t w_hs;          // bf16: h^A, h^L with padding rows zeroed, for dW^A, dW^L (may alias w_dh)
  size_t workspace_bytes;
};

// Rows of the plan's row space (and so of any wave) must stay below this:
// row numbers are int32 in the plan records and the kernels, and wave
// buffers round the rows up to whole 128-row cell tiles.
constexpr int64_t kMaxPlanRows = ((int64_t)1 << 31) - 1 - 256;

// K steps of 16 for hidden size H on the MFMA cores (H_pad = 16 * result),
// -1 if H is too large.
int joint_ks_for(int H);
// Validates dims and lengths; on failure returns false and sets err.
bool check_dims(const Dims& d, std::string& err, int& status);
bool check_lengths(const Dims& d, const int32_t* T_len, const int32_t* U_len, std::string& err);
// A band must hold an alignment: S >= 1, lo[b, 0] = 0, lo non-decreasing in t
// with steps of at most S - 1, 0 <= lo <= U_b, and the last frame's band
// reaching U_b. Frames t >= T_b are not read.
bool check_band(const Dims& d, const int32_t* T_len, const int32_t* U_len, const Band& band, std::string& err);
// Builds the tile plan (deterministic in its inputs). With a band, tiles
// holding no cell of any frame's band are left out.
void build_plan(const Dims& d, const int32_t* T_len, const int32_t* U_len, int H_pad, Plan& p,
                const Band& band = Band());
// Checks a built plan against the library's 32-bit row limits (kMaxPlanRows).
bool check_plan(const Plan& p, std::string& err);
// Whether the bf16 score products run on the persistent score kernels: they
// need at least 8 stages of 64 k per item (the previous item's epilogue runs
// in the first five); the fp8 output layer always uses them (its operand rows
// are padded to at least five stages of 128 bytes).
bool persistent_scores(const Plan& p);
Layout make_layout(const Plan& p);
// The same layout with only the forward pass's workspace regions (z rows,
// V-tile statistics, blank / label scores, padded W^O and bias table) packed
// from offset 0; workspace_bytes is then the forward's need alone. The other
// workspace offsets are not valid in it.
Layout make_forward_layout(const Plan& p);
// Serializes lengths, tiles, groups and gidx in layout order into out
// (plan_bytes bytes, offsets relative to the start of `saved`).
void serialize_plan(const Plan& p, const Layout& L, const int32_t* T_len, const int32_t* U_len,
                    std::vector<char>& out);

}  // namespace rnnt
