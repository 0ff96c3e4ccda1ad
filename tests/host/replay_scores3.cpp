// Host replay of the persistent score kernels' work and address mapping.
//
// For each case read from stdin, builds the tile plan and buffer layout with
// the library's own host code (plan.cpp), then walks, for every wave of the
// plan and for the forward and the backward kernel, every workgroup of the
// 256-workgroup launch through every stage its pipeline issues (the
// prologue's three, then one per stage, past the last item included) and
// every item whose epilogue it runs, using the same constexpr mapping the
// kernel uses (scores3_map.hpp). It checks that
//   - every item's cell tile ct lies in [0, n_ct) and V tile vt in [0, nvt),
//   - the n_ct cell tiles of 128 rows fit in the wave buffers,
//   - every dma source byte range (padded W^O rows, z rows, bias values, the
//     backward coefficients) and every epilogue store range (the forward's
//     per-V-tile statistics, the backward's dh rows) lies inside the buffer
//     region the layout reserves for it.
// In untiled mode (one wave; the forward alone runs on these kernels) the z
// rows are the ones kept in `saved`, and the stored scores (rows of the wave
// only) must lie inside the saved scores.
// Nothing is launched: this is plain C++ against the plan and layout.
//
// Input, one case per line: B T U V HA HL H dtype untiled tile_t tile_u tpw
// (dtype 0 fp32, 1 bf16, 2 bf16 with the fp8 output layer),
// then B values of T_len and B values of U_len, optionally followed by a
// band width S and B * T band starts (a pruned lattice). Output per case:
// "ok <stages checked> tiles <n>" or "skip <reason>" or "FAIL <what>".
#include <stdint.h>

#include <algorithm>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "plan.hpp"
#include "scores3_map.hpp"

using namespace rnnt;

namespace {

struct Region {
  int64_t begin, end;
};

// The region that starts at `off`: up to the next region's offset (or the
// end of the buffer), i.e. the bytes the layout reserves for it.
Region region(int64_t off, const std::vector<int64_t>& offs, int64_t total) {
  int64_t end = total;
  for (int64_t o : offs)
    if (o > off) end = std::min(end, o);
  return Region{off, end};
}

bool inside(const Region& r, int64_t lo, int64_t hi) { return lo >= r.begin && hi <= r.end && lo <= hi; }

std::string run_case(const Dims& d, const std::vector<int32_t>& T_len, const std::vector<int32_t>& U_len,
                     const Band& band, int64_t& checked) {
  std::string err;
  int st = 0;
  if (!check_dims(d, err, st)) return "skip " + err;
  if (!check_lengths(d, T_len.data(), U_len.data(), err)) return "skip " + err;
  if (band.lo && !check_band(d, T_len.data(), U_len.data(), band, err)) return "skip " + err;
  const int ks = joint_ks_for(d.H);
  if (ks < 0) return "skip H";
  Plan p;
  build_plan(d, T_len.data(), U_len.data(), ks * 16, p, band);
  if (!check_plan(p, err)) return "skip " + err;
  const Layout L = make_layout(p);
  // the lattice sweep pairing: every sample once in the alpha role and once in
  // the beta role, alpha longest first (T_b - 1 + U_b), beta the mirror order,
  // and the table inside the plan copy
  {
    if ((int64_t)p.lat_pair.size() != 2 * (int64_t)d.B) return "FAIL pairing table size";
    if (L.off_latpair + sizeof(int32_t) * p.lat_pair.size() > L.plan_bytes) return "FAIL pairing outside the plan copy";
    std::vector<int> n_alpha(d.B, 0), n_beta(d.B, 0);
    auto D = [&](int b) { return T_len[b] - 1 + U_len[b]; };
    for (int j = 0; j < d.B; ++j) {
      const int a = p.lat_pair[2 * j], b = p.lat_pair[2 * j + 1];
      if (a < 0 || a >= d.B || b < 0 || b >= d.B) return "FAIL pairing index out of range";
      ++n_alpha[a];
      ++n_beta[b];
      if (b != p.lat_pair[2 * (d.B - 1 - j)]) return "FAIL pairing not mirrored";
      if (j > 0 && D(a) > D(p.lat_pair[2 * (j - 1)])) return "FAIL pairing not longest first";
    }
    for (int b = 0; b < d.B; ++b)
      if (n_alpha[b] != 1 || n_beta[b] != 1) return "FAIL pairing not one sweep of each kind per sample";
  }
  // the persistent score kernels run in bf16 mode with at least 8 k-steps of 64, and
  // always with the fp8 output layer (E4M3 rows of H8 >= 640 bytes)
  if (!persistent_scores(p)) return "skip not the persistent score path";
  std::vector<int64_t> offs = {
      (int64_t)L.w_dh, (int64_t)L.w_z, (int64_t)L.w_gA, (int64_t)L.w_gL, (int64_t)L.w_PA, (int64_t)L.w_PL,
      (int64_t)L.w_PW, (int64_t)L.w_PB, (int64_t)L.w_PWA, (int64_t)L.w_PBZ, (int64_t)L.w_PWL, (int64_t)L.w_WOT,
      (int64_t)L.w_stats, (int64_t)L.w_hb, (int64_t)L.w_hy, (int64_t)L.w_WOp, (int64_t)L.w_bl,
      (int64_t)L.w_coefA, (int64_t)L.w_coefB, (int64_t)L.w_WAT, (int64_t)L.w_WLT};
  if (d.fp8)
    for (size_t o : {L.w_WO8, L.w_z8, L.w_ew}) offs.push_back((int64_t)o);
  // the rounded gA / gL and the masked encodings live in the wave buffers
  // (dead after the last wave) when they fit there, else in regions of their own
  for (size_t o : {L.w_gb, L.w_hs})
    if (o >= L.w_coefB) offs.push_back((int64_t)o);
  const int64_t W = (int64_t)L.workspace_bytes;
  // the operands: bf16 rows of H_pad values, or (fp8) E4M3 rows of H8 bytes, which the
  // kernel addresses as rows of H8 / 2 two-byte units
  const size_t off_z = d.fp8 ? L.w_z8 : L.w_z, off_wo = d.fp8 ? L.w_WO8 : L.w_WOp;
  const Region rdh = region(L.w_dh, offs, W), rst = region(L.w_stats, offs, W);
  // untiled: z and the scores in `saved` (global rows), the last two regions there
  const std::vector<int64_t> soffs = {(int64_t)L.off_a, (int64_t)L.off_l, (int64_t)L.off_lse, (int64_t)L.off_phi,
                                      (int64_t)L.off_psi, (int64_t)L.off_alpha, (int64_t)L.off_beta,
                                      (int64_t)L.off_lnP, (int64_t)L.off_logits, (int64_t)L.off_z};
  const int64_t SB = (int64_t)L.saved_bytes;
  const Region rz = d.untiled ? region(L.off_z, soffs, SB) : region(off_z, offs, W);
  const Region rlg = d.untiled ? region(L.off_logits, soffs, SB) : Region{0, 0};
  const Region rwo = region(off_wo, offs, W), rbl = region(L.w_bl, offs, W), rco = region(L.w_coefA, offs, W);
  const int64_t buf_rows = (p.max_wave_rows + 127) / 128 * 128;
  const int hrow = d.fp8 ? p.H8 / 2 : p.H_pad;
  const int nvt = p.nvt, nq = hrow / s3map::BK, nbuf = d.fp8 ? 3 : 2;
  const int64_t z_ld = hrow;
  if (d.fp8 && (p.H8 % 128 != 0 || nq < 5)) return "FAIL fp8 operand rows shorter than five stages";

  // per-thread dma offsets relative to a stage's source, over all threads
  // and instructions of an operand: [lo, hi) in bytes
  auto dma_span = [&](int nd, int ld, int64_t& lo, int64_t& hi) {
    lo = INT64_MAX;
    hi = INT64_MIN;
    const int64_t step32 = (int64_t)32 * ld * 2;
    for (int tid = 0; tid < s3map::kThreads; ++tid) {
      const int wave = tid >> 6, lane = tid & 63;
      const uint32_t o0 = s3map::dma_thread_off(0, wave, lane, ld), o1 = s3map::dma_thread_off(1, wave, lane, ld);
      for (int dd = 0; dd < nd; ++dd) {
        const int64_t o = s3map::dma_off(dd, o0, o1, step32);
        lo = std::min(lo, o);
        hi = std::max(hi, o + 16);
      }
    }
  };
  int64_t a_lo, a_hi, b_lo, b_hi;
  dma_span(s3map::NDA, hrow, a_lo, a_hi);
  dma_span(s3map::NDB, (int)z_ld, b_lo, b_hi);

  for (size_t w = 0; w < p.waves.size(); ++w) {
    const WaveInfo& wv = p.waves[w];
    const int n_rows = wv.row_end - wv.row_begin;
    const int n_ct = (n_rows + 127) / 128;
    std::ostringstream where;
    where << "wave " << w << " (rows " << n_rows << ", n_ct " << n_ct << ")";
    if ((int64_t)n_ct * 128 > buf_rows) return "FAIL " + where.str() + ": cell tiles exceed the wave buffer rows";
    if (n_rows <= 0) return "FAIL " + where.str() + ": empty wave";
    // untiled: the wave's z rows start at its first global row
    const int64_t zbase = d.untiled ? (int64_t)L.off_z + (int64_t)wv.row_begin * z_ld * 2 : (int64_t)off_z;
    for (int bwd = 0; bwd < (d.untiled ? 1 : 2); ++bwd) {
      for (int blk = 0; blk < s3map::kGrid; ++blk) {
        const int xcd = blk & 7, slot = blk >> 3;
        const int nctl = s3map::nctl_of(n_ct, xcd);
        const int n_items = s3map::items_of(n_ct, nvt, xcd, slot);
        if (n_items == 0) continue;
        auto bad = [&](const std::string& what, int S) {
          std::ostringstream o;
          o << "FAIL " << where.str() << (bwd ? " bwd" : " fwd") << " block " << blk << " stage " << S << ": "
            << what;
          return o.str();
        };
        // stages 0 .. 2 from the prologue, then S + 3 during stage S
        const int last_S = n_items * nq - 1 + 3;
        for (int S = 0; S <= last_S; ++S) {
          const s3map::Item it = s3map::item_of(S / nq, n_items, nctl, nvt, xcd, slot);
          if (it.ct < 0 || it.ct >= n_ct) return bad("cell tile " + std::to_string(it.ct) + " out of range", S);
          if (it.vt < 0 || it.vt >= nvt) return bad("V tile " + std::to_string(it.vt) + " out of range", S);
          const s3map::StageSrc o = s3map::stage_src(S, nq, n_items, nctl, nvt, xcd, slot, hrow, z_ld, nbuf);
          if (!inside(rwo, off_wo + o.a + a_lo, off_wo + o.a + a_hi)) return bad("W^O rows outside", S);
          if (!inside(rz, zbase + o.b + b_lo, zbase + o.b + b_hi)) return bad("z rows outside", S);
          if (o.par < 0 || o.par >= nbuf) return bad("bias buffer index out of range", S);
          // the z rows a stage reads belong to its cell tile's 128 rows
          if (o.b + b_lo < (int64_t)it.ct * 128 * z_ld * 2 || o.b + b_hi > ((int64_t)it.ct + 1) * 128 * z_ld * 2)
            return bad("z bytes outside the item's cell tile", S);
          if (!inside(rbl, L.w_bl + o.bias, L.w_bl + o.bias + 4 * s3map::kThreads)) return bad("bias outside", S);
          if (bwd && !inside(rco, L.w_coefA + o.coef, L.w_coefA + o.coef + 4 * s3map::kThreads))
            return bad("coefficients outside", S);
          ++checked;
        }
        // epilogue stores of every item: rows ct*128 .. +127, V tile columns
        for (int n = 0; n < n_items; ++n) {
          const s3map::Item it = s3map::item_of(n, n_items, nctl, nvt, xcd, slot);
          const int64_t r0 = (int64_t)it.ct * s3map::BN, r1 = r0 + s3map::BN;
          if (!bwd) {
            // stats[row][vt] as (max, sum) float pairs
            if (!inside(rst, L.w_stats + 8 * (r0 * nvt + it.vt), L.w_stats + 8 * ((r1 - 1) * nvt + it.vt) + 8))
              return bad("statistics store outside", -1);
            // untiled: the scores of rows r0 .. min(r1, n_rows) - 1, V tile columns
            if (d.untiled && r0 < n_rows) {
              const int64_t g0 = (int64_t)wv.row_begin + r0, g1 = (int64_t)wv.row_begin + std::min<int64_t>(r1, n_rows);
              if (!inside(rlg, L.off_logits + 2 * (g0 * p.V_pad + (int64_t)it.vt * 256),
                          L.off_logits + 2 * ((g1 - 1) * p.V_pad + (int64_t)it.vt * 256 + 256)))
                return bad("scores store outside", -1);
            }
          } else {
            if (!inside(rdh, L.w_dh + 2 * (r0 * p.V_pad + (int64_t)it.vt * 256),
                        L.w_dh + 2 * ((r1 - 1) * p.V_pad + (int64_t)it.vt * 256 + 256)))
              return bad("dh store outside", -1);
          }
        }
      }
    }
  }
  return "ok " + std::to_string(checked) + " tiles " + std::to_string(p.tiles.size());
}

}  // namespace

int main() {
  std::string line;
  int fails = 0;
  while (std::getline(std::cin, line)) {
    if (line.empty()) continue;
    std::istringstream in(line);
    Dims d{};
    int bf = 0, un = 0;
    in >> d.B >> d.T >> d.U >> d.V >> d.HA >> d.HL >> d.H >> bf >> un >> d.tile_t >> d.tile_u >> d.tiles_per_wave;
    d.blank = 0;
    d.bf16 = bf != 0;
    d.fp8 = bf == 2;
    d.untiled = un != 0;
    std::vector<int32_t> T_len(d.B), U_len(d.B);
    for (auto& x : T_len) in >> x;
    for (auto& x : U_len) in >> x;
    // optional: band width S > 0, then B * T band starts
    Band band;
    std::vector<int32_t> lo;
    int S = 0;
    if (in >> S && S > 0) {
      lo.resize((size_t)d.B * d.T);
      for (auto& x : lo) in >> x;
      band.lo = lo.data();
      band.S = S;
    }
    in.clear();
    if (!in) {
      std::cout << "FAIL bad input line" << std::endl;
      ++fails;
      continue;
    }
    int64_t checked = 0;
    const std::string r = run_case(d, T_len, U_len, band, checked);
    if (r.rfind("FAIL", 0) == 0) ++fails;
    std::cout << r << std::endl;
  }
  return fails ? 1 : 0;
}
