// Fused joint network + output layer kernels for gfx950.
//
// Forward ("Flash RNN-T", section "Making each operation more efficient": the
// joint kernel and the scores -> two probabilities kernel, here one kernel):
// per lattice cell (b,t,u)
//   z = tanh(a[b,t] + l[b,u])   with a = W^A h^A + b^Z, l = W^L h^L
//   h = W^O z + b^O              (V scores, never written in tiled mode)
//   lse = logsumexp(h), phi = h[blank] - lse, psi = h[y[u+1]] - lse
// ("Neural transducer training ...", section "Transducer training", Eqs.
// (4)-(7): only the softmax denominator is kept, not the probabilities).
//
// Backward recompute ("Flash RNN-T", section "Compute it, use it, make room":
// each tile's scores are recreated in the backward): the same MFMA sequence
// reproduces the forward's scores bit for bit, and the epilogue turns them
// into dh = g*(occ*softmax - [v=blank]*bflow - [v=y]*lflow) (Eq. (10)),
// written to the wave buffer, together with z for the weight gradients.
//
// Work decomposition: a wave owns ROWS consecutive rows of the plan's row
// space (ROWS consecutive t at one u of one tile) and keeps their z as MFMA
// A-fragments in registers for the whole of H, so tanh runs once per cell.
// The four waves of a workgroup share W^O, streamed through LDS in
// 128-score x 128-byte stages (double buffered, XOR-swizzled). The online
// logsumexp runs on the accumulators in the MFMA output layout; the blank and
// label scores come from dot products of the z fragments with the two W^O
// rows, so no score is ever gathered from registers by column.
#include "common.hpp"
#include "kernels.hpp"

namespace rnnt {

namespace {

constexpr int BN = 128;  // scores per V chunk

template <class M>
struct StageRegs {
  u32x4 v[4];
};

// One W^O stage: rows v in [vc*BN, vc*BN+BN), k elements [qs*8*KPL, +8*KPL).
template <class M>
__device__ inline void load_wo_stage(StageRegs<M>& r, const typename M::CT* WO, int V, int H, int vc,
                                     int qs, int tid) {
  constexpr int KPL = M::KPL;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int p = i * 256 + tid;
    int vrow = p >> 3, c = p & 7;
    int v = vc * BN + vrow;
    int k = qs * 8 * KPL + c * KPL;
    if (v < V && k < H) {
      r.v[i] = ldg<u32x4>(WO + (size_t)v * H + k);
    } else {
      r.v[i] = u32x4{0, 0, 0, 0};
    }
  }
}

template <class M>
__device__ inline void store_wo_stage(const StageRegs<M>& r, char* buf, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int p = i * 256 + tid;
    int vrow = p >> 3, c = p & 7;
    *reinterpret_cast<u32x4*>(buf + lds_off(vrow, c)) = r.v[i];
  }
}

// Locate the tile holding global row R0 among tiles [lo, hi].
// Backward weights of cell (t, u) of sample b, each times the cost's
// incoming gradient g: the occupancy exp(alpha + beta - ln P) and the blank
// and label flows exp(alpha + phi + beta(t+1, u) - ln P), exp(alpha + psi +
// beta(t, u+1) - ln P) (zero past the last label). R is the storage type of
// alpha, beta and ln P; the exponents are formed in R and rounded once.
template <typename R>
__device__ inline void cell_weights(const R* al, const R* be, R lp, const float* phi, const float* psi,
                                    const LatGeo& geo, int t, int u, int Tb, int Ub, float g, float& occ, float& cb,
                                    float& cl) {
  const int64_t idx = lat_at(geo, t, u);
  const R A = al[idx];
  const R bn = (t + 1 < Tb) ? be[lat_at(geo, t + 1, u)] : (u == Ub ? R(0) : R(kNegInf));
  occ = g * fexp2((float)(A + be[idx] - lp) * kLog2e);
  cb = g * fexp2((float)(A + (R)phi[idx] + bn - lp) * kLog2e);
  cl = 0.0f;
  if (u < Ub) cl = g * fexp2((float)(A + (R)psi[idx] + be[lat_at(geo, t, u + 1)] - lp) * kLog2e);
}

__device__ inline int find_tile_by_row(const Tile* tiles, int lo, int hi, int R0) {
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (tiles[mid].row0 <= R0) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace

template <class M, int KS, bool BWD>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
joint_kernel(JointArgs p) {
  using CT = typename M::CT;
  using Frag = typename M::Frag;
  using Acc = typename M::Acc;
  constexpr int ROWS = M::ROWS, KPL = M::KPL, NACC = M::NACC;
  constexpr int SPS = 8 / M::GROUPS;  // k-steps per stage
  static_assert(KS % SPS == 0, "H_pad must fill whole stages");
  constexpr int SPV = KS / SPS;       // stages per V chunk
  constexpr int NB = BN / ROWS;       // output blocks per V chunk

  __shared__ __attribute__((aligned(16))) char stage_buf[2][BN * 128];
  __shared__ float row_lds[4][4][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chunk = blockIdx.x * 4 + wave;
  const bool active = chunk < p.n_chunks;
  const int r = lane % ROWS;        // this lane's A row
  const int g = lane / ROWS;        // this lane's k group

  const CT* WO = reinterpret_cast<const CT*>(p.WO);
  const CT* bO = reinterpret_cast<const CT*>(p.bO);
  const int V = p.V, H = p.H, T = p.T, U1 = p.U1;

  // ---- which cells: ROWS consecutive t at one u of one tile
  int b = 0, u = 0, tbase = 0, nvalid = 0, Tb = 1, Ub = 0, R0 = 0;
  if (active) {
    R0 = p.row_begin + chunk * ROWS;
    int ti = find_tile_by_row(p.tiles, p.tile_begin, p.tile_end - 1, R0);
    Tile tl = p.tiles[ti];
    int local = R0 - tl.row0;
    int ul = local / tl.htp;
    int tl0 = local - ul * tl.htp;
    b = tl.b;
    u = tl.u0 + ul;
    tbase = tl.t0 + tl0;
    nvalid = tl.ht - tl0;
    Tb = p.T_len[b];
    Ub = p.U_len[b];
  }
  const bool row_ok = active && r < nvalid;
  const int t_r = tbase + r;
  const int lab_r = (active && u < Ub) ? p.labels[(size_t)b * U1 + u + 1] : -1;

  // ---- z = tanh(a[t] + l[u]) as A fragments, once per cell
  Frag Z[KS];
  {
    const float* arow = p.a + ((size_t)b * T + (row_ok ? t_r : 0)) * p.H_pad;
    const float* lrow = p.l + ((size_t)b * U1 + u) * p.H_pad;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      int k = s * 16 + g * KPL;
      Frag z;
      if (row_ok) {
#pragma unroll
        for (int e4 = 0; e4 < KPL; e4 += 4) {
          f32x4 av = ldg<f32x4>(arow + k + e4);
          f32x4 lv = ldg<f32x4>(lrow + k + e4);
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e4 + e] = to_ct<CT>(joint_act<CT>(av[e] + lv[e]));
        }
      } else {
#pragma unroll
        for (int e = 0; e < KPL; ++e) z[e] = to_ct<CT>(0.0f);
      }
      Z[s] = z;
    }
  }
  const bool write_z = BWD || p.store;
  if (active && write_z) {
    // z^T: lanes with consecutive rows write consecutive addresses of one h row
    CT* zcol = reinterpret_cast<CT*>(p.z_out) + (R0 - p.buf_row_base + r);
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int e = 0; e < KPL; ++e) zcol[(int64_t)(s * 16 + g * KPL + e) * p.z_ld] = Z[s][e];
  }

  // ---- blank and label scores by dot products with the two W^O rows
  float hb = 0.0f, hy = 0.0f;
  if (row_ok) {
    const CT* wb = WO + (size_t)p.blank * H;
    const CT* wy = WO + (size_t)(lab_r >= 0 ? lab_r : 0) * H;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      int k = s * 16 + g * KPL;
      if (k < H) {
        Frag xb = ldg<Frag>(wb + k);
        Frag xy = ldg<Frag>(wy + k);
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
          float zf = to_f32(Z[s][e]);
          hb = __builtin_fmaf(zf, to_f32(xb[e]), hb);
          hy = __builtin_fmaf(zf, to_f32(xy[e]), hy);
        }
      }
    }
  }
#pragma unroll
  for (int off = ROWS; off < 64; off <<= 1) {
    hb += __shfl_xor(hb, off);
    hy += __shfl_xor(hy, off);
  }
  hb += to_f32(bO[p.blank]);
  if (lab_r >= 0) hy += to_f32(bO[lab_r]);

  // ---- per-row backward coefficients: lse, g*occ, g*bflow, g*lflow
  float r_lse[NACC], r_occ[NACC];
  // rows that are no cell keep lse = +inf: their dh is exactly 0 for any score
  float my_lse = kPosInf, my_occ = 0.0f, my_cb = 0.0f, my_cl = 0.0f;
  if (BWD) {
    if (g == 0) {
      if (row_ok) {
        const LatGeo geo = lat_geo(p.lat_off, p.U_len, b);
        size_t idx = (size_t)lat_at(geo, t_r, u);
        float gb = p.dcosts ? p.dcosts[b] : 1.0f;
        my_lse = p.lse[idx];
        if (p.alpha64)
          cell_weights<double>(p.alpha64, p.beta64, p.lnP64[b], p.phi, p.psi, geo, t_r, u, Tb, Ub, gb, my_occ,
                               my_cb, my_cl);
        else
          cell_weights<float>(p.alpha, p.beta, p.lnP[b], p.phi, p.psi, geo, t_r, u, Tb, Ub, gb, my_occ, my_cb,
                              my_cl);
      }
      row_lds[wave][0][r] = my_lse;
      row_lds[wave][1][r] = my_occ;
      row_lds[wave][2][r] = my_cb;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < NACC; ++e) {
      int rr = M::row_of(e, lane);
      r_lse[e] = row_lds[wave][0][rr] * kLog2e;
      r_occ[e] = row_lds[wave][1][rr];
    }
  }

  // ---- stream W^O over V chunks
  float run_m[NACC], run_s[NACC];
#pragma unroll
  for (int e = 0; e < NACC; ++e) {
    run_m[e] = -1e30f;
    run_s[e] = 0.0f;
  }
  Acc acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = Acc{};

  const int VC = (V + BN - 1) / BN;
  const int NS = VC * SPV;  // stages in total
  // Pipeline: stage q is in LDS buffer q&1, stage q+1 in register set (q+1)&1;
  // stage q+2 is requested at the top of step q. SPV is even, so q&1 == qs&1.
  static_assert(SPV % 2 == 0, "stages per V chunk must be even");
  StageRegs<M> sr[2];
  load_wo_stage<M>(sr[0], WO, V, H, 0, 0, tid);
  if (NS > 1) load_wo_stage<M>(sr[1], WO, V, H, 0, 1, tid);
  store_wo_stage<M>(sr[0], stage_buf[0], tid);
  __syncthreads();
  CT* dh_base = BWD ? reinterpret_cast<CT*>(p.logits_out) : nullptr;
  CT* lg_base = (!BWD && p.store) ? reinterpret_cast<CT*>(p.logits_out) : nullptr;

  for (int vc = 0; vc < VC; ++vc) {
#pragma unroll
    for (int qs = 0; qs < SPV; ++qs) {
      const int q = vc * SPV + qs;
      const bool last_q = (qs + 1 == SPV);
      if (q + 2 < NS) {
        const int qs2 = (qs + 2) % SPV;
        const int vc2 = vc + (qs + 2) / SPV;
        load_wo_stage<M>(sr[qs & 1], WO, V, H, vc2, qs2, tid);
      }
      if (active) {
        const char* buf = stage_buf[qs & 1];
#pragma unroll
        for (int ss = 0; ss < SPS; ++ss) {
#pragma unroll
          for (int n = 0; n < NB; ++n) {
            Frag bf = *reinterpret_cast<const Frag*>(buf + lds_off(n * ROWS + r, ss * M::GROUPS + g));
            acc[n] = M::mma(Z[qs * SPS + ss], bf, acc[n]);
          }
        }
      }
      if (last_q && active) {
        // ---------------- epilogue on one V chunk
        if (!BWD) {
          float bias[NB];
          bool okc[NB];
#pragma unroll
          for (int n = 0; n < NB; ++n) {
            int col = vc * BN + n * ROWS + M::col_of(lane);
            okc[n] = col < V;
            bias[n] = okc[n] ? to_f32(bO[col]) : 0.0f;
          }
#pragma unroll
          for (int e = 0; e < NACC; ++e) {
            float cm = -1e30f;
#pragma unroll
            for (int n = 0; n < NB; ++n)
              if (okc[n]) cm = __builtin_fmaxf(cm, acc[n][e] + bias[n]);
            float mn = __builtin_fmaxf(run_m[e], cm);
            float sum = run_s[e] * fexp2((run_m[e] - mn) * kLog2e);
            float mnl = mn * kLog2e;
#pragma unroll
            for (int n = 0; n < NB; ++n)
              if (okc[n]) sum += fexp2(__builtin_fmaf(acc[n][e] + bias[n], kLog2e, -mnl));
            run_s[e] = sum;
            run_m[e] = mn;
          }
          if (lg_base) {
#pragma unroll
            for (int n = 0; n < NB; ++n) {
              int col = vc * BN + n * ROWS + M::col_of(lane);
              if (col < p.V_pad) {
#pragma unroll
                for (int e = 0; e < NACC; ++e) {
                  size_t row = (size_t)(R0 - p.buf_row_base + M::row_of(e, lane));
                  lg_base[row * p.V_pad + col] = to_ct<CT>(okc[n] ? acc[n][e] + bias[n] : 0.0f);
                }
              }
            }
          }
        } else {
#pragma unroll
          for (int n = 0; n < NB; ++n) {
            int col = vc * BN + n * ROWS + M::col_of(lane);
            if (col < p.V_pad) {
              bool okc = col < V;
              float bias = okc ? to_f32(bO[col]) : 0.0f;
              bool is_blank = col == p.blank;
#pragma unroll
              for (int e = 0; e < NACC; ++e) {
                int rr = M::row_of(e, lane);
                float x = acc[n][e] + bias;
                float d = r_occ[e] * fexp2(__builtin_fmaf(x, kLog2e, -r_lse[e]));
                if (is_blank) d -= row_lds[wave][2][rr];
                if (!okc) d = 0.0f;
                dh_base[(size_t)(R0 - p.buf_row_base + rr) * p.V_pad + col] = to_ct<CT>(d);
              }
            }
          }
        }
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[n] = Acc{};
      }
      if (q + 1 < NS) store_wo_stage<M>(sr[(qs + 1) & 1], stage_buf[(qs + 1) & 1], tid);
      __syncthreads();
    }
  }

  if (!BWD) {
    // combine the per-lane running (max, sum) across the lanes sharing rows
#pragma unroll
    for (int e = 0; e < NACC; ++e) {
#pragma unroll
      for (int off = 1; off < ROWS; off <<= 1) {
        float m2 = __shfl_xor(run_m[e], off);
        float s2 = __shfl_xor(run_s[e], off);
        float mn = __builtin_fmaxf(run_m[e], m2);
        run_s[e] = run_s[e] * fexp2((run_m[e] - mn) * kLog2e) + s2 * fexp2((m2 - mn) * kLog2e);
        run_m[e] = mn;
      }
    }
    if (active && M::col_of(lane) == 0) {
#pragma unroll
      for (int e = 0; e < NACC; ++e)
        row_lds[wave][0][M::row_of(e, lane)] = run_m[e] + kLn2 * flog2(run_s[e]);
    }
    __syncthreads();
    if (row_ok && g == 0) {
      float ls = row_lds[wave][0][r];
      size_t idx = (size_t)lat_at(lat_geo(p.lat_off, p.U_len, b), t_r, u);
      // a pruned lattice's cells outside their frame's band emit nothing
      bool in_band = true;
      if (p.band_lo) {
        const int lo = p.band_lo[(size_t)b * T + t_r];
        in_band = u >= lo && u < lo + p.band_S;
      }
      p.lse_out[idx] = ls;
      p.phi_out[idx] = in_band ? hb - ls : kNegInf;
      p.psi_out[idx] = (in_band && u < Ub) ? hy - ls : kNegInf;
    }
  } else {
    // the label column: g*occ*softmax - g*lflow (- g*bflow when the label is blank)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (row_ok && g == 0 && u < Ub) {
      float d = my_occ * fexp2(__builtin_fmaf(hy, kLog2e, -my_lse * kLog2e)) - my_cl;
      if (lab_r == p.blank) d -= my_cb;
      dh_base[(size_t)(R0 - p.buf_row_base + r) * p.V_pad + lab_r] = to_ct<CT>(d);
    }
  }
}

// Backward of the fp32 untiled mode: the forward kept the scores (bias
// included), so dh is formed in place from them without recomputation.
template <class CT>
__global__ void __launch_bounds__(256) dh_inplace_kernel(DhInplaceArgs p) {
  __shared__ float coef[4][5];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t rowg = (int64_t)blockIdx.x * 4 + wave;  // global row of the row space
  if (rowg >= p.n_rows) return;
  const int R0 = p.row_begin + (int)rowg;
  int lo = p.tile_begin, hi = p.tile_end - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (p.tiles[mid].row0 <= R0) lo = mid; else hi = mid - 1;
  }
  Tile tl = p.tiles[lo];
  int local = R0 - tl.row0;
  int ul = local / tl.htp;
  int tloc = local - ul * tl.htp;
  int b = tl.b, u = tl.u0 + ul, t = tl.t0 + tloc;
  bool valid = tloc < tl.ht;
  const int T = p.T, U1 = p.U1;
  int Tb = p.T_len[b], Ub = p.U_len[b];
  if (lane == 0) {
    float ls = 0, co = 0, cb = 0, cl = 0;
    float lab = -1;
    if (valid) {
      const LatGeo geo = lat_geo(p.lat_off, p.U_len, b);
      size_t idx = (size_t)lat_at(geo, t, u);
      float gb = p.dcosts ? p.dcosts[b] : 1.0f;
      ls = p.lse[idx];
      if (p.alpha64)
        cell_weights<double>(p.alpha64, p.beta64, p.lnP64[b], p.phi, p.psi, geo, t, u, Tb, Ub, gb, co, cb, cl);
      else
        cell_weights<float>(p.alpha, p.beta, p.lnP[b], p.phi, p.psi, geo, t, u, Tb, Ub, gb, co, cb, cl);
      if (u < Ub) lab = (float)p.labels[(size_t)b * U1 + u + 1];
    }
    coef[wave][0] = ls * kLog2e;
    coef[wave][1] = co;
    coef[wave][2] = cb;
    coef[wave][3] = cl;
    coef[wave][4] = lab;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  float lsl = coef[wave][0], co = coef[wave][1], cb = coef[wave][2], cl = coef[wave][3];
  int lab = (int)coef[wave][4];
  CT* row = reinterpret_cast<CT*>(p.logits) + (size_t)(R0 - p.buf_row_base) * p.V_pad;
  for (int c = lane; c < p.V_pad; c += 64) {
    float d = 0.0f;
    if (valid && c < p.V) {
      float x = to_f32(row[c]);
      d = co * fexp2(__builtin_fmaf(x, kLog2e, -lsl));
      if (c == p.blank) d -= cb;
      if (c == lab) d -= cl;
    }
    row[c] = to_ct<CT>(d);
  }
}

// ---------------------------------------------------------------- launchers
template <class M, bool BWD>
static hipError_t launch_joint_h(const JointArgs& a, int KS, hipStream_t st) {
  dim3 grid((a.n_chunks + 3) / 4), block(256);
  if (grid.x == 0) return hipSuccess;
#define RNNT_KS_CASE(ks) \
  case ks: hipLaunchKernelGGL((joint_kernel<M, ks, BWD>), grid, block, 0, st, a); break;
  switch (KS) {
    RNNT_KS_CASE(8)
    RNNT_KS_CASE(16)
    RNNT_KS_CASE(24)
    RNNT_KS_CASE(32)
    RNNT_KS_CASE(40)
    RNNT_KS_CASE(48)
    default: return hipErrorInvalidValue;
  }
#undef RNNT_KS_CASE
  return hipGetLastError();
}

hipError_t launch_joint(const JointArgs& a, bool bf16_mode, bool bwd, hipStream_t st) {
  int KS = a.H_pad / 16;
  if (bf16_mode) {
    return bwd ? launch_joint_h<MfmaBf16, true>(a, KS, st) : launch_joint_h<MfmaBf16, false>(a, KS, st);
  }
  return bwd ? launch_joint_h<MfmaF32, true>(a, KS, st) : launch_joint_h<MfmaF32, false>(a, KS, st);
}

hipError_t launch_dh_inplace(const DhInplaceArgs& a, hipStream_t st) {
  dim3 grid((unsigned)((a.n_rows + 3) / 4)), block(256);
  if (grid.x == 0) return hipSuccess;
  hipLaunchKernelGGL(dh_inplace_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace rnnt
