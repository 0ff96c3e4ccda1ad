// Forward and backward variables over each sample's T_b x (U_b+1) lattice
// ("Neural transducer training ...", section "Transducer training", Eq. (8),
// log domain) and the loss (Eq. (9)):
//   alpha(0,0) = 0
//   alpha(t,u) = logaddexp(alpha(t-1,u) + phi(t-1,u), alpha(t,u-1) + psi(t,u-1))
//   beta(T_b-1,U_b) = phi(T_b-1,U_b)
//   beta(t,u)  = logaddexp(phi(t,u) + beta(t+1,u), psi(t,u) + beta(t,u+1))
//   cost_b = -(alpha(T_b-1,U_b) + phi(T_b-1,U_b))
//
// One wavefront per (sample, direction); the alpha and beta waves of a sample
// run concurrently. Lane l owns UPL consecutive u's and the wave sweeps the
// anti-diagonals d = t + u: every cell of diagonal d depends only on diagonal
// d-1 (alpha) or d+1 (beta), so a step is UPL log-add-exps per lane plus one
// lane shift for the neighbour at the lane's u boundary. phi/psi are stored
// u-major ([b][u][t], t fastest), so each lane streams along t; the loads for
// step d+PF are issued at step d into a register ring.
#include "common.hpp"
#include "kernels.hpp"

namespace rnnt {

template <int UPL, int PF>
__global__ void __launch_bounds__(64) lattice_kernel(LatticeArgs p) {
  const int b = blockIdx.x;
  const bool is_beta = blockIdx.y == 1;
  const int lane = threadIdx.x;
  const int Tb = p.T_len[b];
  const int Ub = p.U_len[b];
  const int U1 = Ub + 1;
  const int T = p.T;
  const size_t base = (size_t)b * p.U1 * T;
  const float* phi = p.phi + base;
  const float* psi = p.psi + base;
  const int u0 = lane * UPL;
  const int D = Tb - 1 + Ub;  // last diagonal

  float cur[UPL];
  float rphi[PF][UPL], rpsi[PF][UPL];

  if (!is_beta) {
    float* alpha = p.alpha + base;
    // step d needs phi(t-1,u) = phi[u][d-1-u] and psi(t,u-1) = psi[u-1][d-u], t = d-u
    auto load = [&](int d, float* fp, float* fs) {
#pragma unroll
      for (int i = 0; i < UPL; ++i) {
        int u = u0 + i, t = d - u;
        fp[i] = (u < U1 && t >= 1 && t < Tb) ? phi[(size_t)u * T + t - 1] : kNegInf;
        fs[i] = (u >= 1 && u < U1 && t >= 0 && t < Tb) ? psi[(size_t)(u - 1) * T + t] : kNegInf;
      }
    };
#pragma unroll
    for (int i = 0; i < UPL; ++i) cur[i] = (u0 + i == 0) ? 0.0f : kNegInf;
    if (lane == 0) alpha[0] = 0.0f;
#pragma unroll
    for (int k = 0; k < PF; ++k) load(1 + k, rphi[k], rpsi[k]);
    for (int d0 = 1; d0 <= D; d0 += PF) {
#pragma unroll
      for (int k = 0; k < PF; ++k) {
        const int d = d0 + k;
        if (d <= D) {
        float left = __shfl_up(cur[UPL - 1], 1);
        if (lane == 0) left = kNegInf;
        float nxt[UPL];
#pragma unroll
        for (int i = 0; i < UPL; ++i) {
          float from_t = cur[i] + rphi[k][i];
          float from_u = (i == 0 ? left : cur[i - 1]) + rpsi[k][i];
          nxt[i] = log_add_exp(from_t, from_u);
        }
#pragma unroll
        for (int i = 0; i < UPL; ++i) {
          int u = u0 + i, t = d - u;
          bool ok = u < U1 && t >= 0 && t < Tb;
          cur[i] = ok ? nxt[i] : kNegInf;
          if (ok) alpha[(size_t)u * T + t] = cur[i];
        }
        load(d + PF, rphi[k], rpsi[k]);
        }
      }
    }
    // lnP = alpha(T_b-1, U_b) + phi(T_b-1, U_b), held by the lane owning U_b
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
      if (u0 + i == Ub) {
        float lnP = cur[i] + phi[(size_t)Ub * T + Tb - 1];
        if (p.lnP) p.lnP[b] = lnP;
        if (p.costs) p.costs[b] = -lnP;
      }
    }
  } else {
    float* beta = p.beta + base;
    // step d needs phi(t,u) and psi(t,u) at t = d-u
    auto load = [&](int d, float* fp, float* fs) {
#pragma unroll
      for (int i = 0; i < UPL; ++i) {
        int u = u0 + i, t = d - u;
        bool ok = u < U1 && t >= 0 && t < Tb;
        fp[i] = (ok && t + 1 < Tb) ? phi[(size_t)u * T + t] : kNegInf;
        fs[i] = (ok && u < Ub) ? psi[(size_t)u * T + t] : kNegInf;
      }
    };
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
      int u = u0 + i;
      cur[i] = (u == Ub) ? phi[(size_t)Ub * T + Tb - 1] : kNegInf;
      if (u == Ub) beta[(size_t)Ub * T + Tb - 1] = cur[i];
    }
#pragma unroll
    for (int k = 0; k < PF; ++k) load(D - 1 - k, rphi[k], rpsi[k]);
    for (int d0 = D - 1; d0 >= 0; d0 -= PF) {
#pragma unroll
      for (int k = 0; k < PF; ++k) {
        const int d = d0 - k;
        if (d >= 0) {
        float right = __shfl_down(cur[0], 1);
        if (lane == 63) right = kNegInf;
        float nxt[UPL];
#pragma unroll
        for (int i = 0; i < UPL; ++i) {
          float by_blank = cur[i] + rphi[k][i];
          float by_label = (i == UPL - 1 ? right : cur[i + 1]) + rpsi[k][i];
          nxt[i] = log_add_exp(by_blank, by_label);
        }
#pragma unroll
        for (int i = 0; i < UPL; ++i) {
          int u = u0 + i, t = d - u;
          bool ok = u < U1 && t >= 0 && t < Tb;
          cur[i] = ok ? nxt[i] : kNegInf;
          if (ok) beta[(size_t)u * T + t] = cur[i];
        }
        load(d - PF, rphi[k], rpsi[k]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Windowed variant for U_b + 1 <= 256 (lanes own rows u = lane + 64 i).
// The cells of diagonal d sit at t = d - u in the u-major arrays, so a
// diagonal is a strided gather; per window of 8 diagonals, though, each row
// u needs 8 consecutive t of phi and psi. Those are loaded coalesced (8 lanes
// per row, 32 bytes), staged column-major in LDS (element e of row u at
// e*264 + u floats: both the loader's and the row owners' accesses hit
// distinct banks), and the window's alpha / beta go to an LDS tile flushed
// the same way. The next window's loads are in flight while one computes.
// Row u, element e of a window holds X[u][s_u + e], s_u = base - u, with
// base = d0 - 1 (alpha, diagonals d0 .. d0+7) or d_hi - 7 (beta, diagonals
// d_hi .. d_hi-7); the masks make every out-of-lattice entry -inf.
constexpr int LW = 8;          // diagonals per window
constexpr int LSTR = 264;      // LDS stride of one element column (floats)
constexpr int LROWS = 256;

template <int NI>
__global__ void __launch_bounds__(64) lattice_win_kernel(LatticeArgs p) {
  __shared__ float lds[(4 * LW + LW) * LSTR];  // phi/psi x 2 buffers, output tile
  float* const stg = lds;                       // [buf][arr][e][u]: ((buf*2+arr)*LW + e)*LSTR + u
  float* const out = lds + 4 * LW * LSTR;       // [e][u]
  const int b = blockIdx.x;
  const bool is_beta = blockIdx.y == 1;
  const int lane = threadIdx.x;
  const int Tb = p.T_len[b], Ub = p.U_len[b];
  const int T = p.T;
  const size_t base0 = (size_t)b * p.U1 * T;
  const float* phi = p.phi + base0;
  const float* psi = p.psi + base0;
  float* res = (is_beta ? p.beta : p.alpha) + base0;
  const int D = Tb - 1 + Ub;
  constexpr int NJ = NI * 8;  // load instructions per array per window (8 rows each)
  const int lr = lane >> 3, le = lane & 7;  // loader: row within an 8-row group, element

  // raw values of window `base` for this lane's loader slots. The loads are
  // unconditional (masked entries read element 0 of the sample) and their
  // results are not touched until stage() one window later, so the whole
  // batch is in flight together; stage() applies the masks (-inf).
  float sphi[NJ], spsi[NJ];
  auto okp = [&](int u, int t) { return u <= Ub && t >= 0 && t <= Tb - 2; };
  auto oks = [&](int u, int t) { return u < Ub && t >= 0 && t <= Tb - 1; };
  auto load = [&](int base) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int u = 8 * j + lr, t = base - u + le;
      const int ix = u * T + t;
      sphi[j] = phi[okp(u, t) ? ix : 0];
      spsi[j] = psi[oks(u, t) ? ix : 0];
    }
  };
  auto stage = [&](int buf, int base) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int u = 8 * j + lr, t = base - u + le;
      stg[((buf * 2 + 0) * LW + le) * LSTR + u] = okp(u, t) ? sphi[j] : kNegInf;
      stg[((buf * 2 + 1) * LW + le) * LSTR + u] = oks(u, t) ? spsi[j] : kNegInf;
    }
  };
  // write the window's results: row u, element e -> res[u][s_u + e + shift]
  auto flush = [&](int base, int shift) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int u = 8 * j + lr, t = base - u + le + shift;
      const float v = out[le * LSTR + 8 * j + lr];
      if (u <= Ub && t >= 0 && t < Tb) res[u * T + t] = v;
    }
  };
  // neighbour rows through DPP wave shifts: lane l receives lane l-1's
  // (wave_shr:1) or lane l+1's (wave_shl:1) value, the edge lane `old`
  auto from_prev_lane = [](float v, float old) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), 0x138, 0xf, 0xf, false));
  };
  auto from_next_lane = [](float v, float old) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), 0x130, 0xf, 0xf, false));
  };
  // one lane's value, moved as bits (the readlane builtin takes an int)
  auto lane_value = [](float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };

  float cur[NI];
  if (!is_beta) {
    // diagonal 0: alpha(0, 0) = 0
#pragma unroll
    for (int i = 0; i < NI; ++i) cur[i] = (lane + 64 * i == 0) ? 0.0f : kNegInf;
    if (lane == 0) res[0] = 0.0f;
    float lnP = kNegInf;
    int k = 0;
    load(0);  // window d0 = 1: base = d0 - 1 = 0
    stage(0, 0);
    if (1 + LW <= D) load(LW);
    for (int d0 = 1; d0 <= D; d0 += LW, ++k) {
      const float* sp = stg + ((k & 1) * 2 + 0) * LW * LSTR;
      const float* ss = stg + ((k & 1) * 2 + 1) * LW * LSTR;
#pragma unroll
      for (int w = 0; w < LW; ++w) {
        const int d = d0 + w;
        float nxt[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int u = lane + 64 * i;
          const float wrap = i > 0 ? lane_value(cur[i > 0 ? i - 1 : 0], 63) : kNegInf;
          const float left = from_prev_lane(cur[i], wrap);
          const float from_t = cur[i] + sp[w * LSTR + u];
          const float from_u = left + (u > 0 ? ss[w * LSTR + u - 1] : kNegInf);
          nxt[i] = log_add_exp(from_t, from_u);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int u = lane + 64 * i, t = d - u;
          const bool ok = u <= Ub && t >= 0 && t < Tb;
          cur[i] = ok ? nxt[i] : kNegInf;
          out[w * LSTR + u] = cur[i];
          if (d == D && u == Ub) lnP = cur[i];
        }
      }
      // stage the next window (its loads were in flight), then write this one
      if (d0 + LW <= D) {
        stage((k + 1) & 1, d0 + LW - 1);
        if (d0 + 2 * LW <= D) load(d0 + 2 * LW - 1);
      }
      flush(d0 - 1, 1);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (lane + 64 * i == Ub) {
        if (D == 0) lnP = cur[i];
        const float v = lnP + phi[(size_t)Ub * T + Tb - 1];
        if (p.lnP) p.lnP[b] = v;
        if (p.costs) p.costs[b] = -v;
      }
    }
  } else {
    // diagonal D: beta(T_b-1, U_b) = phi(T_b-1, U_b)
    const float fin = phi[(size_t)Ub * T + Tb - 1];
#pragma unroll
    for (int i = 0; i < NI; ++i) cur[i] = (lane + 64 * i == Ub) ? fin : kNegInf;
    if (lane == 0) res[(size_t)Ub * T + Tb - 1] = fin;
    int k = 0;
    if (D - 1 >= 0) load(D - 1 - (LW - 1));
    if (D - 1 >= 0) stage(0, D - 1 - (LW - 1));
    if (D - 1 - LW >= 0) load(D - 1 - LW - (LW - 1));
    for (int dh = D - 1; dh >= 0; dh -= LW, ++k) {
      const float* sp = stg + ((k & 1) * 2 + 0) * LW * LSTR;
      const float* ss = stg + ((k & 1) * 2 + 1) * LW * LSTR;
#pragma unroll
      for (int w = 0; w < LW; ++w) {
        const int d = dh - w, e = LW - 1 - w;
        float nxt[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int u = lane + 64 * i;
          const float wrap = i + 1 < NI ? lane_value(cur[i + 1 < NI ? i + 1 : i], 0) : kNegInf;
          const float right = from_next_lane(cur[i], wrap);
          const float by_blank = cur[i] + sp[e * LSTR + u];
          const float by_label = right + ss[e * LSTR + u];
          nxt[i] = log_add_exp(by_blank, by_label);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int u = lane + 64 * i, t = d - u;
          const bool ok = u <= Ub && t >= 0 && t < Tb;
          cur[i] = ok ? nxt[i] : kNegInf;
          out[e * LSTR + u] = cur[i];
        }
      }
      if (dh - LW >= 0) {
        stage((k + 1) & 1, dh - LW - (LW - 1));
        if (dh - 2 * LW >= 0) load(dh - 2 * LW - (LW - 1));
      }
      flush(dh - (LW - 1), 0);
    }
  }
}

hipError_t launch_lattice(const LatticeArgs& a, int U1max, hipStream_t st) {
  dim3 grid(a.B, 2), block(64);
  if (a.B == 0) return hipSuccess;
  if (U1max <= 64) hipLaunchKernelGGL((lattice_win_kernel<1>), grid, block, 0, st, a);
  else if (U1max <= 128) hipLaunchKernelGGL((lattice_win_kernel<2>), grid, block, 0, st, a);
  else if (U1max <= 192) hipLaunchKernelGGL((lattice_win_kernel<3>), grid, block, 0, st, a);
  else if (U1max <= 256) hipLaunchKernelGGL((lattice_win_kernel<4>), grid, block, 0, st, a);
  else if (U1max <= 512) hipLaunchKernelGGL((lattice_kernel<8, 8>), grid, block, 0, st, a);
  else if (U1max <= 1024) hipLaunchKernelGGL((lattice_kernel<16, 4>), grid, block, 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rnnt
