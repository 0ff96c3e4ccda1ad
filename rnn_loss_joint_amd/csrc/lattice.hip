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
// Multi-wave variant for U_b + 1 <= 64 NW: wave w of the workgroup owns rows
// u = 64 w + lane, one per lane. The cells of diagonal d sit at t = d - u in
// the u-major arrays, so a diagonal is a strided gather; over a window of SW
// diagonals, though, each row needs SW consecutive t of phi and psi. A wave
// loads them coalesced (16 lanes per row, 64 bytes), transposes them through
// LDS (element e of row slot r at e * SSTR + r: the loader's and the row
// owners' accesses both hit distinct banks) and writes its window of alpha /
// beta back the same way. The next window's loads are in flight while a
// window computes.
//
// The waves form a pipeline along u: alpha at row 64 w needs row 64 w - 1 of
// the previous diagonal, which wave w - 1 owns, so wave w runs one window
// behind wave w - 1 (beta: wave w runs one window behind wave w + 1, whose
// row 64 (w + 1) it needs). The boundary row's values of a window go to an
// LDS ring of the reading wave, indexed by position in the sweep (alpha:
// d - 1, beta: D - 1 - d, so window k holds positions SW k .. SW k + SW - 1);
// one barrier per window separates writer and reader. Step s of the
// workgroup is window s - w of wave w (alpha) or s - (NW - 1 - w) (beta).
//
// Window k covers alpha diagonals d0 .. d0 + SW - 1 (d0 = 1 + SW k) or beta
// diagonals d_hi .. d_hi - SW + 1 (d_hi = D - 1 - SW k). Row slot r, element
// e of a window holds X[row][base - row + e] with base = d0 - 1 (alpha) or
// d_hi - SW + 1 (beta); the psi slot of row u holds row u - 1 for alpha (the
// label transition into u) and row u for beta. Out-of-lattice entries are
// -inf.
constexpr int SW = 16;       // diagonals per window
constexpr int SSTR = 68;     // LDS stride of one element column (floats)
constexpr int SRING = 64;    // boundary ring entries per wave (> 2 SW)
constexpr int SWAVE_LDS = 3 * SW * SSTR;  // phi, psi, output tile

// workgroup barrier that orders LDS only: the global loads in flight for the
// next window stay in flight across it
__device__ inline void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int NW, bool is_beta>
__device__ __attribute__((always_inline)) inline void lattice_sys_body(const LatticeArgs& p, float* lds) {
  const int b = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int u = 64 * wave + lane;
  const int Tb = p.T_len[b], Ub = p.U_len[b];
  const int T = p.T;
  const size_t base0 = (size_t)b * p.U1 * T;
  const float* phi = p.phi + base0;
  const float* psi = p.psi + base0;
  float* res = (is_beta ? p.beta : p.alpha) + base0;
  const int D = Tb - 1 + Ub;
  const int nwin = (D + SW - 1) / SW;
  const int nsteps = nwin > 0 ? nwin + NW - 1 : 0;
  const int lag = is_beta ? NW - 1 - wave : wave;
  const int psi_shift = is_beta ? 0 : 1;
  const bool live = 64 * wave <= Ub;  // a wave past U_b holds only -inf rows

  float* const sphi_l = lds + wave * SWAVE_LDS;  // [e][slot]
  float* const spsi_l = sphi_l + SW * SSTR;
  float* const out = spsi_l + SW * SSTR;
  float* const ring = lds + NW * SWAVE_LDS;       // [wave][SRING]: value the wave reads
  float* const my_ring = ring + wave * SRING;

  // loader lanes: slot r = 4 j + lr (j = 0 .. 15), element le. Element e of
  // row r sits at r T + base - r + e = r (T - 1) + base + e; every index is
  // clamped into the sample's [U1][T] block, so entries outside the lattice
  // read arbitrary values of the sample. They are made finite at staging
  // (fminf maps NaN and +inf to FLT_MAX) and never reach a lattice cell: the
  // cell mask below keeps every out-of-lattice alpha / beta at -inf, and a
  // valid cell's phi / psi operands are in the lattice or are added to such a
  // -inf neighbour.
  const int lr = lane >> 4, le = lane & 15;
  const int lane_ix = lr * (T - 1) + le;
  const int last_ix = p.U1 * T - 1;
  float rphi[16], rpsi[16];
  auto window_base = [&](int k) { return is_beta ? D - 1 - SW * k - (SW - 1) : SW * k; };
  auto load = [&](int k) {
    const int row0 = (64 * wave) * (T - 1) + window_base(k) + lane_ix;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int ip = row0 + 4 * j * (T - 1), is = ip - psi_shift * (T - 1);
      rphi[j] = phi[(unsigned)min(max(ip, 0), last_ix)];
      rpsi[j] = psi[(unsigned)min(max(is, 0), last_ix)];
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      sphi_l[le * SSTR + 4 * j + lr] = fminf(rphi[j], __FLT_MAX__);
      spsi_l[le * SSTR + 4 * j + lr] = fminf(rpsi[j], __FLT_MAX__);
    }
  };
  // results of window k: slot r, element e -> res[row][base - row + e + shift]
  auto flush = [&](int k) {
    const int base = window_base(k) + (is_beta ? 0 : 1);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 64 * wave + 4 * j + lr, t = base - r + le;
      const float v = out[le * SSTR + 4 * j + lr];
      if ((r <= Ub) & ((unsigned)t < (unsigned)Tb)) res[(unsigned)(r * T + t)] = v;
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

  for (int i = threadIdx.x; i < NW * SRING; i += 64 * NW) ring[i] = kNegInf;
  float cur;
  float lnP = kNegInf;
  if (!is_beta) {
    cur = u == 0 ? 0.0f : kNegInf;  // diagonal 0
    if (u == 0) res[0] = 0.0f;
  } else {
    const float fin = phi[(unsigned)(Ub * T + Tb - 1)];  // diagonal D
    cur = u == Ub ? fin : kNegInf;
    if (u == Ub) res[(unsigned)(Ub * T + Tb - 1)] = fin;
  }
  if (live && nwin > 0) {
    load(0);
    stage();
    if (nwin > 1) load(1);
  }
  lds_sync();
  // beta: the boundary value at diagonal D (position -1) for the wave below
  if (is_beta && wave > 0 && lane == 0) ring[(wave - 1) * SRING + SRING - 1] = cur;

  for (int s = 0; s < nsteps; ++s) {
    const int k = s - lag;
    if (live && k >= 0 && k < nwin) {
      // window operands into registers first: element e = w (alpha) or
      // SW - 1 - w (beta); the neighbour row's value one position earlier
      float vp[SW], vs[SW], vn[SW];
#pragma unroll
      for (int w = 0; w < SW; ++w) {
        const int e = is_beta ? SW - 1 - w : w;
        vp[w] = sphi_l[e * SSTR + lane];
        vs[w] = spsi_l[e * SSTR + lane];
      }
      const int slot = (SW * k) & (SRING - 1);
      vn[0] = my_ring[(slot - 1) & (SRING - 1)];
#pragma unroll
      for (int q = 0; q < SW / 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(my_ring + slot + 4 * q);
        if (4 * q + 1 < SW) vn[4 * q + 1] = v.x;
        if (4 * q + 2 < SW) vn[4 * q + 2] = v.y;
        if (4 * q + 3 < SW) vn[4 * q + 3] = v.z;
        if (4 * q + 4 < SW) vn[4 * q + 4] = v.w;
      }
      // position w of the window is diagonal d0 + w (alpha) or d_hi - w
      // (beta); the cell's t = d - u runs up (alpha) or down (beta) with w
      const int t0 = is_beta ? D - 1 - SW * k - u : 1 + SW * k - u;
      const bool row_ok = u <= Ub;
      float res_w[SW];
#pragma unroll
      for (int w = 0; w < SW; ++w) {
        const float nb = is_beta ? from_next_lane(cur, vn[w]) : from_prev_lane(cur, vn[w]);
        const float nxt = log_add_exp(cur + vp[w], nb + vs[w]);
        const int t = is_beta ? t0 - w : t0 + w;
        cur = (row_ok & ((unsigned)t < (unsigned)Tb)) ? nxt : kNegInf;
        res_w[w] = cur;
      }
      if (!is_beta && k == nwin - 1) {
        // diagonal D is position D - 1 - SW k of the last window
#pragma unroll
        for (int w = 0; w < SW; ++w)
          if (w == D - 1 - SW * k && u == Ub) lnP = res_w[w];
      }
#pragma unroll
      for (int w = 0; w < SW; ++w) out[(is_beta ? SW - 1 - w : w) * SSTR + lane] = res_w[w];
      // the edge lane's values go to the neighbour wave's ring
      const int nbw = is_beta ? wave - 1 : wave + 1;
      if (nbw >= 0 && nbw < NW && lane == (is_beta ? 0 : 63)) {
        float* dst = ring + nbw * SRING + slot;
#pragma unroll
        for (int q = 0; q < SW / 4; ++q)
          *reinterpret_cast<float4*>(dst + 4 * q) =
              make_float4(res_w[4 * q], res_w[4 * q + 1], res_w[4 * q + 2], res_w[4 * q + 3]);
      }
      // stage the next window (its loads were in flight), start the one
      // after, then write this window's results
      if (k + 1 < nwin) {
        stage();
        if (k + 2 < nwin) load(k + 2);
      }
      flush(k);
    }
    lds_sync();
  }
  if (!is_beta && u == Ub) {
    if (D == 0) lnP = cur;
    const float v = lnP + phi[(unsigned)(Ub * T + Tb - 1)];
    if (p.lnP) p.lnP[b] = v;
    if (p.costs) p.costs[b] = -v;
  }
}

template <int NW>
__global__ void __launch_bounds__(64 * NW) lattice_sys_kernel(LatticeArgs p) {
  __shared__ __attribute__((aligned(16))) float lds[NW * SWAVE_LDS + NW * SRING];
  if (blockIdx.y == 0) lattice_sys_body<NW, false>(p, lds);
  else lattice_sys_body<NW, true>(p, lds);
}

hipError_t launch_lattice(const LatticeArgs& a, int U1max, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const dim3 grid(a.B, 2);
  if (U1max <= 64) hipLaunchKernelGGL((lattice_sys_kernel<1>), grid, dim3(64), 0, st, a);
  else if (U1max <= 128) hipLaunchKernelGGL((lattice_sys_kernel<2>), grid, dim3(128), 0, st, a);
  else if (U1max <= 192) hipLaunchKernelGGL((lattice_sys_kernel<3>), grid, dim3(192), 0, st, a);
  else if (U1max <= 256) hipLaunchKernelGGL((lattice_sys_kernel<4>), grid, dim3(256), 0, st, a);
  else if (U1max <= 512) hipLaunchKernelGGL((lattice_sys_kernel<8>), grid, dim3(512), 0, st, a);
  else if (U1max <= 1024) hipLaunchKernelGGL((lattice_kernel<16, 4>), grid, dim3(64), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rnnt
