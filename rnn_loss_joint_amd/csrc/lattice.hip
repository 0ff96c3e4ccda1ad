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

hipError_t launch_lattice(const LatticeArgs& a, int U1max, hipStream_t st) {
  dim3 grid(a.B, 2), block(64);
  if (a.B == 0) return hipSuccess;
  if (U1max <= 64) hipLaunchKernelGGL((lattice_kernel<1, 32>), grid, block, 0, st, a);
  else if (U1max <= 128) hipLaunchKernelGGL((lattice_kernel<2, 32>), grid, block, 0, st, a);
  else if (U1max <= 256) hipLaunchKernelGGL((lattice_kernel<4, 16>), grid, block, 0, st, a);
  else if (U1max <= 512) hipLaunchKernelGGL((lattice_kernel<8, 8>), grid, block, 0, st, a);
  else if (U1max <= 1024) hipLaunchKernelGGL((lattice_kernel<16, 4>), grid, block, 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rnnt
