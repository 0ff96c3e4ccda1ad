// Forward and backward variables over each sample's T_b x (U_b+1) lattice
// ("Neural transducer training ...", section "Transducer training", Eq. (8),
// log domain) and the loss (Eq. (9)):
//   alpha(0,0) = 0
//   alpha(t,u) = logaddexp(alpha(t-1,u) + phi(t-1,u), alpha(t,u-1) + psi(t,u-1))
//   beta(T_b-1,U_b) = phi(T_b-1,U_b)
//   beta(t,u)  = logaddexp(phi(t,u) + beta(t+1,u), psi(t,u) + beta(t,u+1))
//   cost_b = -(alpha(T_b-1,U_b) + phi(T_b-1,U_b))
//
// Every cell of anti-diagonal d = t + u depends only on diagonal d - 1
// (alpha) or d + 1 (beta), so the sweep runs over diagonals with one lattice
// row u per lane. The arrays are diagonal-major (lat_ix): diagonal d of a
// sample is one contiguous vector over u, so a wave reads its 64 rows of
// phi / psi and writes its 64 results per diagonal as aligned 256-byte
// vectors.
//
// A workgroup of NW waves serves one (sample, direction); wave w owns rows
// u = 64 w + lane. The waves form a pipeline along u: alpha at row 64 w needs
// row 64 w - 1 of the previous diagonal, which wave w - 1 owns, so wave w
// runs one window of SW diagonals behind wave w - 1 (beta: one window behind
// wave w + 1, whose row 64 (w + 1) it needs). Inside a wave the neighbour
// row comes from the adjacent lane by a DPP shift; across waves, the
// boundary row's values of a window go to an LDS ring of the reading wave,
// indexed by position in the sweep (alpha: d - 1, beta: D - 1 - d, so window
// k holds positions SW k .. SW k + SW - 1); one barrier per window separates
// writer and reader. Step s of the workgroup is window s - w of wave w
// (alpha) or s - (NW - 1 - w) (beta).
//
// Inside the kernel the variables are kept in base 2 (x log2 e), so a
// log-add-exp is max(a, b) + log2(1 + 2^-|a - b|): the scale is applied once
// per operand and once per stored result, not on the sweep's dependency
// chain.
//
// Memory goes through buffer instructions on a resource spanning the
// sample's block of ND x US entries, with the diagonal's offset in the
// scalar offset: a read outside the block returns 0 and a store outside it
// is dropped. A cell outside the lattice gets that out-of-range offset for
// its operand reads and its store, so its bytes are neither read nor
// written, and the per-cell mask keeps its alpha / beta at -inf. A cell in
// the lattice can still have an operand outside it (phi(-1, u) for alpha at
// t = 0, for instance), an arbitrary value of the block (uninitialised
// workspace in the loss path): each operand is made finite or -inf when used
// (NaN and +inf become 1e30) and such an operand only ever meets a -inf
// neighbour. The loads of a window are issued two windows ahead.
#include "common.hpp"
#include "kernels.hpp"

namespace rnnt {

constexpr int SRING = 64;                   // boundary ring entries per wave
constexpr unsigned kOffNone = 0xffffffffu;  // out-of-range buffer offset

// workgroup barrier that orders LDS only: the global loads in flight for the
// next window stay in flight across it
__device__ inline void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// raw buffer resource over `bytes` bytes at p (gfx9 word 3: 32-bit data)
__device__ inline __amdgpu_buffer_rsrc_t sample_rsrc(const float* p, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, (int)bytes, 0x00020000);
}

// one dword through the buffer resource at voff + soff (the builtins move
// raw bits)
__device__ inline float buf_ld(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ inline void buf_st(float v, __amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
}

// operand in base 2, finite or -inf
__device__ inline float operand2(float raw) { return fminf(raw * kLog2e, 1e30f); }

// base-2 log-add-exp; a = b = -inf gives NaN, which only occurs on cells the
// caller masks
__device__ inline float lae2(float a, float b) {
  return __builtin_fmaxf(a, b) + flog2(1.0f + fexp2(-__builtin_fabsf(a - b)));
}

// neighbour rows through DPP wave shifts: lane l receives lane l-1's
// (wave_shr:1) or lane l+1's (wave_shl:1) value, the edge lane `old`
__device__ inline float from_prev_lane(float v, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), 0x138, 0xf, 0xf, false));
}
__device__ inline float from_next_lane(float v, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), 0x130, 0xf, 0xf, false));
}

template <int NW, int SW, bool is_beta>
__device__ __attribute__((always_inline)) inline void lattice_body(const LatticeArgs& p, float* ring) {
  static_assert(SW % 4 == 0 && 2 * SW < SRING, "ring slots of a window must not wrap onto unread ones");
  const int b = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int u = 64 * wave + lane;
  const int Tb = p.T_len[b], Ub = p.U_len[b];
  const int US = lat_us(p.U1), ND = lat_nd(p.T, p.U1);
  const size_t base0 = (size_t)b * ND * US;
  const unsigned blk = (unsigned)(ND * US) * 4u;
  const float* phi = p.phi + base0;
  const auto rphi = sample_rsrc(phi, blk);
  const auto rpsi = sample_rsrc(p.psi + base0, blk);
  const auto rres = sample_rsrc((is_beta ? p.beta : p.alpha) + base0, blk);
  const unsigned dstride = (unsigned)US * 4u;  // bytes per diagonal
  const int D = Tb - 1 + Ub;
  const int nwin = (D + SW - 1) / SW;
  const int nsteps = nwin > 0 ? nwin + NW - 1 : 0;
  const int lag = is_beta ? NW - 1 - wave : wave;
  const bool live = 64 * wave <= Ub;  // a wave past U_b holds only -inf rows
  float* const my_ring = ring + wave * SRING;

  // Operands of window position w. Alpha at diagonal d = 1 + SW k + w reads
  // phi(t-1, u) and psi(t, u-1), both on diagonal d - 1 = SW k + w (psi one
  // row lower: lane offset u - 1; lane 0's read falls outside the block or
  // on an unused entry). Beta at d = D - 1 - SW k - w reads phi(t, u) and
  // psi(t, u) on diagonal d (clamped at 0: those positions are masked).
  const unsigned vo_p = 4u * (unsigned)u;
  const unsigned vo_s = is_beta ? vo_p : vo_p - 4u;
  auto opnd_diag = [&](int k, int w) { return is_beta ? max(D - 1 - SW * k - w, 0) : SW * k + w; };
  // Position w of window k is diagonal d_first + w (alpha) or d_first - w
  // (beta), t = d - u; the cell is in the lattice for w_lo <= w < w_lo + cnt.
  struct Span { int d_first, w_lo; unsigned cnt; };
  auto span = [&](int k) {
    const int d_first = is_beta ? D - 1 - SW * k : 1 + SW * k;
    const int t0 = d_first - u;
    const int w_lo = is_beta ? max(t0 - (Tb - 1), 0) : max(-t0, 0);
    const int w_hi = is_beta ? min(t0, SW - 1) : min(Tb - 1 - t0, SW - 1);
    return Span{d_first, w_lo, u <= Ub ? (unsigned)max(w_hi + 1 - w_lo, 0) : 0u};
  };
  // only a cell in the lattice uses its operands: the others read 0 (an
  // out-of-range offset), which spares their bytes
  auto load = [&](int k, float* rp, float* rs) {
    const Span sp = span(k);
#pragma unroll
    for (int w = 0; w < SW; ++w) {
      const unsigned so = (unsigned)opnd_diag(k, w) * dstride;
      const bool ok = (unsigned)(w - sp.w_lo) < sp.cnt;
      rp[w] = buf_ld(rphi, ok ? vo_p : kOffNone, so);
      rs[w] = buf_ld(rpsi, ok ? vo_s : kOffNone, so);
    }
  };

  for (int i = threadIdx.x; i < NW * SRING; i += 64 * NW) ring[i] = kNegInf;
  float cur;  // base 2
  float lnP2 = kNegInf;
  if (!is_beta) {
    cur = u == 0 ? 0.0f : kNegInf;  // diagonal 0
    if (u == 0) buf_st(0.0f, rres, 0, 0);
  } else {
    const float fin = phi[(size_t)D * US + Ub];  // diagonal D
    cur = u == Ub ? fin * kLog2e : kNegInf;
    if (u == Ub) buf_st(fin, rres, vo_p, (unsigned)D * dstride);
  }
  lds_sync();
  // beta: the boundary value at diagonal D (position -1) for the wave below
  if (is_beta && wave > 0 && lane == 0) ring[(wave - 1) * SRING + SRING - 1] = cur;

  // Step s: issue the loads of window s + 2 - lag into np / ns, then compute
  // window k = s - lag (if this wave has it) from rp / rs, which its loads
  // filled two steps earlier. Register set j holds the windows loaded at
  // steps s with s + 2 = j (mod 3), so the sets rotate with s alone.
  auto step = [&](int s, float* rp, float* rs, float* np, float* ns) {
    const int k = s - lag;
    if (live && k + 2 >= 0 && k + 2 < nwin) load(k + 2, np, ns);
    if (live && k >= 0 && k < nwin) {
      // the neighbour row's value one position earlier
      float vn[SW];
      const int slot = (SW * k) & (SRING - 1);
      vn[0] = my_ring[(slot - 1) & (SRING - 1)];
#pragma unroll
      for (int q = 0; q < SW / 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(my_ring + slot + 4 * q);
        vn[4 * q + 1] = v.x;
        vn[4 * q + 2] = v.y;
        vn[4 * q + 3] = v.z;
        if (4 * q + 4 < SW) vn[4 * q + 4] = v.w;
      }
      const Span sp = span(k);
      const int d_first = sp.d_first, w_lo = sp.w_lo;
      const unsigned cnt = sp.cnt;
      float res_w[SW];
#pragma unroll
      for (int w = 0; w < SW; ++w) {
        const float nb = is_beta ? from_next_lane(cur, vn[w]) : from_prev_lane(cur, vn[w]);
        const float nxt = lae2(cur + operand2(rp[w]), nb + operand2(rs[w]));
        const bool ok = (unsigned)(w - w_lo) < cnt;
        cur = ok ? nxt : kNegInf;
        res_w[w] = cur;
        const int d = is_beta ? d_first - w : d_first + w;
        buf_st(cur * kLn2, rres, ok ? vo_p : kOffNone, (unsigned)max(d, 0) * dstride);
      }
      if (!is_beta && k == nwin - 1) {
        // diagonal D is position D - 1 - SW k of the last window
#pragma unroll
        for (int w = 0; w < SW; ++w)
          if (w == D - 1 - SW * k && u == Ub) lnP2 = res_w[w];
      }
      // the edge lane's values go to the neighbour wave's ring
      const int nbw = is_beta ? wave - 1 : wave + 1;
      if (nbw >= 0 && nbw < NW && lane == (is_beta ? 0 : 63)) {
        float* dst = ring + nbw * SRING + slot;
#pragma unroll
        for (int q = 0; q < SW / 4; ++q)
          *reinterpret_cast<float4*>(dst + 4 * q) =
              make_float4(res_w[4 * q], res_w[4 * q + 1], res_w[4 * q + 2], res_w[4 * q + 3]);
      }
    }
    if (s >= 0) lds_sync();
  };

  // steps -2 and -1 only issue the first two windows' loads
  float r0p[SW], r0s[SW], r1p[SW], r1s[SW], r2p[SW], r2s[SW];
  for (int s = -2; s < nsteps; s += 3) {
    step(s, r1p, r1s, r0p, r0s);
    if (s + 1 < nsteps) step(s + 1, r2p, r2s, r1p, r1s);
    if (s + 2 < nsteps) step(s + 2, r0p, r0s, r2p, r2s);
  }
  if (!is_beta && u == Ub) {
    const float v = (D == 0 ? 0.0f : lnP2 * kLn2) + phi[(size_t)D * US + Ub];
    if (p.lnP) p.lnP[b] = v;
    if (p.costs) p.costs[b] = -v;
  }
}

template <int NW, int SW>
__global__ void __launch_bounds__(64 * NW) lattice_kernel(LatticeArgs p) {
  __shared__ __attribute__((aligned(16))) float ring[NW * SRING];
  if (blockIdx.y == 0) lattice_body<NW, SW, false>(p, ring);
  else lattice_body<NW, SW, true>(p, ring);
}

hipError_t launch_lattice(const LatticeArgs& a, int U1max, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const dim3 grid(a.B, 2);
  const int nw = (U1max + 63) / 64;
  if (nw <= 1) hipLaunchKernelGGL((lattice_kernel<1, 16>), grid, dim3(64), 0, st, a);
  else if (nw <= 2) hipLaunchKernelGGL((lattice_kernel<2, 16>), grid, dim3(128), 0, st, a);
  else if (nw <= 3) hipLaunchKernelGGL((lattice_kernel<3, 16>), grid, dim3(192), 0, st, a);
  else if (nw <= 4) hipLaunchKernelGGL((lattice_kernel<4, 16>), grid, dim3(256), 0, st, a);
  else if (nw <= 6) hipLaunchKernelGGL((lattice_kernel<6, 16>), grid, dim3(384), 0, st, a);
  else if (nw <= 8) hipLaunchKernelGGL((lattice_kernel<8, 16>), grid, dim3(512), 0, st, a);
  else if (nw <= 12) hipLaunchKernelGGL((lattice_kernel<12, 8>), grid, dim3(768), 0, st, a);
  else if (nw <= 16) hipLaunchKernelGGL((lattice_kernel<16, 8>), grid, dim3(1024), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rnnt
