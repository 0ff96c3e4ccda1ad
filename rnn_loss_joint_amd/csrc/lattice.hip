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
// row u per lane. The arrays hold four consecutive diagonals of a row as one
// aligned 16-byte piece (lat_at: the packed layout of `saved`, or the padded
// layout lat_ix of the rnnt_lattice entry point), so a lane reads its operands
// and writes its results for four diagonals with one 16-byte buffer access,
// and a wave's 64 pieces are one contiguous kilobyte.
//
// NW waves serve one (sample, direction); wave w of them owns rows
// u = 64 w + lane. A workgroup holds one such sweep, or two (the alpha sweep
// of one sample and the beta sweep of another: lattice_pair_kernel). The
// sweep is cut into windows whose loads and stores are the groups of SW
// diagonals from a multiple of SW (alpha computes diagonals
// SW k + 1 .. SW k + SW in window k, upwards from the values on diagonal 0;
// beta computes SW j + SW - 1 down to SW j, downwards from the window holding
// D = T_b - 1 + U_b). The waves form a pipeline along u: alpha
// at row 64 w needs row 64 w - 1 of the previous diagonal, which wave w - 1
// owns, so wave w runs one window behind wave w - 1 (beta: one window behind
// wave w + 1, whose row 64 (w + 1) it needs). Inside a wave the neighbour
// row comes from the adjacent lane by a DPP shift; across waves, the edge
// row's values go to an LDS ring of the reading wave (slot d - 1 mod 128 for
// alpha's diagonal d, slot d mod 128 for beta's), aligned so that a window's
// values are four 16-byte entries; one barrier per window separates writer
// and reader. Step s of the workgroup is window s - w of wave w (alpha) or
// s - (NW - 1 - w) (beta). Alpha's window k stores diagonals SW k ..
// SW k + SW - 1, the first of which the previous window computed.
//
// Beta starts from a virtual cell, value 0 at (T_b, U_b), which it carries
// unchanged through the diagonals above D. Inside the kernel the variables are kept in
// base 2 (x log2 e), so a log-add-exp is max(a, b) + log2(1 + 2^-|a - b|):
// the scale is applied once per operand and once per stored result, not on
// the sweep's dependency chain.
//
// Memory goes through buffer instructions on a resource spanning the
// sample's block, with the group's offset in the scalar offset: a read
// outside the block returns 0 and a store outside it is dropped. A lane
// whose row has no cell among a group's diagonals uses an out-of-range
// offset, so those bytes are neither read nor written; a group that holds
// both cells and non-cells of a row is stored entry by entry, so that only
// lattice cells are written. Operand values of non-cells inside a loaded
// group, and operands outside the lattice that a cell at the lattice's edge
// reads (phi(-1, u) for alpha at t = 0, for instance), may be anything, NaN
// included: each operand is made finite or -inf when used (NaN and +inf
// become 1e30) and such an operand only ever meets a -inf neighbour. Every
// step issues the same number of loads and stores, so the compiler's wait
// counts do not fall back to the shortest path; the loads of a window are
// issued PF windows ahead.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace rnnt {

constexpr int SRING = 128;                  // boundary ring entries per wave (diagonal mod 128)
constexpr unsigned kOffNone = 0xffffffffu;  // out-of-range buffer offset

// workgroup barrier that orders LDS only: the global loads in flight for the
// next windows stay in flight across it
__device__ inline void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// raw buffer resource over `bytes` bytes at p (gfx9 word 3: 32-bit data)
__device__ inline __amdgpu_buffer_rsrc_t sample_rsrc(const float* p, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, (int)bytes, 0x00020000);
}

// The raw buffer builtins move integer bits: floats go through bit casts.
typedef unsigned lat_u32x4 __attribute__((ext_vector_type(4)));
__device__ inline void buf_ld4(float* dst, __amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  const lat_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  dst[0] = __uint_as_float(v.x);
  dst[1] = __uint_as_float(v.y);
  dst[2] = __uint_as_float(v.z);
  dst[3] = __uint_as_float(v.w);
}
__device__ inline void buf_st4(const float* v, __amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  const lat_u32x4 w = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, voff, soff, 0);
}
__device__ inline void buf_st(float v, __amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
}

// x + raw log2 e, with a NaN sum made -inf: an operand outside the lattice
// (any value, NaN and infinities included) only ever meets x = -inf, and
// -inf + (NaN, +inf) is NaN; the maximum with -inf returns the other operand
// unless that is NaN (the sum of an fma is a quiet NaN, so no canonicalizing
// is needed). Only one operand of each direction can lie outside the
// lattice at a cell: alpha's phi(t-1, u) at t = 0, and beta's psi(t, U_b)
// (not a label emission, so the caller's value there is arbitrary); the
// other operand of a cell is always a lattice entry (finite or -inf), and
// where it is not, the cell is not one and its result is discarded.
__device__ inline float add_operand2(float x, float raw) {
  return __builtin_fmaxf(__builtin_fmaf(raw, kLog2e, x), kNegInf);
}
__device__ inline float add_operand(float x, float raw) { return __builtin_fmaf(raw, kLog2e, x); }

// base-2 log-add-exp. With CLAMP the exponent is clamped at -126 so that
// a = b = -inf gives -inf instead of NaN (cells outside a pruned lattice's
// band, or log-probs a caller passes); below -126 the correction
// log2(1 + 2^d) is 0 in fp32 either way. Without it (the loss's own
// log-probs, all finite) every cell has a finite term.
template <bool CLAMP>
__device__ inline float lae2(float a, float b) {
  const float d = -__builtin_fabsf(a - b);
  return __builtin_fmaxf(a, b) + flog2(1.0f + fexp2(CLAMP ? __builtin_fmaxf(d, -126.0f) : d));
}

// neighbour rows through DPP wave shifts: lane l receives lane l-1's
// (wave_shr:1) or lane l+1's (wave_shl:1) value, the edge lane `old`
__device__ inline float from_prev_lane(float v, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), 0x138, 0xf, 0xf, false));
}
__device__ inline float from_next_lane(float v, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), 0x130, 0xf, 0xf, false));
}

// Windows of a sweep of D + 1 diagonals (D = T_b - 1 + U_b).
template <int SW>
__device__ inline int lat_windows(int Tb, int Ub) { return (Tb - 1 + Ub) / SW + 1; }

// One (sample, direction) sweep by NW waves: tid is the thread's index among
// them, ring their NW * SRING entries of LDS. Every wave of the workgroup
// passes the same nsteps (at least the sweep's own K + NW - 1) and so takes
// part in the same number of barriers, whatever its sample's length.
template <int NW, int SW, int PF, bool is_beta, bool CLAMP>
__device__ __attribute__((always_inline)) inline void lattice_body(const LatticeArgs& p, float* ring, int b, int tid,
                                                                  int nsteps) {
  static_assert(SW % 4 == 0 && 3 * SW <= SRING, "a window's ring slots must not wrap onto unread ones");
  constexpr int NG = SW / 4;  // groups of four diagonals per window
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int u = 64 * wave + lane;
  const int Tb = p.T_len[b], Ub = p.U_len[b];
  // the sample's block: packed (inside saved) or padded (the rnnt_lattice layout)
  const LatGeo geo = p.lat_off ? lat_geo_packed(p.lat_off[b], Ub) : lat_geo_padded(b, p.T, p.U1);
  const int US = geo.us;
  const size_t base0 = (size_t)geo.base;
  const unsigned blk = (unsigned)(p.lat_off ? lat_block(Tb, Ub) : lat_sample(p.T, p.U1)) * 4u;
  const float* phi = p.phi + base0;
  const auto rphi = sample_rsrc(phi, blk);
  const auto rpsi = sample_rsrc(p.psi + base0, blk);
  const auto rres = sample_rsrc((is_beta ? p.beta : p.alpha) + base0, blk);
  const unsigned gstride = (unsigned)US * 16u;  // bytes per group of four diagonals
  const int D = Tb - 1 + Ub;
  const int K = lat_windows<SW>(Tb, Ub);
  const int lag = is_beta ? NW - 1 - wave : wave;
  float* const my_ring = ring + wave * SRING;

  for (int i = tid; i < NW * SRING; i += 64 * NW) ring[i] = kNegInf;
  // alpha: the values on diagonal 0; beta: the virtual start 0 at (T_b, U_b)
  float cur = u == (is_beta ? Ub : 0) ? 0.0f : kNegInf;  // base 2
  lds_sync();
  // beta: the start value of row 64 w at diagonal D + 1, for the wave below
  if (is_beta && wave > 0 && lane == 0) ring[(wave - 1) * SRING + ((D + 1) & (SRING - 1))] = cur;

  if (64 * wave > Ub) {
    // a wave past U_b holds only -inf rows: it takes part in the barriers
    for (int s = -PF; s < nsteps; s += PF + 1)
      for (int i = 0; i <= PF; ++i)
        if (s + i >= 0) lds_sync();
    return;
  }

  // Window k covers diagonals wlo(k) .. wlo(k) + SW - 1; the sweep visits
  // them upwards (alpha) or downwards (beta). Group g of the window holds
  // diagonals wlo + 4 g .. wlo + 4 g + 3.
  auto wlo = [&](int k) { return SW * (is_beta ? K - 1 - k : k); };
  const unsigned vo = 16u * (unsigned)u;
  // alpha's psi operand is psi(t, u - 1): row u - 1's piece (none for u = 0)
  const unsigned vo_s = is_beta ? vo : (u == 0 ? kOffNone : vo - 16u);

  // Operands of window k, groups of diagonals wlo .. wlo + SW - 1. Alpha at
  // diagonal d reads phi(t-1, u), psi(t, u-1) on diagonal d - 1, so alpha's
  // window k computes diagonals wlo + 1 .. wlo + SW; beta at d reads
  // phi(t, u), psi(t, u) on diagonal d and computes wlo + SW - 1 .. wlo. A
  // group is read only if it serves a cell of this row (the row's cells lie
  // on diagonals u .. u + Tb - 1).
  auto load = [&](int k, float* rp, float* rs) {
    const bool in = k >= 0 && k < K;
    const int w0 = max(wlo(k), 0);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int lo = w0 + 4 * g + (is_beta ? 0 : 1);  // first diagonal served
      const bool need = in && u <= Ub && lo + 3 >= u && lo <= u + Tb - 1;
      const unsigned off = 0u - (unsigned)!need;  // all-ones: no bytes read
      const unsigned so = (unsigned)((w0 >> 2) + g) * gstride;
      buf_ld4(rp + 4 * g, rphi, vo | off, so);
      buf_ld4(rs + 4 * g, rpsi, vo_s | off, so);
    }
  };

  // alpha: the result on diagonal wlo(k), computed by the previous window
  // (at first the values on diagonal 0) and stored with window k's groups
  float prev = cur;

  // Step s: issue the loads of window s + PF - lag into np / ns, compute
  // window k = s - lag (if this wave has it) from rp / rs, which its loads
  // filled PF steps earlier, then store it. Register set j holds the windows
  // loaded at steps s with s + PF = j (mod PF + 1), so the sets rotate with s
  // alone.
  auto step = [&](int s, const float* rp, const float* rs, float* np, float* ns) {
    const int k = s - lag;
    load(k + PF, np, ns);
    float res[SW];
#pragma unroll
    for (int w = 0; w < SW; ++w) res[w] = 0.0f;
    const int w0 = wlo(k);
    const bool active = k >= 0 && k < K;
    // position w of the sweep is diagonal d = dstart + w (alpha) or
    // dstart - w (beta); the row's cell there is t = d - u, in the lattice
    // for w_lo <= w < w_lo + cnt (kept as two integers rather than a lane
    // mask per position, which would take two scalar registers each)
    const int dstart = is_beta ? w0 + SW - 1 : w0 + 1;
    const int t0 = dstart - u;
    const int w_lo = is_beta ? max(t0 - (Tb - 1), 0) : max(-t0, 0);
    const int w_hi = is_beta ? min(t0, SW - 1) : min(Tb - 1 - t0, SW - 1);
    const unsigned cnt = active && u <= Ub ? (unsigned)max(w_hi + 1 - w_lo, 0) : 0u;
    if (active) {
      const int keep = is_beta ? dstart - D : 0;  // beta: positions above D pass the start value on
      // the neighbour row's value one position earlier: ring slot d - 1
      // (alpha) or d + 1 (beta)
      const int slot = w0 & (SRING - 1);
      float blkv[SW], vn[SW];
#pragma unroll
      for (int q = 0; q < SW / 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(my_ring + slot + 4 * q);
        blkv[4 * q] = v.x;
        blkv[4 * q + 1] = v.y;
        blkv[4 * q + 2] = v.z;
        blkv[4 * q + 3] = v.w;
      }
      vn[0] = my_ring[(is_beta ? slot + SW : slot - 1) & (SRING - 1)];
      // the ring values arrive before the window's first diagonal (a
      // scheduling boundary), not read just ahead of each use
#pragma unroll
      for (int q = 0; q < SW / 4; ++q)
        asm volatile("" ::"v"(blkv[4 * q]), "v"(blkv[4 * q + 1]), "v"(blkv[4 * q + 2]), "v"(blkv[4 * q + 3]));
      asm volatile("" ::"v"(vn[0]));
#pragma unroll
      for (int w = 1; w < SW; ++w) vn[w] = is_beta ? blkv[SW - w] : blkv[w - 1];
#pragma unroll
      for (int w = 0; w < SW; ++w) {
        const float op_p = rp[is_beta ? SW - 1 - w : w];
        const float op_s = rs[is_beta ? SW - 1 - w : w];
        const float nb = is_beta ? from_next_lane(cur, vn[w]) : from_prev_lane(cur, vn[w]);
        const float nxt = is_beta ? lae2<CLAMP>(add_operand(cur, op_p), add_operand2(nb, op_s))
                                  : lae2<CLAMP>(add_operand2(cur, op_p), add_operand(nb, op_s));
        const bool ok = (unsigned)(w - w_lo) < cnt;
        cur = ok ? nxt : (w < keep ? cur : kNegInf);
        res[w] = cur;
      }
      // the edge lane's values go to the neighbour wave's ring, by diagonal
      const int nbw = is_beta ? wave - 1 : wave + 1;
      if (nbw >= 0 && nbw < NW && lane == (is_beta ? 0 : 63)) {
        float* dst = ring + nbw * SRING + slot;
#pragma unroll
        for (int q = 0; q < SW / 4; ++q) {
          const int a = 4 * q;
          *reinterpret_cast<float4*>(dst + a) =
              is_beta ? make_float4(res[SW - 1 - a], res[SW - 2 - a], res[SW - 3 - a], res[SW - 4 - a])
                      : make_float4(res[a], res[a + 1], res[a + 2], res[a + 3]);
        }
      }
    }
    // stores: group g holds diagonals w0 + 4 g + e, sweep position
    // SW - 1 - 4 g - e (beta) or 4 g + e - 1 (alpha; position -1 is the
    // previous window's last result)
    const bool prev_ok = active && u <= Ub && (unsigned)(w0 - u) < (unsigned)Tb;
    const int wb = max(w0, 0);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float v[4];
      bool o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int w = is_beta ? SW - 1 - 4 * g - e : 4 * g + e - 1;
        v[e] = (w < 0 ? prev : res[w]) * kLn2;
        o[e] = w < 0 ? prev_ok : (unsigned)(w - w_lo) < cnt;
      }
      const unsigned so = (unsigned)((wb >> 2) + g) * gstride;
      // a group holding both cells and non-cells of some lane's row (only at
      // row starts and ends) is stored entry by entry, every other group with
      // one 16-byte store per lane (the choice is made per group: a choice
      // per window for all its groups made the beta results vary from run to
      // run)
      const bool full = o[0] && o[1] && o[2] && o[3];
      const bool part = (o[0] || o[1] || o[2] || o[3]) && !full;
      if (__builtin_amdgcn_ballot_w64(part) != 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) buf_st(v[e], rres, o[e] ? vo + 4u * e : kOffNone, so);
      } else {
        buf_st4(v, rres, full ? vo : kOffNone, so);
      }
    }
    if (!is_beta && active) prev = res[SW - 1];
    if (s >= 0) lds_sync();
  };

  // Steps -PF .. -1 only issue the first PF windows' loads. The loop runs
  // whole groups of PF + 1 steps (up to PF past the last window, which
  // compute and store nothing), so the loop body has no conditional step;
  // step s + j of a group loads into set j and computes from set j + 1.
  // Groups that start after this wave's last window (step K - 1 + lag) only
  // take part in the barriers; both branches pass the same barriers.
  const int last = K - 1 + lag;
  float rp[PF + 1][SW], rs[PF + 1][SW];
  for (int s = -PF; s < nsteps; s += PF + 1) {
    if (s <= last) {
#pragma unroll
      for (int j = 0; j <= PF; ++j) step(s + j, rp[(j + 1) % (PF + 1)], rs[(j + 1) % (PF + 1)], rp[j], rs[j]);
    } else {
#pragma unroll
      for (int j = 0; j <= PF; ++j)
        if (s + j >= 0) lds_sync();
    }
  }
  if (!is_beta && u == Ub) {
    // alpha(T_b-1, U_b) as this lane stored it (its last window's stores
    // complete first)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const int64_t last = lat_at(LatGeo{0, US}, Tb - 1, Ub);
    const float v = p.alpha[base0 + last] + phi[last];
    if (p.lnP) p.lnP[b] = v;
    if (p.costs) p.costs[b] = -v;
  }
}

// PF: windows of loads in flight ahead of the one computed (each costs
// 2 SW registers; 3 windows measured no faster than 2).
//
// Paired sweeps (up to four waves per sweep, so that two waves per SIMD keep
// the registers they need): workgroup j runs the alpha sweep
// of sample pair[2 j] on waves 0 .. NW-1 and the beta sweep of sample
// pair[2 j + 1] on waves NW .. 2 NW-1 (without a pairing, both of sample j).
// The two halves share the four SIMDs of one CU, two waves per SIMD, until
// the shorter sweep ends; after that the longer one has its SIMDs alone and
// runs faster (about 1.6x per diagonal, measured). Pairing the longest
// samples' sweeps with the shortest ones therefore shortens the longest
// workgroup, which sets the launch's time. Used when the 2 B sweeps
// outnumber the CUs (with fewer, each unpaired sweep has a CU of its own).
template <int NW, int SW, bool CLAMP>
__global__ void __launch_bounds__(128 * NW) lattice_pair_kernel(LatticeArgs p) {
  constexpr int PF = 2;
  __shared__ __attribute__((aligned(16))) float ring[2 * NW * SRING];
  const int j = blockIdx.x;
  const int ba = p.pair ? p.pair[2 * j] : j, bb = p.pair ? p.pair[2 * j + 1] : j;
  const int nsteps = max(lat_windows<SW>(p.T_len[ba], p.U_len[ba]), lat_windows<SW>(p.T_len[bb], p.U_len[bb])) + NW - 1;
  const int half = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) / NW;
  const int tid = threadIdx.x - half * 64 * NW;
  if (half == 0) lattice_body<NW, SW, PF, false, CLAMP>(p, ring, ba, tid, nsteps);
  else lattice_body<NW, SW, PF, true, CLAMP>(p, ring + NW * SRING, bb, tid, nsteps);
}

// One workgroup per (sample, direction): sweeps of more than four waves, and
// batches whose sweeps do not outnumber the CUs.
template <int NW, int SW, bool CLAMP>
__global__ void __launch_bounds__(64 * NW) lattice_kernel(LatticeArgs p) {
  constexpr int PF = 2;
  __shared__ __attribute__((aligned(16))) float ring[NW * SRING];
  const int b = blockIdx.x;
  const int nsteps = lat_windows<SW>(p.T_len[b], p.U_len[b]) + NW - 1;
  if (blockIdx.y == 0) lattice_body<NW, SW, PF, false, CLAMP>(p, ring, b, threadIdx.x, nsteps);
  else lattice_body<NW, SW, PF, true, CLAMP>(p, ring, b, threadIdx.x, nsteps);
}

template <bool CLAMP>
hipError_t launch_lattice_t(const LatticeArgs& a, int nw, bool paired, hipStream_t st) {
  const dim3 pairs(a.B), grid(a.B, 2);
  if (paired && nw <= 4) {
    if (nw <= 1) hipLaunchKernelGGL((lattice_pair_kernel<1, 16, CLAMP>), pairs, dim3(128), 0, st, a);
    else if (nw <= 2) hipLaunchKernelGGL((lattice_pair_kernel<2, 16, CLAMP>), pairs, dim3(256), 0, st, a);
    else if (nw <= 3) hipLaunchKernelGGL((lattice_pair_kernel<3, 16, CLAMP>), pairs, dim3(384), 0, st, a);
    else hipLaunchKernelGGL((lattice_pair_kernel<4, 16, CLAMP>), pairs, dim3(512), 0, st, a);
    return hipGetLastError();
  }
  if (nw <= 1) hipLaunchKernelGGL((lattice_kernel<1, 16, CLAMP>), grid, dim3(64), 0, st, a);
  else if (nw <= 2) hipLaunchKernelGGL((lattice_kernel<2, 16, CLAMP>), grid, dim3(128), 0, st, a);
  else if (nw <= 3) hipLaunchKernelGGL((lattice_kernel<3, 16, CLAMP>), grid, dim3(192), 0, st, a);
  else if (nw <= 4) hipLaunchKernelGGL((lattice_kernel<4, 16, CLAMP>), grid, dim3(256), 0, st, a);
  else if (nw <= 6) hipLaunchKernelGGL((lattice_kernel<6, 16, CLAMP>), grid, dim3(384), 0, st, a);
  else if (nw <= 8) hipLaunchKernelGGL((lattice_kernel<8, 16, CLAMP>), grid, dim3(512), 0, st, a);
  else if (nw <= 12) hipLaunchKernelGGL((lattice_kernel<12, 8, CLAMP>), grid, dim3(768), 0, st, a);
  else if (nw <= 16) hipLaunchKernelGGL((lattice_kernel<16, 8, CLAMP>), grid, dim3(1024), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_lattice(const LatticeArgs& a, int U1max, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const int nw = (U1max + 63) / 64;
  // pair the sweeps only when they outnumber the CUs: with fewer, each
  // unpaired sweep gets a CU of its own
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidDevice;
  const bool paired = 2 * (int64_t)a.B > cus;
  return a.clamp ? launch_lattice_t<true>(a, nw, paired, st) : launch_lattice_t<false>(a, nw, paired, st);
}

// Pruned lattice: the two log-probs of every cell outside its frame's band
// are -inf, so no alignment leaves such a cell (tiles the plan left out are
// never computed; the forward's merge writes the in-band cells of the others).
__global__ void band_fill_kernel(const int32_t* __restrict__ T_len, const int32_t* __restrict__ U_len,
                                 const int64_t* __restrict__ lat_off, const int32_t* __restrict__ band_lo, int S,
                                 int T, int U1, float* __restrict__ phi, float* __restrict__ psi) {
  const int b = blockIdx.y;
  const int Tb = T_len[b], Ub = U_len[b];
  const int64_t n = (int64_t)Tb * (Ub + 1);
  const LatGeo geo = lat_geo(lat_off, U_len, b);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / (Ub + 1)), u = (int)(i - (int64_t)t * (Ub + 1));
    const int lo = band_lo[(size_t)b * T + t];
    if (u < lo || u >= lo + S) {
      const int64_t ix = lat_at(geo, t, u);
      phi[ix] = kNegInf;
      psi[ix] = kNegInf;
    }
  }
}

hipError_t launch_band_fill(const int32_t* T_len, const int32_t* U_len, const int64_t* lat_off,
                            const int32_t* band_lo, int S, int B, int T, int U1, float* phi, float* psi,
                            hipStream_t st) {
  if (B == 0) return hipSuccess;
  const int64_t cells = (int64_t)T * U1;
  const int bx = (int)std::min<int64_t>(64, (cells + 255) / 256);
  hipLaunchKernelGGL(band_fill_kernel, dim3(bx, B), dim3(256), 0, st, T_len, U_len, lat_off, band_lo, S, T, U1, phi,
                     psi);
  return hipGetLastError();
}

// fp32 mode: the same recursions carried in fp64 (phi and psi widened from
// fp32). One workgroup per (sample, direction) walks the anti-diagonals, one
// barrier per diagonal; the previous diagonal is read back from the output
// array, which the workgroup's own stores made visible at the barrier. This
// sweep costs a few milliseconds at most at these sizes; its purpose is the
// precision of alpha + beta - ln P, which the backward pass exponentiates.
__device__ inline double lae64(double x, double y) {
  const double m = fmax(x, y);
  if (m == -INFINITY) return m;
  return m + log1p(exp(-fabs(x - y)));
}

__global__ void __launch_bounds__(256) lattice64_kernel(LatticeArgs p) {
  const int b = blockIdx.x;
  const bool is_beta = blockIdx.y != 0;
  const int Tb = p.T_len[b], Ub = p.U_len[b];
  const LatGeo geo = p.lat_off ? lat_geo_packed(p.lat_off[b], Ub) : lat_geo_padded(b, p.T, p.U1);
  double* out = is_beta ? p.beta64 : p.alpha64;
  const int D = Tb - 1 + Ub;  // last anti-diagonal
  for (int k = 0; k <= D; ++k) {
    const int dg = is_beta ? D - k : k;
    for (int u = threadIdx.x; u <= Ub; u += blockDim.x) {
      const int t = dg - u;
      if (t < 0 || t >= Tb) continue;
      const int64_t ix = lat_at(geo, t, u);
      double v;
      if (!is_beta) {
        if (t == 0 && u == 0) {
          v = 0.0;
        } else {
          double x = -INFINITY, y = -INFINITY;
          if (t > 0) {
            const int64_t j = lat_at(geo, t - 1, u);
            x = out[j] + (double)p.phi[j];
          }
          if (u > 0) {
            const int64_t j = lat_at(geo, t, u - 1);
            y = out[j] + (double)p.psi[j];
          }
          v = lae64(x, y);
        }
      } else {
        const double ph = (double)p.phi[ix];
        if (t == Tb - 1 && u == Ub) {
          v = ph;
        } else {
          double x = -INFINITY, y = -INFINITY;
          if (t + 1 < Tb) x = ph + out[lat_at(geo, t + 1, u)];
          if (u < Ub) y = (double)p.psi[ix] + out[lat_at(geo, t, u + 1)];
          v = lae64(x, y);
        }
      }
      out[ix] = v;
    }
    __syncthreads();
  }
  if (!is_beta && threadIdx.x == 0) {
    const int64_t ix = lat_at(geo, Tb - 1, Ub);
    const double v = out[ix] + (double)p.phi[ix];
    p.lnP64[b] = v;
    if (p.lnP) p.lnP[b] = (float)v;
    if (p.costs) p.costs[b] = (float)-v;
  }
}

hipError_t launch_lattice64(const LatticeArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  if (!a.alpha64 || !a.beta64 || !a.lnP64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lattice64_kernel, dim3(a.B, 2), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace rnnt
