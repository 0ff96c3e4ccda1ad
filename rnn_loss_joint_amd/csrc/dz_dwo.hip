// bf16 backward products of one wave on the large-tile MFMA core
// (mfma_core.hpp), in one launch: dz = dh W^O with dtanh and the per-tile u / t
// sums ("Neural transducer training ...", section "Sample-wise method", the
// joint backward), and the split-K partials of dW^O = dh^T z and db^O.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_core.hpp"

namespace rnnt {

// ============================================================================ dW^O, db^O
// C[v, h] = sum over rows k of dh[k, v] * z[k, h]; column h = H of z reads the
// ones page, so C[v, H] = sum_k dh[k, v] = db^O[v]. Split-K partials.
// Workgroup ids are arranged so the tiles of one k split share an XCD (L2).
constexpr int kDwoLds = 2 * 2 * m3::MnTile<256>::BYTES;
__device__ __attribute__((always_inline)) inline void dwo_body(const DwoArgs& p, char* lds, int id) {
  using namespace m3;
  const int tid = threadIdx.x;
  const int nv = (p.V + BM - 1) / BM, nh = (p.H + 1 + 255) / 256;
  const int xcd = id & 7, local = id >> 3;
  const int per = nv * nh;
  const int split = (local / per) * 8 + xcd;
  if (split >= p.splits) return;
  const int rem = local % per;
  const int vt = rem / nh, ht = rem % nh;
  const int kb = split * p.k_per_split;
  const int ke = min(p.K, kb + p.k_per_split);

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  MnTile<256> la;
  la.init(Opnd{reinterpret_cast<const bf16*>(p.dh) + (int64_t)kb * p.dh_ld, p.dh_ld, p.V, max(0, ke - kb), -1},
          vt * 256, wave, tid & 63);
  MnTile<256> lb;
  lb.init(Opnd{reinterpret_cast<const bf16*>(p.z) + (int64_t)kb * p.z_ld, p.z_ld, p.H, max(0, ke - kb), p.H},
          ht * 256, wave, tid & 63);
  Acc<256> acc;
  acc.zero();
  const int kl = (max(0, ke - kb) + BK - 1) / BK * BK;
  core<256, true, 2>(acc, la, lb, kl, lds, tid);

  const int lane = tid & 63, wr = wave >> 1, wc = wave & 1;
  float* C = p.PW + (int64_t)split * p.V * p.H;
#pragma unroll
  for (int j = 0; j < Acc<256>::WN; ++j) {
    const int h = ht * 256 + wc * 128 + j * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < Acc<256>::WM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int v = vt * 256 + acc_row(wr, i, e, lane);
        if (v < p.V) {
          if (h < p.H) C[(int64_t)v * p.H + h] = acc.c[i][j][e];
          else if (h == p.H) p.PB[(int64_t)split * p.V + v] = acc.c[i][j][e];
        }
      }
  }
}


// ============================================================================ dz, dtanh, sums
// Workgroup = one 32-row strip of a tile (32 consecutive t) x 128 columns of
// H, walking the tile's u values eight at a time: M row i of a pass is
// (u = u0 + 8*ug + i/32, t = strip t + i%32). dz = dh . W^O (W^O^T operand is
// k-contiguous), ds = dz (1 - z^2) with z read from the row-major z buffer;
// sums over u stay in registers across passes (gA partial, written once);
// sums over the strip's t are written per u (gL partial).
constexpr int kDzLds = 3 * (m3::KcTile<256>::BYTES + m3::KcTile<128>::BYTES);
__device__ __attribute__((always_inline)) inline void dz2_body(const DzArgs& p, char* lds, int id) {
  using namespace m3;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), wr = wave >> 1, wc = wave & 1;
  const int nh = (p.H + 127) / 128;
  const int xcd = id & 7, local = id >> 3;
  const int strip_rel = (local / nh) * 8 + xcd;
  if (strip_rel >= p.n_strips) return;
  const int ht = local % nh;
  const int strip = p.strip_begin + strip_rel;
  const int h0 = ht * 128;

  int lo = p.tile_begin, hi = p.tile_end - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (p.tiles[mid].strip0 <= strip) lo = mid; else hi = mid - 1;
  }
  const Tile tl = p.tiles[lo];
  const int slot = lo - p.tile_begin;
  const int s_local = strip - tl.strip0;
  const int tl0 = s_local * 32;
  const int tile_row = tl.row0 - p.wave_row_base;
  const bf16* dh = reinterpret_cast<const bf16*>(p.dh);
  const bf16* zb = reinterpret_cast<const bf16*>(p.z);
  const bf16* wot = reinterpret_cast<const bf16*>(p.WOT);

  KcTile<128> lb;
  lb.init(wave, lane, p.V_pad, [&](int row) -> const bf16* {
    const int h = h0 + row;
    return h < p.H ? wot + (int64_t)h * p.V_pad : nullptr;
  });

  // gA partial: per wave, 32 t (lane rows) x its 64 columns, summed over u
  float gacc[Acc<128>::WN][16];
#pragma unroll
  for (int j = 0; j < Acc<128>::WN; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) gacc[j][e] = 0.0f;

  const int ngroups = (tl.wu + 7) / 8;
  for (int ug = 0; ug < ngroups; ++ug) {
    KcTile<256> la;
    la.init(wave, lane, p.V_pad, [&](int row) -> const bf16* {
      const int ul = ug * 8 + row / 32;
      return ul < tl.wu ? dh + (int64_t)(tile_row + ul * tl.htp + tl0 + row % 32) * p.V_pad : nullptr;
    });
    Acc<128> acc;
    acc.zero();
    core<128, false, 3>(acc, la, lb, (p.V_pad + BK - 1) / BK * BK, lds, tid);

    // wave rows: 4 blocks of 32 rows = u_local ug*8 + wr*4 + i. Row
    // 8(e>>2) + (e&3) of a block is wave-uniform, so each z load is a scalar
    // row base plus one per-lane offset (4 (lane>>5) rows + column h). All z
    // of the pass are loaded before any is used (one wait on memory per pass;
    // u rows past the tile read its first row and go unused).
    bf16x2 zv[4][Acc<128>::WN][8];  // packed pairs (elements 2q, 2q+1): 64 registers
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int zrow0 = tile_row + min(ug * 8 + wr * 4 + i, tl.wu - 1) * tl.htp + tl0;
#pragma unroll
      for (int j = 0; j < Acc<128>::WN; ++j) {
        const int h = h0 + wc * 64 + j * 32 + (lane & 31);
        const int loff = 4 * (lane >> 5) * p.z_ld + (h < p.H ? h : 0);
#pragma unroll
        for (int e = 0; e < 16; ++e)
          zv[i][j][e >> 1][e & 1] = (zb + (int64_t)(zrow0 + 8 * (e >> 2) + (e & 3)) * p.z_ld)[loff];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ul = ug * 8 + wr * 4 + i;
      if (ul >= tl.wu) continue;  // wave-uniform
#pragma unroll
      for (int j = 0; j < Acc<128>::WN; ++j) {
        const int h = h0 + wc * 64 + j * 32 + (lane & 31);
        const bool hok = h < p.H;
        float lsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float zf = (float)zv[i][j][e >> 1][e & 1];
          const float ds = hok ? acc.c[i][j][e] * (1.0f - zf * zf) : 0.0f;
          gacc[j][e] += ds;
          lsum += ds;
        }
        lsum += __shfl_xor(lsum, 32);
        if (lane < 32 && hok)
          p.PL[(((int64_t)slot * (p.tile_tp / 32) + s_local) * p.tile_u + ul) * p.H + h] = lsum;
      }
    }
  }

  // combine the two wave rows (same columns), then one write per (t, h)
  float* red = reinterpret_cast<float*>(lds);
  constexpr int PER = Acc<128>::WN * 16;
  if (wr == 1) {
#pragma unroll
    for (int j = 0; j < Acc<128>::WN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[((wc * PER) + j * 16 + e) * 64 + lane] = gacc[j][e];
  }
  __syncthreads();
  if (wr == 0) {
#pragma unroll
    for (int j = 0; j < Acc<128>::WN; ++j) {
      const int h = h0 + wc * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float v = gacc[j][e] + red[((wc * PER) + j * 16 + e) * 64 + lane];
        const int t = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (h < p.H) p.PA[((int64_t)slot * p.tile_tp + tl0 + t) * p.H + h] = v;
      }
    }
  }
}

// dz and dW^O of one wave in one launch: both read the same dh rows. The
// dW^O workgroups come first (ids 0 .. n_dwo-1, whole k splits per XCD, one
// round on part of the CUs); the dz workgroups fill the remaining CUs and
// then all of them. n_dwo is a multiple of 8, so both keep their XCD maps.
__global__ void __launch_bounds__(256) dz_dwo_kernel(DzArgs dz, DwoArgs dw, int n_dwo) {
  static_assert(kDzLds >= kDwoLds, "one LDS array serves both roles");
  __shared__ __attribute__((aligned(1024))) char lds[kDzLds];
  const int id = blockIdx.x;
  if (id < n_dwo) dwo_body(dw, lds, id);
  else dz2_body(dz, lds, id - n_dwo);
}

hipError_t launch_dz_dwo(const DzArgs& a, const DwoArgs& w, hipStream_t st) {
  const int nv = (w.V + 255) / 256, nhw = (w.H + 1 + 255) / 256;
  const int n_dwo = w.K > 0 ? (w.splits + 7) / 8 * 8 * nv * nhw : 0;
  const int nh = (a.H + 127) / 128;
  const int n_dz = a.n_strips > 0 ? (a.n_strips + 7) / 8 * 8 * nh : 0;
  if (n_dwo + n_dz == 0) return hipSuccess;
  hipLaunchKernelGGL(dz_dwo_kernel, dim3(n_dwo + n_dz), dim3(256), 0, st, a, w, n_dwo);
  return hipGetLastError();
}

}  // namespace rnnt
