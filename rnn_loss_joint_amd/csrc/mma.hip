// bf16 kernels on the large-tile MFMA core (mfma_core.hpp):
//   zrow     z = tanh(a + l) rows of a wave (and, in the forward, the blank /
//            label scores);
//   scores   256-score x 256-cell tiles of W^O z + b^O: forward (max, sum)
//            statistics (and the scores themselves in untiled mode) or
//            backward dh; used where the persistent kernels of scores3.hip
//            do not apply (untiled mode, H_pad < 512);
//   lse_merge  logsumexp over the V tiles' statistics, phi and psi.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_core.hpp"

namespace rnnt {


// ============================================================================ z and the two scores
// One workgroup per (32-t strip of a tile, group of 8 u values): thread
// (tt, q) = (tid / 8, tid % 8) owns t = strip start + tt and the 8-wide k
// chunks q, q+8, ...; each chunk of a[b, t] is loaded once and combined with
// the group's 8 rows of l (a and l arrive scaled by kTanhArgScale). Those 8 rows (and, with SCORES, the blank and
// label rows of W^O) are shared by all 32 t of the workgroup, so they are
// staged in LDS once instead of being loaded by every thread (which kept the
// vector memory address unit ~75 % busy). Writes z[row, k] = bf16(tanh(a + l))
// for k < H (0 up to z_ld and on padding rows t >= t0 + ht) and, with
// SCORES, the blank and label scores of each row as dot products of that
// bf16 z with the two W^O rows (plus the biases).
// ZM selects the outputs: bit 0 the bf16 z rows, bit 1 the E4M3 rows
// z8 = E4M3(z 2^8) of the fp8 output layer; with bit 1 the two scores are
// those of the E4M3 operands: the rounded z (exact in bf16) against the W^O
// rows of WO8 (decoded to bf16, also exact), scaled back by 2^-(8+e).
constexpr int kZHmax = 768;  // H_pad bound (the library's H <= 768)
template <bool SCORES, int NCH, int ZM>
__global__ void __launch_bounds__(256) zrow_kernel(ZArgs p) {
  constexpr bool Z16 = (ZM & 1) != 0, F8 = (ZM & 2) != 0;
  __shared__ __attribute__((aligned(16))) char smem[8 * kZHmax * 4 + (SCORES ? 9 * kZHmax * 2 : 0)];
  float* const ls = reinterpret_cast<float*>(smem);                 // [8][H_pad] l rows
  bf16* const ws = reinterpret_cast<bf16*>(smem + 8 * kZHmax * 4);  // [9][H_pad] blank, label rows
  const int tid = threadIdx.x;
  const int ug = blockIdx.x % p.n_ug;
  const int strip = p.strip_begin + blockIdx.x / p.n_ug;
  int lo = p.tile_begin, hi = p.tile_end - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (p.tiles[mid].strip0 <= strip) lo = mid; else hi = mid - 1;
  }
  const Tile tl = p.tiles[lo];
  const int u_first = ug * 8;
  if (u_first >= tl.wu) return;  // workgroup-uniform
  const int nu = min(8, tl.wu - u_first);
  const int tt = tid >> 3, q = tid & 7;
  const int tloc = (strip - tl.strip0) * 32 + tt;
  const bool row_ok = tloc < tl.ht;
  const int b = tl.b;
  const int u0 = tl.u0 + u_first;
  const int Hp = p.H_pad;
  const float* arow = p.a + ((size_t)b * p.T + tl.t0 + (row_ok ? tloc : 0)) * Hp;
  const float* lrow0 = p.l + ((size_t)b * p.U1 + u0) * Hp;
  const int64_t row0 = (int64_t)tl.row0 - p.buf_row_base + (int64_t)u_first * tl.htp + tloc;
  bf16* zb = reinterpret_cast<bf16*>(p.z);
  const bf16* WO = reinterpret_cast<const bf16*>(p.WO);
  const bf16* bO = reinterpret_cast<const bf16*>(p.bO);

  float hb[8], hy[8];
  int lab[8];
  if constexpr (SCORES) {
    const int Ub = p.U_len[b];
#pragma unroll
    for (int uu = 0; uu < 8; ++uu) {
      hb[uu] = 0.0f;
      hy[uu] = 0.0f;
      lab[uu] = (uu < nu && u0 + uu < Ub) ? p.labels[(size_t)b * p.U1 + u0 + uu + 1] : -1;
    }
  }
  // stage the group's l rows (rows past the tile repeat its last one) and the
  // W^O rows (0 past H)
  const int n4 = Hp / 4;
  for (int i = tid; i < 8 * n4; i += 256) {
    const int uu = i / n4, c = i - uu * n4;
    reinterpret_cast<f32x4*>(ls)[i] = ldg<f32x4>(lrow0 + (size_t)min(uu, nu - 1) * Hp + 4 * c);
  }
  if constexpr (SCORES) {
    const int n8 = Hp / 8;
    for (int i = tid; i < 9 * n8; i += 256) {
      const int r = i / n8, k = 8 * (i - r * n8);
      const int v = r == 0 ? p.blank : max(lab[r - 1], 0);
      if constexpr (F8) {
        // E4M3 W^O 2^e (zero past H) decoded; every E4M3 value is exact in bf16
        const u32x2 w8 = ldg<u32x2>(reinterpret_cast<const char*>(p.WO8) + (size_t)v * p.H8 + k);
        f32x8 wf;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w8[h], false);
          const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w8[h], true);
          wf[4 * h] = lo[0];
          wf[4 * h + 1] = lo[1];
          wf[4 * h + 2] = hi[0];
          wf[4 * h + 3] = hi[1];
        }
        reinterpret_cast<bf16x8*>(ws)[i] = __builtin_convertvector(wf, bf16x8);
      } else {
        reinterpret_cast<bf16x8*>(ws)[i] = k < p.H ? ldg<bf16x8>(WO + (size_t)v * p.H + k) : bf16x8{};
      }
    }
  }
  __syncthreads();
  // The thread's NCH 8-column chunks k = q*8 + 64 c (z_ld = 64 NCH) of a are
  // loaded half at a time, before any of that half's stores: with no load
  // among the stores and a fixed count of both, the compiler's waits cover
  // only the loads, and the stores are not drained chunk by chunk.
  constexpr int ZPH = NCH / 2;
  auto a_at = [&](int k) { return row_ok && k < p.H ? k : 0; };
#pragma unroll
  for (int c0 = 0; c0 < NCH; c0 += ZPH) {
    f32x4 av[ZPH][2];
#pragma unroll
    for (int c = 0; c < ZPH; ++c) {
      const int k = a_at(q * 8 + 64 * (c0 + c));
      av[c][0] = ldg<f32x4>(arow + k);
      av[c][1] = ldg<f32x4>(arow + k + 4);
    }
#pragma unroll
    for (int c = 0; c < ZPH; ++c) {
    const int k = q * 8 + 64 * (c0 + c);
    const bool kok = row_ok && k < p.H;
    const int kk = kok ? k : 0;
    const f32x4 a0 = av[c][0], a1 = av[c][1];
    bf16x8 xb;
    if constexpr (SCORES) xb = *reinterpret_cast<const bf16x8*>(ws + kk);
#pragma unroll
    for (int uu = 0; uu < 8; ++uu) {
      if (uu >= nu) continue;  // workgroup-uniform
      const f32x4 l0 = *reinterpret_cast<const f32x4*>(ls + uu * Hp + kk);
      const f32x4 l1 = *reinterpret_cast<const f32x4*>(ls + uu * Hp + kk + 4);
      f32x8 zf;
#pragma unroll
      for (int e = 0; e < 4; ++e) zf[e] = tanh_from_scaled(a0[e] + l0[e]);
#pragma unroll
      for (int e = 0; e < 4; ++e) zf[e + 4] = tanh_from_scaled(a1[e] + l1[e]);
      bf16x8 z = __builtin_convertvector(zf, bf16x8);  // adjacent pairs: one packed convert each
      if (!kok) z = bf16x8{};
      if constexpr (F8) {
        // E4M3(z 2^8), two packed converts per four values (round to nearest even)
        u32x2 q8;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(zf[4 * h] * 256.0f, zf[4 * h + 1] * 256.0f, 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(zf[4 * h + 2] * 256.0f, zf[4 * h + 3] * 256.0f, w, true);
          q8[h] = kok ? (uint32_t)w : 0u;
        }
        *reinterpret_cast<u32x2*>(reinterpret_cast<char*>(p.z8) + (row0 + (int64_t)uu * tl.htp) * p.z8_ld + k) = q8;
        if constexpr (SCORES) {
          // the scores' operand is the rounded value
          f32x8 zq;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)q8[h], false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)q8[h], true);
            zq[4 * h] = lo[0];
            zq[4 * h + 1] = lo[1];
            zq[4 * h + 2] = hi[0];
            zq[4 * h + 3] = hi[1];
          }
          z = __builtin_convertvector(zq, bf16x8);
        }
      }
      if constexpr (SCORES) {
        const bf16x8 xy = *reinterpret_cast<const bf16x8*>(ws + (uu + 1) * Hp + kk);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {  // bf16 pair dot products, fp32 accumulation
          const bf16x2 zz = {z[e], z[e + 1]};
          hb[uu] = __builtin_amdgcn_fdot2_f32_bf16(zz, bf16x2{xb[e], xb[e + 1]}, hb[uu], false);
          hy[uu] = __builtin_amdgcn_fdot2_f32_bf16(zz, bf16x2{xy[e], xy[e + 1]}, hy[uu], false);
        }
      }
      if constexpr (Z16) *reinterpret_cast<bf16x8*>(zb + (row0 + (int64_t)uu * tl.htp) * p.z_ld + k) = z;
    }
    }
  }
  if constexpr (SCORES) {
    const float bb = (float)bO[p.blank];
    const float sc = F8 ? __builtin_ldexpf(1.0f, -(8 + *p.ew)) : 1.0f;
#pragma unroll
    for (int uu = 0; uu < 8; ++uu) {
      float vb = hb[uu], vy = hy[uu];
#pragma unroll
      for (int off = 1; off < 8; off <<= 1) {
        vb += __shfl_xor(vb, off);
        vy += __shfl_xor(vy, off);
      }
      if (q == 0 && uu < nu) {
        const int64_t rr = row0 + (int64_t)uu * tl.htp;
        p.hb[rr] = __builtin_fmaf(vb, sc, bb);
        p.hy[rr] = lab[uu] >= 0 ? __builtin_fmaf(vy, sc, (float)bO[lab[uu]]) : 0.0f;
      }
    }
  }
}

hipError_t launch_zrow(const ZArgs& a, hipStream_t st) {
  if (a.n_strips == 0) return hipSuccess;
  if (a.H_pad > kZHmax || a.H_pad % 8 != 0 || a.z_ld > a.H_pad) return hipErrorInvalidValue;  // LDS staging bound
  const int zm = (a.z ? 1 : 0) | (a.z8 ? 2 : 0);
  if (zm == 0 || (a.z8 && (!a.WO8 || !a.ew || a.z8_ld < a.z_ld || a.H8 < a.z_ld))) return hipErrorInvalidValue;
  dim3 grid(a.n_strips * a.n_ug), block(256);
  switch (a.z_ld) {
#define RNNT_ZROW(N)                                                                         \
  case 64 * N:                                                                               \
    if (zm == 1) {                                                                           \
      if (a.hb) hipLaunchKernelGGL((zrow_kernel<true, N, 1>), grid, block, 0, st, a);        \
      else hipLaunchKernelGGL((zrow_kernel<false, N, 1>), grid, block, 0, st, a);            \
    } else if (zm == 2) {                                                                    \
      if (!a.hb) return hipErrorInvalidValue;                                                \
      hipLaunchKernelGGL((zrow_kernel<true, N, 2>), grid, block, 0, st, a);                  \
    } else {                                                                                 \
      if (a.hb) return hipErrorInvalidValue;                                                 \
      hipLaunchKernelGGL((zrow_kernel<false, N, 3>), grid, block, 0, st, a);                 \
    }                                                                                        \
    break;
    RNNT_ZROW(2) RNNT_ZROW(4) RNNT_ZROW(6) RNNT_ZROW(8) RNNT_ZROW(10) RNNT_ZROW(12)
#undef RNNT_ZROW
    default: return hipErrorInvalidValue;  // z rows are 128-column multiples up to kZHmax
  }
  return hipGetLastError();
}

// ============================================================================ row GEMM
// The joint pre-projections a = (W^A h^A + b^Z) s and l = (W^L h^L) s ("Neural
// transducer training ...", section "Transducer training", Eqs. (3)-(4), the
// separable joint), s = kTanhArgScale: 256 rows x 128 columns per workgroup
// on the large-tile core (both operands k-contiguous, streamed by dma).
__global__ void __launch_bounds__(256) rowgemm_kernel(RowGemmArgs p) {
  using namespace m3;
  __shared__ __attribute__((aligned(1024))) char lds[3 * (KcTile<256>::BYTES + KcTile<128>::BYTES)];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), wr = wave >> 1, wc = wave & 1;
  const int n0 = blockIdx.x * 128, m0 = blockIdx.y * 256;
  const bf16* A = reinterpret_cast<const bf16*>(p.A);
  const bf16* B = reinterpret_cast<const bf16*>(p.B);
  KcTile<256> la;
  la.init(wave, lane, p.K, [&](int row) -> const bf16* {
    const int m = m0 + row;
    return m < p.M ? A + (int64_t)m * p.lda : nullptr;
  });
  KcTile<128> lb;
  lb.init(wave, lane, p.K, [&](int row) -> const bf16* {
    const int n = n0 + row;
    return n < p.N ? B + (int64_t)n * p.ldb : nullptr;
  });
  Acc<128> acc;
  acc.zero();
  core<128, false, 3>(acc, la, lb, (p.K + BK - 1) / BK * BK, lds, tid);

  const bf16* bias = reinterpret_cast<const bf16*>(p.bias);
#pragma unroll
  for (int j = 0; j < Acc<128>::WN; ++j) {
    const int n = n0 + wc * 64 + j * 32 + (lane & 31);
    if (n >= p.c_cols) continue;
    const bool nok = n < p.N;
    const float bn = (nok && bias) ? (float)bias[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < Acc<128>::WM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + acc_row(wr, i, e, lane);
        if (m < p.M) p.C[(int64_t)m * p.ldc + n] = nok ? (acc.c[i][j][e] + bn) * p.scale : 0.0f;
      }
  }
}

hipError_t launch_rowgemm(const RowGemmArgs& a, hipStream_t st) {
  if (a.M <= 0 || a.c_cols <= 0) return hipSuccess;
  if (a.K % 8 || a.lda % 8 || a.ldb % 8 || reinterpret_cast<uintptr_t>(a.A) % 16 ||
      reinterpret_cast<uintptr_t>(a.B) % 16)
    return hipErrorInvalidValue;  // 16-byte operand pieces
  // at most 65535 row tiles per launch (grid y)
  constexpr int kMaxRows = 65535 * 256;
  for (int m0 = 0; m0 < a.M; m0 += kMaxRows) {
    RowGemmArgs c = a;
    c.A = reinterpret_cast<const bf16*>(a.A) + (int64_t)m0 * a.lda;
    c.C = a.C + (int64_t)m0 * a.ldc;
    c.M = std::min(kMaxRows, a.M - m0);
    dim3 grid((a.c_cols + 127) / 128, (c.M + 255) / 256), block(256);
    hipLaunchKernelGGL(rowgemm_kernel, grid, block, 0, st, c);
  }
  return hipGetLastError();
}

__global__ void mask_rows_kernel(bf16x8* __restrict__ dst, const bf16x8* __restrict__ src, int64_t n8, int c8,
                                 int Tdim, const int32_t* __restrict__ len, int add) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / c8;
    const int b = (int)(r / Tdim), t = (int)(r - (int64_t)b * Tdim);
    dst[i] = t < len[b] + add ? src[i] : bf16x8{};
  }
}

hipError_t launch_mask_rows(void* dst, const void* src, int64_t rows, int cols, int Tdim, const int32_t* len, int add,
                            hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (cols % 8 || reinterpret_cast<uintptr_t>(dst) % 16 || reinterpret_cast<uintptr_t>(src) % 16)
    return hipErrorInvalidValue;
  const int64_t n8 = rows * (cols / 8);
  const int blocks = (int)std::min<int64_t>((n8 + 255) / 256, 8192);
  hipLaunchKernelGGL(mask_rows_kernel, dim3(blocks), dim3(256), 0, st, reinterpret_cast<bf16x8*>(dst),
                     reinterpret_cast<const bf16x8*>(src), n8, cols / 8, Tdim, len, add);
  return hipGetLastError();
}

// ============================================================================ scores^T tiles
// C[v, c] = sum_k W^O[v, k] z[c, k] for a 256-score x 256-cell tile, so each
// lane holds whole cells (columns) and the reductions over the vocabulary are
// lane-local. The V tiles of one cell tile share an XCD.
//   forward: per cell, (max, sum exp) over the tile's scores (+ b^O) ->
//            partial statistics [row, V tile]; optionally the scores.
//   backward: dh = g*occ*exp(h - lse) - [v=blank] g*bflow - [v=y] g*lflow,
//            written [row, V_pad] in bf16.
template <bool BWD>
__global__ void __launch_bounds__(256) scores_kernel(ScoresArgs p) {
  using namespace m3;
  constexpr int STAGES_BYTES = 2 * 2 * KcTile<256>::BYTES;
  __shared__ __attribute__((aligned(1024))) char lds[STAGES_BYTES + 6 * 256 * 4];
  float* cell = reinterpret_cast<float*>(lds + STAGES_BYTES);  // [5][256] per-cell coefficients
  float* bias_l = cell + 5 * 256;  // b^O * log2(e) of this V tile; -1e30 past V
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), wr = wave >> 1, wc = wave & 1;
  const int nvt = (p.V + 255) / 256;
  const int id = blockIdx.x;
  const int xcd = id & 7, local = id >> 3;
  const int ct = (local / nvt) * 8 + xcd;
  const int vt = local % nvt;
  const int c0 = ct * 256;  // first row (buffer-relative) of the cell tile
  if (c0 >= p.n_rows) return;
  const bf16* WO = reinterpret_cast<const bf16*>(p.WO);
  const bf16* bO = reinterpret_cast<const bf16*>(p.bO);
  const bf16* zb = reinterpret_cast<const bf16*>(p.z);

  {
    const int v = vt * 256 + tid;
    bias_l[tid] = v < p.V ? (float)bO[v] * kLog2e : -1e30f;
  }
  // per-cell coefficients (backward)
  if (BWD) {
    const int rr = c0 + tid;  // buffer row
    // rows that are no cell keep lse = +inf: their dh is exactly 0 for any score
    float ls = kPosInf, co = 0.0f, cb = 0.0f, cl = 0.0f, lab = -1.0f;
    if (rr < p.n_rows) {
      const int R = rr + p.buf_row_base;
      int lo = p.tile_begin, hi = p.tile_end - 1;
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (p.tiles[mid].row0 <= R) lo = mid; else hi = mid - 1;
      }
      const Tile tl = p.tiles[lo];
      const int local_r = R - tl.row0;
      const int ul = local_r / tl.htp, tloc = local_r - ul * tl.htp;
      if (tloc < tl.ht) {
        const int b = tl.b, u = tl.u0 + ul, t = tl.t0 + tloc;
        const int Tb = p.T_len[b], Ub = p.U_len[b];
        const LatGeo geo = lat_geo(p.lat_off, p.U_len, b);
        const size_t idx = (size_t)lat_at(geo, t, u);
        const float lp = p.lnP[b];
        const float gb = p.dcosts ? p.dcosts[b] : 1.0f;
        const float A = p.alpha[idx], Bt = p.beta[idx];
        ls = p.lse[idx];
        const float bn = (t + 1 < Tb) ? p.beta[lat_at(geo, t + 1, u)] : (u == Ub ? 0.0f : kNegInf);
        co = gb * fexp2((A + Bt - lp) * kLog2e);
        cb = gb * fexp2((A + p.phi[idx] + bn - lp) * kLog2e);
        if (u < Ub) {
          cl = gb * fexp2((A + p.psi[idx] + p.beta[lat_at(geo, t, u + 1)] - lp) * kLog2e);
          lab = (float)p.labels[(size_t)b * p.U1 + u + 1];
        }
      }
    }
    cell[0 * 256 + tid] = ls * kLog2e;
    cell[1 * 256 + tid] = co;
    cell[2 * 256 + tid] = cb;
    cell[3 * 256 + tid] = cl;
    cell[4 * 256 + tid] = lab;
  }

  KcTile<256> la;
  la.init(wave, lane, p.H, [&](int row) -> const bf16* {
    const int v = vt * 256 + row;
    return v < p.V ? WO + (int64_t)v * p.H : nullptr;
  });
  KcTile<256> lb;
  lb.init(wave, lane, p.H, [&](int row) -> const bf16* {
    const int rr = c0 + row;
    return rr < p.n_rows ? zb + (int64_t)rr * p.z_ld : nullptr;
  });
  Acc<256> acc;
  acc.zero();
  core<256, false, 2>(acc, la, lb, (p.H + BK - 1) / BK * BK, lds, tid);

  // Lane columns: cells wc*128 + j*32 + (lane & 31). Rows: scores
  // acc_row(wr, i, e, lane); for fixed (i, e>>2) four consecutive rows, so the
  // bias of a lane's 16 rows of block i is four 16-byte LDS reads. Rows past V
  // carry a bias of -1e30 and drop out of the max and the sum.
  auto bias_block = [&](int i, f32x4* bq) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      bq[g] = *reinterpret_cast<const f32x4*>(bias_l + wr * 128 + i * 32 + 8 * g + 4 * (lane >> 5));
  };
  if (!BWD) {
    // scaled scores y = (W^O z + b^O) log2(e); per cell max and sum of
    // 2^(y - max), block by block (16 rows) with the running sum rescaled.
    float my[4], sm[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) { my[j] = -1e30f; sm[j] = 0.0f; }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 bq[4];
      bias_block(i, bq);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float y[16];
        float bm = my[j];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          y[e] = __builtin_fmaf(acc.c[i][j][e], kLog2e, bq[e >> 2][e & 3]);
          bm = __builtin_fmaxf(bm, y[e]);
        }
        float bs = sm[j] * fexp2(my[j] - bm);
#pragma unroll
        for (int e = 0; e < 16; ++e) bs += fexp2(y[e] - bm);
        my[j] = bm;
        sm[j] = bs;
      }
    }
    float mrow[4], srow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // combine with the other half-wave (same cells, other score rows)
      const float m2 = __shfl_xor(my[j], 32), s2 = __shfl_xor(sm[j], 32);
      const float mn = __builtin_fmaxf(my[j], m2);
      srow[j] = sm[j] * fexp2(my[j] - mn) + s2 * fexp2(m2 - mn);
      mrow[j] = mn;
    }
    // combine the two wave rows through LDS (stage buffers are free after the core)
    float* red = reinterpret_cast<float*>(lds);
    if (wr == 1 && lane < 32) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        red[(wc * 4 + j) * 64 + lane] = mrow[j];
        red[(wc * 4 + j) * 64 + 32 + lane] = srow[j];
      }
    }
    lds_barrier();
    if (wr == 0 && lane < 32) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float m2 = red[(wc * 4 + j) * 64 + lane], s2 = red[(wc * 4 + j) * 64 + 32 + lane];
        const float mn = __builtin_fmaxf(mrow[j], m2);
        const float sv = srow[j] * fexp2(mrow[j] - mn) + s2 * fexp2(m2 - mn);
        const int rr = c0 + wc * 128 + j * 32 + lane;
        if (rr < p.n_rows) p.stats[((int64_t)rr * nvt + vt)] = f32x2{mn * kLn2, sv};
      }
    }
    if (p.logits) {  // untiled: keep (W^O z) log2 e as fp16 (no bias), 4 consecutive v per store
      f16* lg = reinterpret_cast<f16*>(p.logits);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 bq[4];
        bias_block(i, bq);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = c0 + wc * 128 + j * 32 + (lane & 31);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int v = vt * 256 + acc_row(wr, i, 4 * g, lane);
            f16x4 w;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              w[q] = (f16)__builtin_amdgcn_fmed3f(acc.c[i][j][4 * g + q] * kLog2e, -kF16Max, kF16Max);
            if (rr < p.n_rows && v < p.V_pad)
              *reinterpret_cast<f16x4*>(lg + (int64_t)(rr + p.buf_row_base) * p.V_pad + v) = w;
          }
        }
      }
    }
  } else {
    // dh = co 2^(y - lse log2 e) - cb [v = blank] - cl [v = label]
    bf16* dh = reinterpret_cast<bf16*>(p.dh);
    float lsl[4], co[4], cb[4], cl[4];
    int lab[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cc = wc * 128 + j * 32 + (lane & 31);
      lsl[j] = cell[0 * 256 + cc];
      co[j] = cell[1 * 256 + cc];
      cb[j] = cell[2 * 256 + cc];
      cl[j] = cell[3 * 256 + cc];
      lab[j] = (int)cell[4 * 256 + cc];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 bq[4];
      bias_block(i, bq);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = c0 + wc * 128 + j * 32 + (lane & 31);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int v = vt * 256 + acc_row(wr, i, 4 * g, lane);
          bf16x4 w;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int vv = v + q;
            float d = co[j] * fexp2(__builtin_fmaf(acc.c[i][j][4 * g + q], kLog2e, bq[g][q]) - lsl[j]);
            d -= (vv == p.blank) ? cb[j] : 0.0f;
            d -= (vv == lab[j]) ? cl[j] : 0.0f;
            w[q] = (bf16)d;
          }
          if (rr < p.n_rows && v < p.V_pad) *reinterpret_cast<bf16x4*>(dh + (int64_t)rr * p.V_pad + v) = w;
        }
      }
    }
  }
}

hipError_t launch_scores(const ScoresArgs& a, bool bwd, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  const int nvt = (a.V + 255) / 256;
  const int nct = (a.n_rows + 255) / 256;
  const int groups = (nct + 7) / 8;
  dim3 grid(groups * 8 * nvt), block(256);
  if (bwd) hipLaunchKernelGGL(scores_kernel<true>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(scores_kernel<false>, grid, block, 0, st, a);
  return hipGetLastError();
}

// lse = logsumexp over the V tiles' partial statistics; phi, psi from the
// blank / label scores, for the valid cells. One workgroup per 32 t x 32 u
// block of a tile: the block's rows are read in row order (t fastest) and
// the results, transposed through LDS, are written group of four diagonals
// by group in (row, diagonal) order, so that each wave writes the 16-byte
// pieces of 16 consecutive rows (256 contiguous bytes of the lattice
// layout).
constexpr int kMB = 32, kMS = 34;  // block edge, LDS row stride (conflict-free both ways)
__global__ void __launch_bounds__(256) lse_merge_kernel(MergeArgs p) {
  __shared__ float sm[3][kMB * kMS];  // lse, phi, psi at [u][t]
  const Tile tl = p.tiles[p.tile_begin + blockIdx.x];
  const int tb = blockIdx.y * kMB, ub = blockIdx.z * kMB;
  if (tb >= tl.ht || ub >= tl.wu) return;
  const int nt = min(kMB, tl.ht - tb), nu = min(kMB, tl.wu - ub);
  const int b = tl.b, Ub = p.U_len[b];
  const LatGeo geo = lat_geo(p.lat_off, p.U_len, b);
#pragma unroll
  for (int i = threadIdx.x; i < kMB * kMB; i += 256) {
    const int ul = i / kMB, tt = i % kMB;
    if (ul >= nu || tt >= nt) continue;
    const int rr = tl.row0 + (ub + ul) * tl.htp + tb + tt - p.buf_row_base;
    float M = -1e30f;
    for (int v = 0; v < p.nvt; ++v) M = __builtin_fmaxf(M, p.stats[(int64_t)rr * p.nvt + v][0]);
    float S = 0.0f;
    for (int v = 0; v < p.nvt; ++v) {
      const f32x2 st = p.stats[(int64_t)rr * p.nvt + v];
      S += st[1] * fexp2((st[0] - M) * kLog2e);
    }
    const float lse = M + kLn2 * flog2(S);
    const int t = tl.t0 + tb + tt, u = tl.u0 + ub + ul;
    // a pruned lattice's cells outside their frame's band emit nothing
    bool in_band = true;
    if (p.band_lo) {
      const int lo = p.band_lo[(size_t)b * p.T + t];
      in_band = u >= lo && u < lo + p.band_S;
    }
    sm[0][ul * kMS + tt] = lse;
    sm[1][ul * kMS + tt] = in_band ? p.hb[rr] - lse : kNegInf;
    sm[2][ul * kMS + tt] = in_band && u < Ub ? p.hy[rr] - lse : kNegInf;
  }
  __syncthreads();
  // the block's diagonals T0 + U0 .. T0 + U0 + 62 lie in 17 groups from q0 on
  const int T0 = tl.t0 + tb, U0 = tl.u0 + ub, q0 = (T0 + U0) >> 2;
  constexpr int kGroups = (2 * kMB - 1 + 3) / 4 + 1;
#pragma unroll
  for (int i = threadIdx.x; i < kGroups * kMB * 4; i += 256) {
    const int e = i & 3, ul = (i >> 2) % kMB, gq = (i >> 2) / kMB;
    const int tt = 4 * (q0 + gq) + e - T0 - U0 - ul;  // t - T0 of the cell on that diagonal
    if (ul >= nu || tt < 0 || tt >= nt) continue;
    const size_t idx = (size_t)lat_at(geo, T0 + tt, U0 + ul);
    p.lse[idx] = sm[0][ul * kMS + tt];
    p.phi[idx] = sm[1][ul * kMS + tt];
    p.psi[idx] = sm[2][ul * kMS + tt];
  }
}

hipError_t launch_lse_merge(const MergeArgs& a, int tile_t, int tile_u, hipStream_t st) {
  const int ntiles = a.tile_end - a.tile_begin;
  if (ntiles <= 0) return hipSuccess;
  const dim3 grid(ntiles, (tile_t + kMB - 1) / kMB, (tile_u + kMB - 1) / kMB);
  hipLaunchKernelGGL(lse_merge_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace rnnt
