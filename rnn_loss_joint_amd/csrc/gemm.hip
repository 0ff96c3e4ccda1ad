// MFMA GEMMs for the joint pre-projections, the backward through the output
// layer and joint network, and the deterministic reductions that follow them
// ("Neural transducer training ...", section "Sample-wise method": the
// per-piece gradients of the joint network and output layer are accumulated,
// which gives the same result as one batched computation).
//
// Engine: 256 threads, 128 x 128 output tile, 2 x 2 waves of 64 x 64, k in
// 128-byte LDS stages (64 bf16 or 32 fp32), double buffered. Operands are
// staged into the swizzled [row][k] LDS layout of common.hpp either directly
// (k-contiguous sources) or through a 4 x 8 / 4 x 4 register transpose
// (m-contiguous sources), so every MFMA fragment is one 16-byte LDS read.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace rnnt {

namespace {

constexpr int TM = 128;  // workgroup tile

__device__ inline bool kvalid(const Operand& o, int k) {
  if (!o.kv_len) return true;
  int s = k / o.kv_T;
  return (k - s * o.kv_T) < o.kv_len[s] + o.kv_add;
}

// k-contiguous operand: piece i of thread tid is row i*32 + tid/8, chunk tid%8.
// A stage is loaded into a register set (load) and later written to LDS
// (store), so two sets give a prefetch distance of two stages.
template <class M, class S>
struct KcLoader {
  using CT = typename M::CT;
  static constexpr int KPL = M::KPL;
  struct Regs {
    u32x4 v[4];
  };
  const S* rowp[4];
  int c, K;
  __device__ void init(int tid, int K_) {
    c = tid & 7;
    K = K_;
  }
  __device__ void set_row(int i, const S* p) { rowp[i] = p; }
  __device__ void load(int k0, Regs& r) const {
    int k = k0 + c * KPL;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (rowp[i] && k < K) {
        if constexpr (sizeof(S) == sizeof(CT)) {
          r.v[i] = ldg<u32x4>(rowp[i] + k);
        } else {  // bf16 source, fp32 compute: 4 bf16 -> 4 floats
          u32x2 x = ldg<u32x2>(rowp[i] + k);
          r.v[i] = u32x4{x[0] << 16, x[0] & 0xffff0000u, x[1] << 16, x[1] & 0xffff0000u};
        }
      } else {
        r.v[i] = u32x4{0, 0, 0, 0};
      }
    }
  }
  __device__ void store(char* buf, int tid, const Regs& r) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(buf + lds_off(i * 32 + (tid >> 3), c)) = r.v[i];
  }
};

// m-contiguous operand: a thread covers 4 k rows x ER consecutive m and
// writes them transposed (bf16: ER = 8, one v_perm per output dword; fp32:
// ER = 4, register moves). bf16: 16 k-groups x 16 m-groups; fp32: 8 x 32.
template <class M, class S, bool COLSUM>
struct MnLoader {
  using CT = typename M::CT;
  static constexpr bool BF = sizeof(CT) == 2;
  static constexpr int ER = BF ? 8 : 4;
  static constexpr int NRQ = TM / ER;
  struct Regs {
    u32x4 v[4];  // v[i] = k row i: bf16 x 8 m (BF) or f32 x 4 m
  };
  Operand o;
  int K, m0, kq, rq;
  float cs[ER];
  __device__ void init(const Operand& op, int K_, int m0_, int tid) {
    o = op;
    K = K_;
    m0 = m0_;
    kq = tid / NRQ;
    rq = tid % NRQ;
#pragma unroll
    for (int e = 0; e < ER; ++e) cs[e] = 0.0f;
  }
  __device__ void load(int k0, Regs& r) {
    const int m = m0 + rq * ER;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int k = k0 + kq * 4 + i;
      bool ok = k < K && kvalid(o, k);
      const S* src = reinterpret_cast<const S*>(o.base) + (int64_t)k * o.ld + m;
      if (ok && m + ER <= o.rows) {
        if constexpr (BF || sizeof(S) == 4) {
          r.v[i] = ldg<u32x4>(src);  // 8 bf16 or 4 floats
        } else {                     // bf16 source, fp32 compute
          u32x2 x = ldg<u32x2>(src);
          r.v[i] = u32x4{x[0] << 16, x[0] & 0xffff0000u, x[1] << 16, x[1] & 0xffff0000u};
        }
      } else if (!ok || m >= o.rows) {
        r.v[i] = u32x4{0, 0, 0, 0};
      } else {  // partial m range at the edge
        if constexpr (BF) {
          uint32_t w[4] = {0, 0, 0, 0};
          const uint16_t* s16 = reinterpret_cast<const uint16_t*>(src);
          for (int e = 0; e < ER; ++e)
            if (m + e < o.rows) w[e >> 1] |= (uint32_t)s16[e] << (16 * (e & 1));
          r.v[i] = u32x4{w[0], w[1], w[2], w[3]};
        } else {
          float f[4] = {0, 0, 0, 0};
          for (int e = 0; e < ER; ++e)
            if (m + e < o.rows) f[e] = to_f32(src[e]);
          r.v[i] = __builtin_bit_cast(u32x4, f32x4{f[0], f[1], f[2], f[3]});
        }
      }
    }
  }
  // Column sums are taken here, one stage after the load was issued, so
  // they do not force an early wait on the outstanding loads.
  __device__ void store(char* buf, int, const Regs& r) {
    if constexpr (COLSUM) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (BF) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t x = r.v[i][w];
            cs[2 * w] += __uint_as_float(x << 16);
            cs[2 * w + 1] += __uint_as_float(x & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t x = r.v[i][w];  // scalar copy: a bit_cast of the vector element itself
            cs[w] += __uint_as_float(x);   // was miscompiled to read one element for every w
          }
        }
      }
    }
    if constexpr (BF) {
      // row m gets k = 4kq..4kq+3: dwords (k0|k1<<16, k2|k3<<16) of its m
#pragma unroll
      for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t sel = h ? 0x07060302u : 0x05040100u;
          u32x2 out = {__builtin_amdgcn_perm(r.v[1][w], r.v[0][w], sel),
                       __builtin_amdgcn_perm(r.v[3][w], r.v[2][w], sel)};
          const int row = rq * ER + 2 * w + h;
          *reinterpret_cast<u32x2*>(buf + lds_off(row, kq >> 1) + (kq & 1) * 8) = out;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < ER; ++e) {
        u32x4 out = {r.v[0][e], r.v[1][e], r.v[2][e], r.v[3][e]};
        *reinterpret_cast<u32x4*>(buf + lds_off(rq * ER + e, kq)) = out;
      }
    }
  }
};

template <class M>
struct WaveTile {
  static constexpr int W = 64 / M::ROWS;  // blocks per wave in m and n
  typename M::Acc acc[W][W];
  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < W; ++i)
#pragma unroll
      for (int j = 0; j < W; ++j) acc[i][j] = typename M::Acc{};
  }
  // one LDS stage: A rows [wr*64, +64), B rows [wc*64, +64)
  __device__ void mma_stage(const char* abuf, const char* bbuf, int wr, int wc, int lane) {
    using Frag = typename M::Frag;
    constexpr int SPS = 8 / M::GROUPS;
    const int r = lane % M::ROWS, g = lane / M::ROWS;
#pragma unroll
    for (int ss = 0; ss < SPS; ++ss) {
      Frag af[W], bfr[W];
#pragma unroll
      for (int i = 0; i < W; ++i)
        af[i] = *reinterpret_cast<const Frag*>(abuf + lds_off(wr * 64 + i * M::ROWS + r, ss * M::GROUPS + g));
#pragma unroll
      for (int j = 0; j < W; ++j)
        bfr[j] = *reinterpret_cast<const Frag*>(bbuf + lds_off(wc * 64 + j * M::ROWS + r, ss * M::GROUPS + g));
#pragma unroll
      for (int i = 0; i < W; ++i)
#pragma unroll
        for (int j = 0; j < W; ++j) acc[i][j] = M::mma(af[i], bfr[j], acc[i][j]);
    }
  }
};

// Full k loop over [kb, ke): two LDS buffers, two register sets per operand.
// Stage s+2 is requested from memory while stage s is multiplied and stage
// s+1 (requested one stage earlier) is written to LDS.
template <class M, class LA, class LB>
__device__ void mainloop(WaveTile<M>& wt, LA& la, LB& lb, int kb, int ke, char* lds, int tid) {
  constexpr int KST = 8 * M::KPL;
  constexpr int SB = TM * 128;  // bytes per operand stage
  const int lane = tid & 63, wave = tid >> 6, wr = wave >> 1, wc = wave & 1;
  if (kb >= ke) return;
  const int n = (ke - kb + KST - 1) / KST;
  typename LA::Regs a0, a1;
  typename LB::Regs b0, b1;
  la.load(kb, a0);
  lb.load(kb, b0);
  if (n > 1) {
    la.load(kb + KST, a1);
    lb.load(kb + KST, b1);
  }
  la.store(lds, tid, a0);
  lb.store(lds + 2 * SB, tid, b0);
  __syncthreads();
  for (int s = 0; s < n; s += 2) {
    // stage s in buffer 0, stage s+1 in set 1
    if (s + 2 < n) {
      la.load(kb + (s + 2) * KST, a0);
      lb.load(kb + (s + 2) * KST, b0);
    }
    wt.mma_stage(lds, lds + 2 * SB, wr, wc, lane);
    if (s + 1 < n) {
      la.store(lds + SB, tid, a1);
      lb.store(lds + 3 * SB, tid, b1);
    }
    __syncthreads();
    if (s + 1 >= n) break;
    // stage s+1 in buffer 1, stage s+2 in set 0
    if (s + 3 < n) {
      la.load(kb + (s + 3) * KST, a1);
      lb.load(kb + (s + 3) * KST, b1);
    }
    wt.mma_stage(lds + SB, lds + 3 * SB, wr, wc, lane);
    if (s + 2 < n) {
      la.store(lds, tid, a0);
      lb.store(lds + 2 * SB, tid, b0);
    }
    __syncthreads();
  }
}

}  // namespace

// ---------------------------------------------------------------- generic GEMM
template <class M, int KIND, class SA, class SB, bool COLSUM>
__global__ void __launch_bounds__(256) gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) char lds[4 * TM * 128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wr = wave >> 1, wc = wave & 1;
  const int n0 = blockIdx.x * TM, m0 = blockIdx.y * TM, split = blockIdx.z;
  const int kb = split * g.k_per_split;
  const int ke = min(g.K, kb + g.k_per_split);
  WaveTile<M> wt;
  wt.zero();
  const bool do_cs = COLSUM && blockIdx.x == 0;

  if constexpr (KIND == GEMM_KC_KC || KIND == GEMM_KC_MN) {
    KcLoader<M, SA> la;
    la.init(tid, g.K);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int m = m0 + i * 32 + (tid >> 3);
      la.set_row(i, m < g.A.rows ? reinterpret_cast<const SA*>(g.A.base) + (int64_t)m * g.A.ld : nullptr);
    }
    if constexpr (KIND == GEMM_KC_KC) {
      KcLoader<M, SB> lb;
      lb.init(tid, g.K);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int n = n0 + i * 32 + (tid >> 3);
        lb.set_row(i, n < g.B.rows ? reinterpret_cast<const SB*>(g.B.base) + (int64_t)n * g.B.ld : nullptr);
      }
      mainloop<M>(wt, la, lb, kb, ke, lds, tid);
    } else {
      MnLoader<M, SB, false> lb;
      lb.init(g.B, g.K, n0, tid);
      mainloop<M>(wt, la, lb, kb, ke, lds, tid);
    }
  } else {
    MnLoader<M, SA, COLSUM> la;
    la.init(g.A, g.K, m0, tid);
    if constexpr (KIND == GEMM_MN_MN) {
      MnLoader<M, SB, false> lb;
      lb.init(g.B, g.K, n0, tid);
      mainloop<M>(wt, la, lb, kb, ke, lds, tid);
    } else {
      KcLoader<M, SB> lb;
      lb.init(tid, g.K);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int n = n0 + i * 32 + (tid >> 3);
        lb.set_row(i, n < g.B.rows ? reinterpret_cast<const SB*>(g.B.base) + (int64_t)n * g.B.ld : nullptr);
      }
      mainloop<M>(wt, la, lb, kb, ke, lds, tid);
    }
    if constexpr (COLSUM) {
      if (do_cs) {
        // sum the per-thread column sums over the k groups
        float* red = reinterpret_cast<float*>(lds);
        constexpr int ER = MnLoader<M, SA, COLSUM>::ER;
        constexpr int NKQ = 256 / (TM / ER);
        __syncthreads();
#pragma unroll
        for (int e = 0; e < ER; ++e) red[la.kq * TM + la.rq * ER + e] = la.cs[e];
        __syncthreads();
        if (tid < TM && m0 + tid < g.M) {
          float s = 0.0f;
          for (int q = 0; q < NKQ; ++q) s += red[q * TM + tid];
          g.colsum[(int64_t)split * g.M + m0 + tid] = s;
        }
      }
    }
  }

  // epilogue: C[m, n] = acc (+ bias[n]); columns in [N, c_cols) get 0
  constexpr int W = WaveTile<M>::W;
  float* C = g.C + (int64_t)split * g.split_stride;
  const float osc = g.out_scale != 0.0f ? g.out_scale : 1.0f;
#pragma unroll
  for (int j = 0; j < W; ++j) {
    int n = n0 + wc * 64 + j * M::ROWS + M::col_of(lane);
    if (n >= g.c_cols) continue;
    float bias = 0.0f;
    if (g.bias && n < g.N)
      bias = g.bias_bf16 ? (float)reinterpret_cast<const bf16*>(g.bias)[n] : reinterpret_cast<const float*>(g.bias)[n];
#pragma unroll
    for (int i = 0; i < W; ++i) {
#pragma unroll
      for (int e = 0; e < M::NACC; ++e) {
        int m = m0 + wr * 64 + i * M::ROWS + M::row_of(e, lane);
        if (m < g.M) C[(int64_t)m * g.ldc + n] = (n < g.N) ? (wt.acc[i][j][e] + bias) * osc : 0.0f;
      }
    }
  }
}

template <class M, int KIND, class SA, class SB, bool CS>
static void launch_gemm_t(const GemmArgs& g, int splits, hipStream_t st) {
  dim3 grid((g.c_cols + TM - 1) / TM, (g.M + TM - 1) / TM, splits), block(256);
  hipLaunchKernelGGL((gemm_kernel<M, KIND, SA, SB, CS>), grid, block, 0, st, g);
}

hipError_t launch_gemm(const GemmArgs& g, GemmKind kind, bool bf16_compute, bool a_bf16, bool b_bf16,
                       int splits, hipStream_t st) {
  if (g.M <= 0 || g.c_cols <= 0 || splits <= 0) return hipSuccess;
  const bool cs = g.colsum != nullptr;
  if (bf16_compute) {
    if (!a_bf16 || !b_bf16) return hipErrorInvalidValue;
    switch (kind) {
      case GEMM_KC_KC: launch_gemm_t<MfmaBf16, GEMM_KC_KC, bf16, bf16, false>(g, splits, st); break;
      case GEMM_KC_MN: launch_gemm_t<MfmaBf16, GEMM_KC_MN, bf16, bf16, false>(g, splits, st); break;
      case GEMM_MN_MN:
        if (cs) launch_gemm_t<MfmaBf16, GEMM_MN_MN, bf16, bf16, true>(g, splits, st);
        else launch_gemm_t<MfmaBf16, GEMM_MN_MN, bf16, bf16, false>(g, splits, st);
        break;
      case GEMM_MN_KC:
        if (cs) launch_gemm_t<MfmaBf16, GEMM_MN_KC, bf16, bf16, true>(g, splits, st);
        else launch_gemm_t<MfmaBf16, GEMM_MN_KC, bf16, bf16, false>(g, splits, st);
        break;
    }
  } else {
#define RNNT_F32_CASES(SA, SB)                                                            \
  switch (kind) {                                                                        \
    case GEMM_KC_KC: launch_gemm_t<MfmaF32, GEMM_KC_KC, SA, SB, false>(g, splits, st); break; \
    case GEMM_KC_MN: launch_gemm_t<MfmaF32, GEMM_KC_MN, SA, SB, false>(g, splits, st); break; \
    case GEMM_MN_MN:                                                                     \
      if (cs) launch_gemm_t<MfmaF32, GEMM_MN_MN, SA, SB, true>(g, splits, st);           \
      else launch_gemm_t<MfmaF32, GEMM_MN_MN, SA, SB, false>(g, splits, st);             \
      break;                                                                             \
    case GEMM_MN_KC:                                                                     \
      if (cs) launch_gemm_t<MfmaF32, GEMM_MN_KC, SA, SB, true>(g, splits, st);           \
      else launch_gemm_t<MfmaF32, GEMM_MN_KC, SA, SB, false>(g, splits, st);             \
      break;                                                                             \
  }
    if (!a_bf16 && !b_bf16) { RNNT_F32_CASES(float, float) }
    else if (!a_bf16 && b_bf16) { RNNT_F32_CASES(float, bf16) }
    else return hipErrorInvalidValue;
#undef RNNT_F32_CASES
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- dz + dtanh + sums
// Workgroup = one 32-row strip (32 consecutive t of one tile) x 128 columns
// of H. It walks the tile's u values four at a time: rows of the 128-row
// M-tile are (u = u0 + 4*ug + i/32, t = strip t + i%32). For each group it
// computes dz = dh . W^O, ds = dz * (1 - z^2), adds ds over u into per-strip
// gA sums held in registers, and writes the sum over the strip's t of ds for
// every u (gL partial, one row per (strip, u)). The gA sums are written once
// at the end. Every partial slot has exactly one writer.
template <class M>
__global__ void __launch_bounds__(256) dz_kernel(DzArgs p) {
  using CT = typename M::CT;
  constexpr int ROWS = M::ROWS, NACC = M::NACC;
  constexpr int W = WaveTile<M>::W;
  constexpr int TS = 32 / ROWS;  // M-blocks per 32-row strip
  __shared__ __attribute__((aligned(16))) char lds[4 * TM * 128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wr = wave >> 1, wc = wave & 1;
  const int strip = p.strip_begin + blockIdx.x;
  const int h0 = blockIdx.y * TM;

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
  const CT* dh = reinterpret_cast<const CT*>(p.dh);
  const CT* zb = reinterpret_cast<const CT*>(p.z);

  float gacc[TS][W][NACC];
#pragma unroll
  for (int a = 0; a < TS; ++a)
#pragma unroll
    for (int j = 0; j < W; ++j)
#pragma unroll
      for (int e = 0; e < NACC; ++e) gacc[a][j][e] = 0.0f;

  const CT* wot = reinterpret_cast<const CT*>(p.WOT);
  KcLoader<M, CT> lb;
  lb.init(tid, p.V_pad);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int h = h0 + i * 32 + (tid >> 3);
    lb.set_row(i, h < p.H ? wot + (int64_t)h * p.V_pad : nullptr);
  }
  const int ngroups = (tl.wu + 3) / 4;
  for (int ug = 0; ug < ngroups; ++ug) {
    KcLoader<M, CT> la;
    la.init(tid, p.V_pad);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int row = i * 32 + (tid >> 3);
      int ul = ug * 4 + row / 32;
      la.set_row(i, ul < tl.wu ? dh + (int64_t)(tile_row + ul * tl.htp + tl0 + row % 32) * p.V_pad : nullptr);
    }
    WaveTile<M> wt;
    wt.zero();
    mainloop<M>(wt, la, lb, 0, p.V_pad, lds, tid);

    // epilogue for this u group
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const int mrow = wr * 64 + i * ROWS;  // first M row of the block
      const int ul = ug * 4 + mrow / 32;
      const int ts = (mrow % 32) / ROWS;
      const bool uok = ul < tl.wu;
      const int64_t zrow0 = (int64_t)(tile_row + ul * tl.htp + tl0 + (mrow % 32));
#pragma unroll
      for (int j = 0; j < W; ++j) {
        const int h = h0 + wc * 64 + j * ROWS + M::col_of(lane);
        float lsum = 0.0f;
#pragma unroll
        for (int e4 = 0; e4 < NACC; e4 += 4) {
          // rows row_of(e4..e4+3) are consecutive: one 4-element load of z^T
          float zz[4] = {0.0f, 0.0f, 0.0f, 0.0f};
          if (uok && h < p.H) {
            const CT* zp = zb + (int64_t)h * p.z_ld + zrow0 + M::row_of(e4, lane);
            if constexpr (sizeof(CT) == 2) {
              u32x2 w = ldg<u32x2>(zp);
              const uint32_t w0 = w[0], w1 = w[1];
              zz[0] = __uint_as_float(w0 << 16);
              zz[1] = __uint_as_float(w0 & 0xffff0000u);
              zz[2] = __uint_as_float(w1 << 16);
              zz[3] = __uint_as_float(w1 & 0xffff0000u);
            } else {
              f32x4 w = ldg<f32x4>(zp);
              zz[0] = w[0]; zz[1] = w[1]; zz[2] = w[2]; zz[3] = w[3];
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int e = e4 + q;
            float ds = (uok && h < p.H) ? wt.acc[i][j][e] * (1.0f - zz[q] * zz[q]) : 0.0f;
            gacc[ts][j][e] += ds;
            lsum += ds;
          }
        }
        wt.acc[i][j][0] = lsum;  // stash per-block t-sum for the gL reduction below
      }
    }
    // gL partial: sum over the strip's 32 t for each u (two u per wave row)
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const int ul = ug * 4 + wr * 2 + uu;
#pragma unroll
      for (int j = 0; j < W; ++j) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < W; ++i)
          if ((i * ROWS) / 32 == uu) s += wt.acc[i][j][0];
#pragma unroll
        for (int off = ROWS; off < 64; off <<= 1) s += __shfl_xor(s, off);
        const int h = h0 + wc * 64 + j * ROWS + M::col_of(lane);
        if (lane < ROWS && ul < tl.wu && h < p.H)
          p.PL[(((int64_t)slot * (p.tile_tp / 32) + s_local) * p.tile_u + ul) * p.H + h] = s;
      }
    }
    __syncthreads();
  }

  // gA partial: combine the two wave rows, then one write per (t, h)
  float* red = reinterpret_cast<float*>(lds);
  constexpr int PER = TS * W * NACC;
  if (wr == 1) {
#pragma unroll
    for (int a = 0; a < TS; ++a)
#pragma unroll
      for (int j = 0; j < W; ++j)
#pragma unroll
        for (int e = 0; e < NACC; ++e) red[((wc * PER) + (a * W + j) * NACC + e) * 64 + lane] = gacc[a][j][e];
  }
  __syncthreads();
  if (wr == 0) {
#pragma unroll
    for (int a = 0; a < TS; ++a)
#pragma unroll
      for (int j = 0; j < W; ++j) {
        const int h = h0 + wc * 64 + j * ROWS + M::col_of(lane);
#pragma unroll
        for (int e = 0; e < NACC; ++e) {
          float v = gacc[a][j][e] + red[((wc * PER) + (a * W + j) * NACC + e) * 64 + lane];
          const int t = a * ROWS + M::row_of(e, lane);
          if (h < p.H) p.PA[((int64_t)slot * p.tile_tp + tl0 + t) * p.H + h] = v;
        }
      }
  }
}

hipError_t launch_dz(const DzArgs& a, bool bf16_mode, hipStream_t st) {
  dim3 grid(a.n_strips, (a.H + TM - 1) / TM), block(256);
  if (a.n_strips == 0) return hipSuccess;
  if (bf16_mode) hipLaunchKernelGGL(dz_kernel<MfmaBf16>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(dz_kernel<MfmaF32>, grid, block, 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- reductions
// One workgroup per (group, row j of the group): dst row += the partial rows
// of the group's tiles, in plan order (deterministic). 16-byte accesses: H is
// a multiple of 8 and every partial row starts 16-byte aligned.
__global__ void __launch_bounds__(256) group_reduce_kernel(GroupReduceArgs p) {
  const Tile* tiles = p.tiles;
  const int gi = blockIdx.x, j = blockIdx.y;
  const Group gr = p.groups[gi];
  if (j >= gr.len) return;
  f32x4* dst = reinterpret_cast<f32x4*>(p.G + ((int64_t)gr.b * p.Gdim + gr.start + j) * p.H);
  for (int h4 = threadIdx.x; h4 < p.H / 4; h4 += blockDim.x) {
    f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = 0; c < gr.count; ++c) {
      const int tid = p.idx[gr.first + c];
      const int nsub = p.n_sub ? tiles[tid].htp / 32 : 1;
      const float* src = p.P + (int64_t)(tid - p.tile_begin) * p.tile_stride + (int64_t)j * p.H + 4 * h4;
      for (int q = 0; q < nsub; ++q) s += *reinterpret_cast<const f32x4*>(src + q * p.sub_stride);
    }
    dst[h4] += s;
  }
}

hipError_t launch_group_reduce(const GroupReduceArgs& a, hipStream_t st) {
  if (a.n_groups == 0) return hipSuccess;
  if (a.H % 4 || a.tile_stride % 4 || a.sub_stride % 4 || reinterpret_cast<uintptr_t>(a.P) % 16 ||
      reinterpret_cast<uintptr_t>(a.G) % 16)
    return hipErrorInvalidValue;  // the kernel moves 16-byte pieces
  dim3 grid(a.n_groups, a.max_len), block(256);
  hipLaunchKernelGGL(group_reduce_kernel, grid, block, 0, st, a);
  return hipGetLastError();
}

__global__ void to_bf16_kernel(const f32x4* __restrict__ src, bf16x4* __restrict__ dst, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = __builtin_convertvector(src[i], bf16x4);
}

hipError_t launch_to_bf16(const float* src, void* dst, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (n % 4) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  const int blocks = (int)std::min<int64_t>((n4 + 255) / 256, 8192);
  hipLaunchKernelGGL(to_bf16_kernel, dim3(blocks), dim3(256), 0, st, reinterpret_cast<const f32x4*>(src),
                     reinterpret_cast<bf16x4*>(dst), n4);
  return hipGetLastError();
}

// out[i] (+)= sum over q of P[q stride + i], q in order; T = float or f32x4
// (n and stride then count 16-byte pieces)
template <class T>
__global__ void split_reduce_kernel(T* out, const T* P, int64_t n, int splits, int64_t stride, int acc) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    T s = acc ? out[i] : T{};
    for (int q = 0; q < splits; ++q) s += P[q * stride + i];
    out[i] = s;
  }
}

hipError_t launch_split_reduce(float* out, const float* P, int64_t n, int splits, int64_t stride,
                               bool accumulate, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (n % 4 == 0 && stride % 4 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0 &&
      reinterpret_cast<uintptr_t>(P) % 16 == 0) {
    const int blocks = (int)std::min<int64_t>((n / 4 + 255) / 256, 4096);
    hipLaunchKernelGGL(split_reduce_kernel<f32x4>, dim3(blocks), dim3(256), 0, st, reinterpret_cast<f32x4*>(out),
                       reinterpret_cast<const f32x4*>(P), n / 4, splits, stride / 4, accumulate ? 1 : 0);
  } else {
    const int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(split_reduce_kernel<float>, dim3(blocks), dim3(256), 0, st, out, P, n, splits, stride,
                       accumulate ? 1 : 0);
  }
  return hipGetLastError();
}

// W^O [V, H] -> W^O^T [H, V_pad] through a 32 x 32 LDS tile.
template <class T>
__global__ void __launch_bounds__(256) transpose_wo_kernel(T* dst, const T* src, int V, int H, int V_pad) {
  __shared__ T tile[32][33];
  const int v0 = blockIdx.x * 32, h0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int y = ty; y < 32; y += 8) {
    int v = v0 + y, h = h0 + tx;
    tile[y][tx] = (v < V && h < H) ? src[(int64_t)v * H + h] : T(0.0f);
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    int h = h0 + y, v = v0 + tx;
    if (h < H && v < V_pad) dst[(int64_t)h * V_pad + v] = tile[tx][y];
  }
}

hipError_t launch_transpose_wo(void* dst, const void* src, int V, int H, int V_pad, bool bf16, hipStream_t st) {
  dim3 grid((V_pad + 31) / 32, (H + 31) / 32), block(256);
  if (bf16)
    hipLaunchKernelGGL(transpose_wo_kernel<__bf16>, grid, block, 0, st, reinterpret_cast<__bf16*>(dst),
                       reinterpret_cast<const __bf16*>(src), V, H, V_pad);
  else
    hipLaunchKernelGGL(transpose_wo_kernel<float>, grid, block, 0, st, reinterpret_cast<float*>(dst),
                       reinterpret_cast<const float*>(src), V, H, V_pad);
  return hipGetLastError();
}

__global__ void fill_kernel(float* p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int blocks = (int)std::min<int64_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(fill_kernel, dim3(blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

__global__ void fill_bytes_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0u;
}

hipError_t launch_fill_bytes(void* p, int64_t nbytes, hipStream_t st) {
  int64_t n = nbytes / 4;
  if (n <= 0) return hipSuccess;
  int blocks = (int)std::min<int64_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(fill_bytes_kernel, dim3(blocks), dim3(256), 0, st, reinterpret_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace rnnt
