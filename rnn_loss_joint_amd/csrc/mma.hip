// Large-tile bf16 MFMA core for gfx950 and the bf16 kernels built on it.
//
// Core: 256 threads = 4 waves in a 2 x 2 grid over a BM x BN output tile
// (BM = 256, BN = 256 or 128), each wave 128 x BN/2, v_mfma_f32_32x32x16_bf16.
// Operand tiles are moved global -> LDS by global_load_lds_dwordx4 (no VGPR
// staging), NSTAGE stages in flight. A k-contiguous tile is stored
// [row][64 k] with 16-byte chunks XOR-swizzled by the row; an m-contiguous
// tile is stored [64 k][m] with 8-byte units XOR-swizzled by k and is read
// with ds_read_b64_tr_b16, which hands each lane four consecutive k of one m,
// so both orientations become MFMA fragments without register transposes.
// Pieces outside the operand read a zero page (or a page of bf16 ones, used
// to append a column of ones to an operand).
// Each kernel declares exactly one __shared__ array and carves every LDS
// region out of it: with several LDS variables the compiler attaches alias
// scopes and then makes every read of the stage buffers wait for all dma in
// flight, which removes the overlap of loads and MFMAs.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace rnnt {

__device__ __attribute__((aligned(16))) uint32_t g_zero_page[4] = {0u, 0u, 0u, 0u};
__device__ __attribute__((aligned(16))) uint32_t g_ones_page[4] = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u,
                                                                  0x3F803F80u};

namespace m3 {

constexpr int BM = 256;
constexpr int BK = 64;  // k (bf16 elements) per stage

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ inline void dma16(const void* g, const char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (lds_void*)(lds_wave_base), 16, 0, 0);
}

// k-contiguous fragment: row `row`, k-step ss of the stage, lane group g
__device__ inline bf16x8 frag_kc(const char* buf, int row, int ss, int g) {
  return *reinterpret_cast<const bf16x8*>(buf + lds_off(row, ss * 2 + g));
}

// XOR applied to the 8-byte unit index of k row k of an m-contiguous tile.
// A transposed read takes 4 units of each of 4 consecutive k rows per 16
// lanes (32 lanes: 8 units); the pattern puts those on distinct banks both
// per 16 lanes (128 bytes) and per 32 lanes (256 bytes).
__device__ inline int mn_swz(int k) { return (k & 1) * 20 ^ (k & 2) * 4; }

// ds_read_b64_tr_b16 issued from inline asm. Through the builtin the compiler
// makes every such read wait for all global->LDS dma in flight; here the
// caller waits on lgkmcnt itself (wait_frags) before the data is used.
typedef __attribute__((address_space(3))) const char lds_cchar;
__device__ inline u32x2 ds_read_tr16(const char* p) {
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"((uint32_t)(uintptr_t)(lds_cchar*)p));
  return v;
}

// m-contiguous fragment for m in [m_base, m_base+32), k-step ss; rowbytes =
// bytes of one k row of the tile. The two reads are outstanding on return.
__device__ inline bf16x8 frag_mn(const char* buf, int m_base, int ss, int lane, int rowbytes) {
  const int G = lane >> 4, L = lane & 15;
  const int m = m_base + 16 * (G & 1) + 4 * (L & 3);
  u32x4 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = ss * 16 + 8 * (G >> 1) + 4 * h + (L >> 2);
    const int unit = (m >> 2) ^ mn_swz(k);
    const u32x2 v = ds_read_tr16(buf + k * rowbytes + unit * 8);
    out[2 * h] = v[0];
    out[2 * h + 1] = v[1];
  }
  return __builtin_bit_cast(bf16x8, out);
}

// Waits until at most N LDS operations are outstanding; the fragments pass
// through the asm so that their uses cannot be scheduled above the wait.
template <int N, int NA, int NB>
__device__ inline void wait_frags(bf16x8 (&a)[NA], bf16x8 (&b)[NB]) {
  static_assert(NA == 4 && (NB == 4 || NB == 2), "fragment counts");
  if constexpr (NB == 4)
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3])
                 : "n"(N));
  else
    asm volatile("s_waitcnt lgkmcnt(%6)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1])
                 : "n"(N));
}

// Operand description for the core.
struct Opnd {
  const bf16* base;
  int64_t ld;      // elements between consecutive rows (kc) or k rows (mn)
  int rows;        // valid extent of the non-k dimension
  int K;           // valid k extent
  int ones_row;    // mn only: this m index reads the ones page (-1 = none)
};

// Loader of a k-contiguous operand tile [ROWS][BK]; rows given per thread.
template <int ROWS>
struct KcTile {
  static constexpr int INSTR = ROWS * 128 / 1024 / 4;  // dma instructions per wave per stage
  static constexpr int BYTES = ROWS * 128;
  const bf16* rowp[INSTR];
  int K, c;
  // row r of the tile is at rowptr(r) (nullptr = outside the operand)
  template <class F>
  __device__ void init(int wave, int lane, int K_, F rowptr) {
    K = K_;
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
      const int row = (i * 4 + wave) * 8 + (lane >> 3);
      rowp[i] = rowptr(row);
    }
    c = lane & 7;
  }
  // dma instruction i of stage k0 (i < INSTR, compile-time after unrolling)
  __device__ void issue_one(const char* stage, int wave, int lane, int k0, int i) const {
    const int row = (i * 4 + wave) * 8 + (lane >> 3);
    const int lc = c ^ swz(row);
    const int k = k0 + lc * 8;
    const void* g = (rowp[i] && k < K) ? (const void*)(rowp[i] + k) : (const void*)g_zero_page;
    dma16(g, stage + (i * 4 + wave) * 1024);
  }
};

// Loader of an m-contiguous operand tile [BK][M] (M = 256 or 128).
template <int M>
struct MnTile {
  static_assert(M >= 128, "mn_swz needs at least 32 units per k row");
  static constexpr int SLOTS = M / 8;                  // 16-byte slots per k row
  static constexpr int KPI = 64 / SLOTS;               // k rows per dma instruction
  static constexpr int INSTR = BK / KPI / 4;           // instructions per wave per stage
  static constexpr int BYTES = BK * M * 2;
  static constexpr int ROWBYTES = M * 2;
  // Instruction i of a thread moves k row kr0 + 4 KPI i; kr0 & 3 and hence
  // the swizzled column m are the same for every i, so one pointer (k row
  // kr0, column m) plus a uniform row offset addresses them all.
  const char* p0;      // data: &base[kr0][m]; otherwise the ones or zero page
  const char* zero;
  int64_t ldb;         // bytes per k row
  int kr0, K;
  bool data;
  __device__ void init(const Opnd& op, int m0, int wave, int lane) {
    kr0 = wave * KPI + lane / SLOTS;
    const int ls = (lane % SLOTS) ^ (mn_swz(kr0) >> 1);
    const int m = m0 + ls * 8;
    ldb = op.ld * 2;
    K = op.K;
    zero = reinterpret_cast<const char*>(g_zero_page);
    data = m < op.rows;
    p0 = data ? reinterpret_cast<const char*>(op.base + (int64_t)kr0 * op.ld + m)
              : (m == op.ones_row ? reinterpret_cast<const char*>(g_ones_page) : zero);
  }
  __device__ void issue_one(const char* stage, int wave, int lane, int k0, int i) const {
    const int kofs = k0 + i * 4 * KPI;  // uniform
    const char* g = kr0 + kofs < K ? (data ? p0 + kofs * ldb : p0) : zero;
    dma16(g, stage + (i * 4 + wave) * 1024);
  }
};

template <int BN>
struct Acc {
  static constexpr int WM = 4, WN = BN / 64;  // 32x32 blocks per wave
  f32x16 c[WM][WN];
  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) c[i][j] = f32x16{};
  }
};

// Workgroup barrier for LDS hand-over only: the wave's own LDS reads are
// complete, outstanding global->LDS dma is left in flight (a __syncthreads
// fence would wait for it).
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Number of outstanding dma instructions allowed while the oldest stage must be complete.
template <int N>
__device__ inline void wait_vm() {
  if constexpr (N >= 63) asm volatile("s_waitcnt vmcnt(63)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Main loop over k in [0, K_loop) (multiple of BK). LA/LB: tile loaders;
// MN selects the m-contiguous fragment reader for both operands. Stage s
// lives at lds + (s % NSTAGE) * STAGE_BYTES (A then B).
//
// Software pipeline, per stage of four k-steps: every MFMA of k-step ss is
// followed by a share of the fragment reads of k-step ss+1 (double-buffered
// registers), so LDS reads and their address arithmetic run under the MFMAs.
// The hand-over to the next stage (wait for its dma, barrier) sits before
// k-step 3; k-step 3 then reads the next stage's first fragments and issues
// the dma of stage q + NSTAGE into the slot just released.
template <int BN, bool MN, int NSTAGE, class LA, class LB>
__device__ void core(Acc<BN>& acc, const LA& la, const LB& lb, int K_loop, char* lds, int tid) {
  constexpr int WM = Acc<BN>::WM, WN = Acc<BN>::WN;
  constexpr int NMF = WM * WN;  // MFMAs per k-step
  constexpr int NFR = WM + WN;  // fragments per k-step
  constexpr int A_BYTES = LA::BYTES, B_BYTES = LB::BYTES;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int NDMA = LA::INSTR + LB::INSTR;  // dma per thread per stage
  static_assert(BK / 16 == 4, "four k-steps per stage");
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int r = lane & 31, g = lane >> 5;
  const int nq = K_loop / BK;
  if (nq == 0) return;

#define RNNT_FI __attribute__((always_inline))
  auto slot = [&](int s) RNNT_FI -> char* { return lds + (s % NSTAGE) * STAGE; };
  // d-th dma of stage s; a stage at or past nq reads only the zero page
  auto issue_dma = [&](int d, int s) RNNT_FI {
    char* st = slot(s);
    if (d < LA::INSTR) la.issue_one(st, wave, lane, s * BK, d);
    else lb.issue_one(st + A_BYTES, wave, lane, s * BK, d - LA::INSTR);
  };
  auto read_frag = [&](int f, const char* st, int ss, bf16x8* a, bf16x8* b) RNNT_FI {
    if (f < WM) {
      const int m = wr * 128 + f * 32;
      if constexpr (MN) a[f] = frag_mn(st, m, ss, lane, LA::ROWBYTES);
      else a[f] = frag_kc(st, m + r, ss, g);
    } else {
      const int n = wc * (BN / 2) + (f - WM) * 32;
      if constexpr (MN) b[f - WM] = frag_mn(st + A_BYTES, n, ss, lane, LB::ROWBYTES);
      else b[f - WM] = frag_kc(st + A_BYTES, n + r, ss, g);
    }
  };

  bf16x8 af[2][WM], bfr[2][WN];
  // one k-step: MFMAs on register buffer CB; the fragments of (rd_st, rd_ss)
  // go to buffer CB^1, spread over the MFMA slots; with DMA, also the dma of
  // stage dma_stage.
  auto kstep = [&](auto CB, auto DMA, const char* rd_st, int rd_ss, int dma_stage) RNNT_FI {
    constexpr int cb = decltype(CB)::value;
    constexpr bool dma = decltype(DMA)::value;
    if constexpr (MN) wait_frags<0>(af[cb], bfr[cb]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < NMF; ++x) {
      const int i = x / WN, j = x % WN;
      acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cb][i], bfr[cb][j], acc.c[i][j], 0, 0, 0);
#pragma unroll
      for (int f = 0; f < NFR; ++f)
        if (f * NMF / NFR == x) read_frag(f, rd_st, rd_ss, af[cb ^ 1], bfr[cb ^ 1]);
      if constexpr (dma) {
#pragma unroll
        for (int d = 0; d < NDMA; ++d)
          if (d * NMF / NDMA == x) issue_dma(d, dma_stage);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using NoDma = std::integral_constant<bool, false>;
  using Dma = std::integral_constant<bool, true>;

  // Prologue: stages 0 .. NSTAGE-2 in flight, stage 0 landed and its first
  // fragments read, then stage NSTAGE-1 in flight. From here on every stage
  // s issues exactly NDMA dma per thread (stages past the end read zeros),
  // so "stage s landed" is always "at most NSTAGE-2 later stages in flight".
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
#pragma unroll
    for (int d = 0; d < NDMA; ++d) issue_dma(d, s);
  wait_vm<(NSTAGE - 2) * NDMA>();
  lds_barrier();
#pragma unroll
  for (int f = 0; f < NFR; ++f) read_frag(f, slot(0), 0, af[0], bfr[0]);
#pragma unroll
  for (int d = 0; d < NDMA; ++d) issue_dma(d, NSTAGE - 1);

  for (int q = 0; q < nq; ++q) {
    const char* cur = slot(q);
    kstep(C0{}, NoDma{}, cur, 1, 0);
    kstep(C1{}, NoDma{}, cur, 2, 0);
    kstep(C0{}, NoDma{}, cur, 3, 0);
    wait_vm<(NSTAGE - 2) * NDMA>();  // stage q+1 landed
    lds_barrier();                     // every wave is done with slot q
    kstep(C1{}, Dma{}, slot(q + 1), 0, q + NSTAGE);
  }
  wait_vm<0>();   // the zero-page dma past the end must land before LDS is reused
  lds_barrier();  // LDS free for the caller's epilogue
#undef RNNT_FI
}

// row / col of accumulator element e of block (i, j) for this lane
__device__ inline int acc_row(int wr, int i, int e, int lane) { return wr * 128 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

}  // namespace m3

// ============================================================================ dW^O, db^O
// C[v, h] = sum over rows k of dh[k, v] * z[k, h]; column h = H of z reads the
// ones page, so C[v, H] = sum_k dh[k, v] = db^O[v]. Split-K partials.
// Workgroup ids are arranged so the tiles of one k split share an XCD (L2).
__global__ void __launch_bounds__(256) dwo_kernel(DwoArgs p) {
  using namespace m3;
  __shared__ __attribute__((aligned(1024))) char lds[2 * 2 * MnTile<256>::BYTES];
  const int tid = threadIdx.x;
  const int nv = (p.V + BM - 1) / BM, nh = (p.H + 1 + 255) / 256;
  const int id = blockIdx.x;
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

hipError_t launch_dwo(const DwoArgs& a, hipStream_t st) {
  const int nv = (a.V + 255) / 256, nh = (a.H + 1 + 255) / 256;
  const int groups = (a.splits + 7) / 8;
  dim3 grid(groups * 8 * nv * nh), block(256);
  hipLaunchKernelGGL(dwo_kernel, grid, block, 0, st, a);
  return hipGetLastError();
}

// ============================================================================ dz, dtanh, sums
// Workgroup = one 32-row strip of a tile (32 consecutive t) x 128 columns of
// H, walking the tile's u values eight at a time: M row i of a pass is
// (u = u0 + 8*ug + i/32, t = strip t + i%32). dz = dh . W^O (W^O^T operand is
// k-contiguous), ds = dz (1 - z^2) with z read from the row-major z buffer;
// sums over u stay in registers across passes (gA partial, written once);
// sums over the strip's t are written per u (gL partial).
__global__ void __launch_bounds__(256) dz2_kernel(DzArgs p) {
  using namespace m3;
  __shared__ __attribute__((aligned(1024))) char lds[3 * (KcTile<256>::BYTES + KcTile<128>::BYTES)];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), wr = wave >> 1, wc = wave & 1;
  const int nh = (p.H + 127) / 128;
  const int id = blockIdx.x;
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
    // row base plus one per-lane offset (4 (lane>>5) rows + column h).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ul = ug * 8 + wr * 4 + i;
      if (ul >= tl.wu) continue;  // wave-uniform
      const int zrow0 = tile_row + ul * tl.htp + tl0;
#pragma unroll
      for (int j = 0; j < Acc<128>::WN; ++j) {
        const int h = h0 + wc * 64 + j * 32 + (lane & 31);
        const bool hok = h < p.H;
        const int loff = 4 * (lane >> 5) * p.z_ld + (hok ? h : 0);
        float zv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const bf16* zr = zb + (int64_t)(zrow0 + 8 * (e >> 2) + (e & 3)) * p.z_ld;
          zv[e] = (float)zr[loff];
        }
        float lsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float ds = hok ? acc.c[i][j][e] * (1.0f - zv[e] * zv[e]) : 0.0f;
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

hipError_t launch_dz2(const DzArgs& a, hipStream_t st) {
  if (a.n_strips == 0) return hipSuccess;
  const int nh = (a.H + 127) / 128;
  const int groups = (a.n_strips + 7) / 8;
  dim3 grid(groups * 8 * nh), block(256);
  hipLaunchKernelGGL(dz2_kernel, grid, block, 0, st, a);
  return hipGetLastError();
}

// ============================================================================ z and the two scores
// One workgroup per (32-t strip of a tile, group of 8 u values): thread
// (tt, q) = (tid / 8, tid % 8) owns t = strip start + tt and the 8-wide k
// chunks q, q+8, ...; each chunk of a[b, t] is loaded once and combined with
// the group's 8 rows of l. Writes z[row, k] = bf16(tanh(a + l)) for k < H (0
// up to z_ld and on padding rows t >= t0 + ht) and, with SCORES, the blank
// and label scores of each row as dot products of that bf16 z with the two
// W^O rows (plus the biases).
template <bool SCORES>
__global__ void __launch_bounds__(256) zrow_kernel(ZArgs p) {
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
  const float* arow = p.a + ((size_t)b * p.T + tl.t0 + (row_ok ? tloc : 0)) * p.H_pad;
  const float* lrow0 = p.l + ((size_t)b * p.U1 + u0) * p.H_pad;
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
  const bf16* wb = WO + (size_t)p.blank * p.H;
  for (int k = q * 8; k < p.z_ld; k += 64) {
    const bool kok = row_ok && k < p.H;
    f32x4 a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = a0;
    bf16x8 xb;
    if (kok) {
      a0 = ldg<f32x4>(arow + k);
      a1 = ldg<f32x4>(arow + k + 4);
      if constexpr (SCORES) xb = ldg<bf16x8>(wb + k);
    }
#pragma unroll
    for (int uu = 0; uu < 8; ++uu) {
      if (uu >= nu) continue;  // workgroup-uniform
      bf16x8 z;
      if (kok) {
        const float* lrow = lrow0 + (size_t)uu * p.H_pad;
        const f32x4 l0 = ldg<f32x4>(lrow + k), l1 = ldg<f32x4>(lrow + k + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          z[e] = (bf16)tanh_fast(a0[e] + l0[e]);
          z[e + 4] = (bf16)tanh_fast(a1[e] + l1[e]);
        }
        if constexpr (SCORES) {
          const bf16x8 xy = ldg<bf16x8>(WO + (size_t)(lab[uu] >= 0 ? lab[uu] : 0) * p.H + k);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            hb[uu] = __builtin_fmaf((float)z[e], (float)xb[e], hb[uu]);
            hy[uu] = __builtin_fmaf((float)z[e], (float)xy[e], hy[uu]);
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = (bf16)0.0f;
      }
      *reinterpret_cast<bf16x8*>(zb + (row0 + (int64_t)uu * tl.htp) * p.z_ld + k) = z;
    }
  }
  if constexpr (SCORES) {
    const float bb = (float)bO[p.blank];
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
        p.hb[rr] = vb + bb;
        p.hy[rr] = lab[uu] >= 0 ? vy + (float)bO[lab[uu]] : 0.0f;
      }
    }
  }
}

hipError_t launch_zrow(const ZArgs& a, hipStream_t st) {
  if (a.n_strips == 0) return hipSuccess;
  dim3 grid(a.n_strips * a.n_ug), block(256);
  if (a.hb) hipLaunchKernelGGL(zrow_kernel<true>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(zrow_kernel<false>, grid, block, 0, st, a);
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
    float ls = 0.0f, co = 0.0f, cb = 0.0f, cl = 0.0f, lab = -1.0f;
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
        const size_t idx = ((size_t)b * p.U1 + u) * p.T + t;
        const float lp = p.lnP[b];
        const float gb = p.dcosts ? p.dcosts[b] : 1.0f;
        const float A = p.alpha[idx], Bt = p.beta[idx];
        ls = p.lse[idx];
        const float bn = (t + 1 < Tb) ? p.beta[idx + 1] : (u == Ub ? 0.0f : kNegInf);
        co = gb * fexp2((A + Bt - lp) * kLog2e);
        cb = gb * fexp2((A + p.phi[idx] + bn - lp) * kLog2e);
        if (u < Ub) {
          cl = gb * fexp2((A + p.psi[idx] + p.beta[idx + p.T] - lp) * kLog2e);
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
    if (p.logits) {  // untiled: keep the scores (bias included), 4 consecutive v per store
      bf16* lg = reinterpret_cast<bf16*>(p.logits);
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
              const float y = __builtin_fmaf(acc.c[i][j][4 * g + q], kLog2e, bq[g][q]) * kLn2;
              w[q] = (bf16)(v + q < p.V ? y : 0.0f);
            }
            if (rr < p.n_rows && v < p.V_pad)
              *reinterpret_cast<bf16x4*>(lg + (int64_t)(rr + p.buf_row_base) * p.V_pad + v) = w;
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
// blank / label scores; written to the [b, u, t] arrays for valid cells.
__global__ void __launch_bounds__(256) lse_merge_kernel(MergeArgs p) {
  const int rr = blockIdx.x * 256 + threadIdx.x;
  if (rr >= p.n_rows) return;
  const int R = rr + p.buf_row_base;
  int lo = p.tile_begin, hi = p.tile_end - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (p.tiles[mid].row0 <= R) lo = mid; else hi = mid - 1;
  }
  const Tile tl = p.tiles[lo];
  const int local_r = R - tl.row0;
  const int ul = local_r / tl.htp, tloc = local_r - ul * tl.htp;
  if (tloc >= tl.ht) return;
  const int b = tl.b, u = tl.u0 + ul, t = tl.t0 + tloc;
  float M = -1e30f;
  for (int v = 0; v < p.nvt; ++v) M = __builtin_fmaxf(M, p.stats[(int64_t)rr * p.nvt + v][0]);
  float S = 0.0f;
  for (int v = 0; v < p.nvt; ++v) {
    const f32x2 st = p.stats[(int64_t)rr * p.nvt + v];
    S += st[1] * fexp2((st[0] - M) * kLog2e);
  }
  const float lse = M + kLn2 * flog2(S);
  const size_t idx = ((size_t)b * p.U1 + u) * p.T + t;
  p.lse[idx] = lse;
  p.phi[idx] = p.hb[rr] - lse;
  p.psi[idx] = u < p.U_len[b] ? p.hy[rr] - lse : kNegInf;
}

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((a.n_rows + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace rnnt
