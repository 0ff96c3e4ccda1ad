// bf16 MFMA building blocks for gfx950 shared by the large-tile kernels:
// global -> LDS dma, swizzled LDS fragment reads for v_mfma_f32_32x32x16_bf16,
// the lgkm / vm waits and barrier the pipelines use, operand tile loaders and
// the software-pipelined main loop.
//
// Every kernel that uses these must declare exactly one __shared__ array and
// carve all its LDS regions out of it: with several LDS variables the
// compiler attaches alias scopes and then makes every read of a stage buffer
// wait for all dma in flight, which removes the overlap of loads and MFMAs.
#pragma once

#include <algorithm>
#include <type_traits>

#include "common.hpp"

namespace rnnt {

// Sources for operand pieces outside the data: zeros, and bf16 ones (used to
// append a column of ones to an operand). One copy per code object.
static __device__ __attribute__((aligned(16))) uint32_t g_zero_page[4] = {0u, 0u, 0u, 0u};
static __device__ __attribute__((aligned(16))) uint32_t g_ones_page[4] = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u,
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

}  // namespace rnnt
