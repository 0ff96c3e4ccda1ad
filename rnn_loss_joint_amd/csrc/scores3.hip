// Persistent score-tile kernels of the bf16 tiled path, and their helpers.
//
// The output projection h = W^O z + b^O ("Neural transducer training ...",
// section "Transducer training", Eq. (4)) is computed transposed, 256 scores
// (rows) x 128 lattice cells (columns) per work item, so each lane holds whole
// cells and the reductions over the vocabulary stay lane-local:
//   forward : per cell and 256-score slice, (max, sum 2^(y - max)) of the
//             scaled scores y = (W^O z + b^O) log2 e (the log-softmax
//             denominator of Eq. (5) in pieces, merged afterwards);
//   backward: dh = occupancy * softmax (Eq. (10) without the blank / label
//             terms, which a separate pass subtracts) written as bf16;
//   forward with a store (untiled mode): also the scaled products
//             (W^O z) log2 e without the bias, as fp16, for a backward
//             without recomputation (which adds b^O log2 e back in fp32).
//
// One workgroup per CU (256 threads, 4 waves of 128 x 64 outputs) walks its
// list of items; the A operand (a 256-row slice of a zero-padded copy of
// W^O) and the B operand (128 rows of z) move global -> LDS by dma in three
// 48 KB stages. The epilogue of item n runs inside the first five stages of
// item n+1, a few VALU instructions after each MFMA, on the second of two
// accumulator sets, so exp2 and the other vector work overlap the matrix
// cores. Per-item bias and cell coefficients arrive by dma with the stages.
//
// FP8 variant: the same pipeline over OCP E4M3 operands (z scaled by 2^8,
// W^O by 2^e): a stage's 128 bytes per row are 128 k values, taken by two
// 32 x 32 x 64 MFMAs per block; an fp8 fragment (32 bytes per lane) is the
// pair of 16-byte pieces the bf16 kernel reads for two k-steps, so the LDS
// layout, swizzle and dma are unchanged. The fragments are single-buffered
// (each one re-read right after its last MFMA of the k-step), which keeps
// the register count of the bf16 kernel's double buffers. The scores are
// scaled back by 2^-(8+e) in the epilogue.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_core.hpp"
#include "scores3_map.hpp"

namespace rnnt {
namespace s3 {

constexpr int BN = s3map::BN;  // cells per item
constexpr int BK = s3map::BK;
constexpr int NST = s3map::NST;  // stages in flight
constexpr int A_BYTES = s3map::A_BYTES;
constexpr int B_BYTES = s3map::B_BYTES;
constexpr int STAGE = A_BYTES + B_BYTES;
constexpr int NDA = s3map::NDA;  // 16-byte dma per thread per stage
constexpr int NDB = s3map::NDB;
// backward: per wave, one finished 32 x 32 block of dh (bf16) [cell][score],
// rows of 80 bytes (64 used), so dh goes out as whole 64-byte row pieces
constexpr int DHS_ROW = 80, DHS_WAVE = 32 * DHS_ROW;
// LDS regions after the stages. Item n's bias (and, backward, coefficients)
// sit in buffer n mod NBUF: with bf16 an item has at least 8 stages, so the
// dma of item n+1's first stages (issued three stages ahead) starts after
// item n-1's epilogue (in item n's first five stages) has read its buffers;
// with fp8 (5 stages per item at H = 640) it does not, so three buffers.
// The block staging area serves the backward's dh and the stored scores.
template <bool BWD, bool FP8, bool STORE>
struct Lay {
  static constexpr int NBUF = FP8 ? 3 : 2;
  static constexpr int OFF_BIAS = NST * STAGE;               // [NBUF][256] f32: b^O log2 e
  static constexpr int OFF_COEF = OFF_BIAS + NBUF * 256 * 4; // [NBUF][128][2] f32: (lse log2 e, occupancy)
  static constexpr int OFF_RED = OFF_COEF + NBUF * 256 * 4;  // [2 wc][2 j][2][32] f32 (forward)
  static constexpr int RED_BYTES = (BWD && FP8) ? 0 : 2 * 2 * 2 * 32 * 4;
  static constexpr int OFF_DHS = OFF_RED + RED_BYTES;
  static constexpr int BYTES = (BWD || STORE) ? OFF_DHS + 4 * DHS_WAVE : OFF_DHS;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};
constexpr int WM = 4, WN = 2;  // 32 x 32 blocks per wave
constexpr int EPI_STAGES = 5;  // stages of item n+1 that carry the epilogue of item n

typedef __attribute__((address_space(3))) void lds_void;

__device__ inline void dma_b128(const char* g, char* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g, (lds_void*)l, 16, 0, 0);
}
__device__ inline void dma_b32(const char* g, char* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g, (lds_void*)l, 4, 0, 0);
}

}  // namespace s3

typedef int i32x8 __attribute__((ext_vector_type(8)));

template <bool BWD, bool FP8, bool STORE>
__global__ void __launch_bounds__(256) scores3_kernel(Scores3Args p) {
  static_assert(!STORE || (!BWD && !FP8), "scores are stored by the bf16 forward only");
  using namespace s3;
  using m3::lds_barrier;
  using m3::wait_vm;
  using LY = Lay<BWD, FP8, STORE>;
  constexpr int NBUF = LY::NBUF, OFF_BIAS = LY::OFF_BIAS, OFF_COEF = LY::OFF_COEF, OFF_RED = LY::OFF_RED,
                OFF_DHS = LY::OFF_DHS;
  __shared__ __attribute__((aligned(1024))) char lds[LY::BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int r = lane & 31, g = lane >> 5;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  // row lengths in 2-byte units (fp8: 128 values per stage and row)
  const int hrow = FP8 ? p.H8 / 2 : p.H_pad;
  const int64_t zld = FP8 ? p.z8_ld / 2 : p.z_ld;
  const int nvt = p.nvt, nq = hrow / BK;
  // items (ct, vt) of this workgroup, see scores3_map.hpp
  const int nctl = s3map::nctl_of(p.n_ct, xcd);
  const int n_items = s3map::items_of(p.n_ct, nvt, xcd, slot);
  if (n_items == 0) return;
  constexpr int ND = NDA + NDB + (BWD ? 2 : 1);  // dma per thread per stage

  // Per-thread dma source offsets (bytes). Instruction d moves rows
  // 32 d + 8 wave + lane/8 (8 rows x 8 chunks of 16 bytes); the chunk swizzle
  // of those rows depends only on d & 1, so two offsets per operand plus a
  // uniform 32 d rows address every instruction.
  uint32_t offA[2], offB[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    offA[i] = s3map::dma_thread_off(i, wave, lane, hrow);
    offB[i] = s3map::dma_thread_off(i, wave, lane, (int)zld);
  }
  const int64_t stepA = (int64_t)32 * hrow * 2, stepB = (int64_t)32 * zld * 2;
  // Fragment reads: row wr*128 + 32 f + r of A (wc*64 + 32 f + r of B), chunk
  // (2 ss + g) ^ swz(row); swz(row) = s0 ^ 4 (f & 1) with s0 = swz(r), so the
  // per-lane part is rb + (c0[ss] ^ 64 (f & 1)) and 4096 f is an immediate.
  const int s0 = swz(r);
  const uint32_t rbA = (uint32_t)((wr * 128 + r) * 128), rbB = (uint32_t)(A_BYTES + (wc * 64 + r) * 128);
  const char* WOp = reinterpret_cast<const char*>(FP8 ? p.WO8 : p.WOp);
  const char* zb = reinterpret_cast<const char*>(FP8 ? p.z8 : p.z);
  // scores in log2 units: acc (log2 e) for bf16, acc 2^-(8+e) (log2 e) for fp8
  const float ysc = FP8 ? kLog2e * __builtin_ldexpf(1.0f, -(8 + *p.ew)) : kLog2e;
  const char* blt = reinterpret_cast<const char*>(p.bl);
  const char* cft = reinterpret_cast<const char*>(p.coefA);

  auto item_of = [&](int n, int& ct, int& vt) {
    const s3map::Item it = s3map::item_of(n, n_items, nctl, nvt, xcd, slot);
    ct = it.ct;
    vt = it.vt;
  };
  struct Src {
    const char *a, *b, *bias, *coef;
    char* st;
    int par;
  };
  auto stage_src = [&](int S) {
    const s3map::StageSrc o = s3map::stage_src(S, nq, n_items, nctl, nvt, xcd, slot, hrow, zld, NBUF);
    Src s;
    s.a = WOp + o.a;
    s.b = zb + o.b;
    s.bias = blt + o.bias;
    s.coef = cft + o.coef;
    s.st = lds + (S % NST) * STAGE;
    s.par = o.par;
    return s;
  };
  auto issue_one = [&](const Src& s, int d) {
    if (d < NDA) s3::dma_b128(s.a + s3map::dma_off(d, offA[0], offA[1], stepA), s.st + (d * 4 + wave) * 1024);
    else if (d < NDA + NDB)
      s3::dma_b128(s.b + s3map::dma_off(d - NDA, offB[0], offB[1], stepB), s.st + A_BYTES + ((d - NDA) * 4 + wave) * 1024);
    else if (d == NDA + NDB) s3::dma_b32(s.bias + tid * 4, lds + OFF_BIAS + s.par * 1024 + wave * 256);
    else s3::dma_b32(s.coef + tid * 4, lds + OFF_COEF + s.par * 1024 + wave * 256);
  };
  auto read_frag = [&](int f, const char* st, int ss, bf16x8* a, bf16x8* b) {
    const uint32_t c0 = (uint32_t)((((2 * ss + g) ^ s0) << 4));
    if (f < WM) {
      const uint32_t o = rbA + (c0 ^ (uint32_t)(64 * (f & 1)));
      a[f] = *reinterpret_cast<const bf16x8*>(st + o + 4096 * f);
    } else {
      const int fb = f - WM;
      const uint32_t o = rbB + (c0 ^ (uint32_t)(64 * (fb & 1)));
      b[fb] = *reinterpret_cast<const bf16x8*>(st + o + 4096 * fb);
    }
  };

  // fp8 fragment f of k-step ks (0, 1) of a stage: the 16-byte pieces of the
  // bf16 k-steps 2 ks and 2 ks + 1, i.e. chunks (4 ks + g) ^ s0 and
  // (4 ks + 2 + g) ^ s0 of the row, with bit 2 of the chunk flipped for odd
  // f. Rows start at multiples of 128 bytes, so every piece's offset is the
  // lane's base rb + ((g ^ s0) << 4) XOR a constant below 128. The base
  // passes through an empty asm at each read so the compiler forms the XOR
  // there instead of keeping all sixteen offsets live (which spilled).
  const uint32_t baseA8 = rbA + (uint32_t)((g ^ s0) << 4), baseB8 = rbB + (uint32_t)((g ^ s0) << 4);
  auto read_frag8 = [&](int f, const char* st, int ks, i32x8* a, i32x8* b) {
    const int ff = f < WM ? f : f - WM;
    uint32_t base = f < WM ? baseA8 : baseB8;
    asm volatile("" : "+v"(base));
    const uint32_t k0 = (uint32_t)(64 * ks) ^ (uint32_t)(64 * (ff & 1));
    i32x8* dst = f < WM ? &a[ff] : &b[ff];
    reinterpret_cast<u32x4*>(dst)[0] = *reinterpret_cast<const u32x4*>(st + (base ^ k0) + 4096 * ff);
    reinterpret_cast<u32x4*>(dst)[1] = *reinterpret_cast<const u32x4*>(st + (base ^ k0 ^ 32u) + 4096 * ff);
  };

  f32x16 acc[2][WM][WN];
  bf16x8 af[2][WM], bfr[2][WN];
  i32x8 af8[WM], bf8[WN];

  // ---------------------------------------------------------------- epilogue state
  // The item being finalized: its cell tile, V tile and parity (LDS buffers).
  int e_ct = 0, e_vt = 0, e_par = 0;
  bool e_live = false;
  // forward: running (max, sum) per column block j; backward: (lse log2 e,
  // occupancy) per column block
  float em[2], es[2];
  float y[16];
  float ebm = 0.0f;
  f32x4 bq[4];
  float* stats2 = reinterpret_cast<float*>(p.stats);
  bf16* dh = reinterpret_cast<bf16*>(p.dh);
  bf16* lg = reinterpret_cast<bf16*>(p.logits);  // 2-byte pieces moved as they are (fp16 values)
  char* const dhs = lds + OFF_DHS + wave * DHS_WAVE;  // block staging (backward dh, stored scores)
  bf16x8 fl[2];

  // One chunk (issued after one MFMA) of epilogue task T on accumulator set E.
  auto epi_chunk = [&](auto EE, auto TT, auto XX) __attribute__((always_inline)) {
    constexpr int E = decltype(EE)::value;
    constexpr int T = decltype(TT)::value;
    constexpr int X = decltype(XX)::value;
    const float* bias = reinterpret_cast<const float*>(lds + OFF_BIAS + e_par * 1024);
    if constexpr (!BWD) {
      if constexpr (T < 16) {
        constexpr int b = T >> 1, i = b >> 1, j = b & 1;
        if constexpr ((T & 1) == 0) {
          // task A(b): scaled scores of block (i, j) and their max
          if constexpr (X == 0) {
            if constexpr (j == 0) {
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4)
                bq[q4] = *reinterpret_cast<const f32x4*>(bias + wr * 128 + i * 32 + 8 * q4 + 4 * g);
            }
            if constexpr (b < 2) {
              em[j] = -1e30f;
              es[j] = 0.0f;
            }
            ebm = em[j];
          }
#pragma unroll
          for (int e = 2 * X; e < 2 * X + 2; ++e) {
            y[e] = __builtin_fmaf(acc[E][i][j][e], ysc, bq[e >> 2][e & 3]);
            ebm = __builtin_fmaxf(ebm, y[e]);
          }
          if constexpr (STORE && (X & 1) == 1) {
            // products 8 (e4 / 4) + 4 g .. +3 of the block for cell r, scaled
            // to log2 units without the bias (y minus it: the bias can be far
            // larger, and the backward adds it back in fp32), as fp16 (clamped
            // to its range), into the staging buffer. The store path's per-lane
            // offsets are formed from the lane index at each use (laundered
            // through an empty asm) rather than kept live across the loop,
            // where the registers are needed by the pipeline.
            constexpr int e4 = 2 * X - 2;
            f16x4 w;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              w[q] = (f16)__builtin_amdgcn_fmed3f(y[e4 + q] - bq[(e4 + q) >> 2][(e4 + q) & 3], -kF16Max, kF16Max);
            int ln = lane;
            asm volatile("" : "+v"(ln));
            *reinterpret_cast<f16x4*>(dhs + (ln & 31) * DHS_ROW + (8 * (e4 >> 2) + 4 * (ln >> 5)) * 2) = w;
          }
        } else {
          // task B(b): fold 2^(y - max) into the running sum
          if constexpr (X == 0) es[j] *= fexp2(em[j] - ebm);
          es[j] += fexp2(y[2 * X] - ebm) + fexp2(y[2 * X + 1] - ebm);
          if constexpr (X == 7) em[j] = ebm;
          if constexpr (STORE && X < 4) {
            // block b, staged in task A(b), leaves the staging buffer (cells
            // 16 h + lane / 4, scores 8 (lane % 4) .. +7, h = X / 2) before
            // block b + 1 is written there in task A(b + 1); one piece is read
            // per even chunk and stored in the next; rows past the wave are not stored
            constexpr int h = X >> 1;
            int ln = lane;
            asm volatile("" : "+v"(ln));
            if constexpr ((X & 1) == 0) {
              fl[0] = *reinterpret_cast<const bf16x8*>(dhs + (16 * h + (ln >> 2)) * DHS_ROW + (ln & 3) * 16);
            } else {
              const int rr = e_ct * BN + wc * 64 + j * 32 + 16 * h + (ln >> 2);
              const int v = e_vt * 256 + wr * 128 + i * 32 + 8 * (ln & 3);
              if (e_live && rr < p.n_rows) *reinterpret_cast<bf16x8*>(lg + (int64_t)rr * p.V_pad + v) = fl[0];
            }
          }
        }
      } else if constexpr (T == 16 && X == 0) {
        // combine the two half-waves (same cells, other score rows); wave row 1 -> LDS
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float m2 = __shfl_xor(em[j], 32), s2 = __shfl_xor(es[j], 32);
          const float mn = __builtin_fmaxf(em[j], m2);
          es[j] = es[j] * fexp2(em[j] - mn) + s2 * fexp2(m2 - mn);
          em[j] = mn;
        }
        float* red = reinterpret_cast<float*>(lds + OFF_RED);
        int ln = lane;
        if constexpr (STORE) asm volatile("" : "+v"(ln));  // formed here, not kept live (see the store path)
        if (wr == 1 && ln < 32) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            red[((wc * 2 + j) * 2 + 0) * 32 + ln] = em[j];
            red[((wc * 2 + j) * 2 + 1) * 32 + ln] = es[j];
          }
        }
      } else if constexpr (T == 19 && X == 0) {
        // after the stage barrier: wave row 0 merges and stores (max ln 2, sum)
        const float* red = reinterpret_cast<const float*>(lds + OFF_RED);
        int ln = lane;
        if constexpr (STORE) asm volatile("" : "+v"(ln));  // formed here, not kept live (see the store path)
        if (wr == 0 && ln < 32 && e_live) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const float m2 = red[((wc * 2 + j) * 2 + 0) * 32 + ln];
            const float s2 = red[((wc * 2 + j) * 2 + 1) * 32 + ln];
            const float mn = __builtin_fmaxf(em[j], m2);
            const float sv = es[j] * fexp2(em[j] - mn) + s2 * fexp2(m2 - mn);
            const int64_t rr = (int64_t)e_ct * BN + wc * 64 + j * 32 + ln;
            *reinterpret_cast<f32x2*>(stats2 + 2 * (rr * nvt + e_vt)) = f32x2{mn * kLn2, sv};
          }
        }
      }
    } else {
      // task T = 2 b + 3 (b = 0 .. 7), chunks 0 - 3: block b, finished in task
      // T - 1, leaves the staging buffer (cells 16 h + lane / 4, scores
      // 8 (lane % 4) .. +7 of the block) before block b + 1 is first written
      // there in chunk 3; the wave's LDS accesses complete in order
      if constexpr (T >= 3 && T <= 17 && (T & 1) == 1 && X < 4) {
        constexpr int pb = (T - 3) >> 1, pi = pb >> 1, pj = pb & 1;
        if constexpr (X < 2) {
          fl[X] = *reinterpret_cast<const bf16x8*>(dhs + (16 * X + (lane >> 2)) * DHS_ROW + (lane & 3) * 16);
        } else if (e_live) {
          constexpr int h = X - 2;
          const int64_t rr = (int64_t)e_ct * BN + wc * 64 + pj * 32 + 16 * h + (lane >> 2);
          const int v = e_vt * 256 + wr * 128 + pi * 32 + 8 * (lane & 3);
          *reinterpret_cast<bf16x8*>(dh + rr * p.V_pad + v) = fl[h];
        }
      }
      if constexpr (T == 0 && X == 0) {
        const float* cf = reinterpret_cast<const float*>(lds + OFF_COEF + e_par * 1024);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const f32x2 c = *reinterpret_cast<const f32x2*>(cf + 2 * (wc * 64 + j * 32 + r));
          em[j] = c[0];
          es[j] = c[1];
        }
      } else if constexpr (T >= 1 && T < 17) {
        // block b = (T-1)/2, half hh: elements 8 hh + X; dh = co 2^(y - lse log2 e)
        constexpr int b = (T - 1) >> 1, hh = (T - 1) & 1, i = b >> 1, j = b & 1;
        if constexpr (X == 0 && hh == 0 && j == 0) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            bq[q4] = *reinterpret_cast<const f32x4*>(bias + wr * 128 + i * 32 + 8 * q4 + 4 * g);
        }
        constexpr int e = 8 * hh + X;
        y[e] = es[j] * fexp2(__builtin_fmaf(acc[E][i][j][e], ysc, bq[e >> 2][e & 3]) - em[j]);
        if constexpr (X == 3 || X == 7) {
          // scores 8 (e4 / 4) + 4 g .. +3 of the block for cell r, into the staging buffer
          constexpr int e4 = e - 3;
          bf16x4 w;
#pragma unroll
          for (int q = 0; q < 4; ++q) w[q] = (bf16)y[e4 + q];
          *reinterpret_cast<bf16x4*>(dhs + r * DHS_ROW + (8 * (e4 >> 2) + 4 * g) * 2) = w;
        }
      }
    }
  };

  // One k-step: MFMAs on register buffer CB into accumulator set C (ZERO:
  // first k-step of an item), fragments of (rd_st, rd_ss) into buffer CB^1,
  // optionally the dma of stage dma_s, and epilogue task T on set C^1
  // (T < 0: none).
  auto kstep = [&](auto CB, auto CC, auto ZERO, auto TT, const char* rd_st, int rd_ss, bool dma,
                   int dma_s) __attribute__((always_inline)) {
    constexpr int cb = decltype(CB)::value;
    constexpr int C = decltype(CC)::value;
    constexpr bool zero = decltype(ZERO)::value;
    constexpr int T = decltype(TT)::value;
    Src ds{};
    if (dma) ds = stage_src(dma_s);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < WM * WN; ++x) {
      const int i = x / WN, j = x % WN;
      acc[C][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cb][i], bfr[cb][j],
                                                             zero ? f32x16{} : acc[C][i][j], 0, 0, 0);
      if (x < WM + WN) read_frag(x, rd_st, rd_ss, af[cb ^ 1], bfr[cb ^ 1]);
      if (dma) {
#pragma unroll
        for (int d = 0; d < ND; ++d)
          if (d * 8 / ND == x) issue_one(ds, d);
      }
      if constexpr (T >= 0) {
        using Cx = std::integral_constant<int, C ^ 1>;
        using Tx = std::integral_constant<int, T>;
        if (x == 0) epi_chunk(Cx{}, Tx{}, std::integral_constant<int, 0>{});
        if (x == 1) epi_chunk(Cx{}, Tx{}, std::integral_constant<int, 1>{});
        if (x == 2) epi_chunk(Cx{}, Tx{}, std::integral_constant<int, 2>{});
        if (x == 3) epi_chunk(Cx{}, Tx{}, std::integral_constant<int, 3>{});
        if (x == 4) epi_chunk(Cx{}, Tx{}, std::integral_constant<int, 4>{});
        if (x == 5) epi_chunk(Cx{}, Tx{}, std::integral_constant<int, 5>{});
        if (x == 6) epi_chunk(Cx{}, Tx{}, std::integral_constant<int, 6>{});
        if (x == 7) epi_chunk(Cx{}, Tx{}, std::integral_constant<int, 7>{});
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // fp8 k-step (64 k): 8 MFMAs 32 x 32 x 64 into set C, column block j
  // outer, so fragment B0 is free after MFMA 3 and A_i after MFMA 4 + i; each
  // is then re-read for (rd_st, rd_ks). Epilogue tasks T (chunks after MFMAs
  // 0-3, two each) and T + 1 (after 4-7) on set C^1, in order.
  auto kstep8 = [&](auto CC, auto ZERO, auto TT, const char* rd_st, int rd_ks, bool dma,
                    int dma_s) __attribute__((always_inline)) {
    constexpr int C = decltype(CC)::value;
    constexpr bool zero = decltype(ZERO)::value;
    constexpr int T = decltype(TT)::value;
    Src ds{};
    if (dma) ds = stage_src(dma_s);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < WM * WN; ++x) {
      const int i = x % WM, j = x / WM;
      acc[C][i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af8[i], bf8[j], zero ? f32x16{} : acc[C][i][j],
                                                                    0, 0, 0, 0, 0, 0);
      if (x == WM - 1) read_frag8(WM, rd_st, rd_ks, af8, bf8);       // B0
      if (x >= WM) read_frag8(x - WM, rd_st, rd_ks, af8, bf8);       // A_i
      if (x == 2 * WM - 1) read_frag8(WM + 1, rd_st, rd_ks, af8, bf8);  // B1
      if (dma) {
#pragma unroll
        for (int d = 0; d < ND; ++d)
          if (d * 8 / ND == x) issue_one(ds, d);
      }
      if constexpr (T >= 0) {
        using Cx = std::integral_constant<int, C ^ 1>;
        using Ta = std::integral_constant<int, T>;
        using Tb = std::integral_constant<int, T + 1>;
        if (x == 0) { epi_chunk(Cx{}, Ta{}, std::integral_constant<int, 0>{}); epi_chunk(Cx{}, Ta{}, std::integral_constant<int, 1>{}); }
        if (x == 1) { epi_chunk(Cx{}, Ta{}, std::integral_constant<int, 2>{}); epi_chunk(Cx{}, Ta{}, std::integral_constant<int, 3>{}); }
        if (x == 2) { epi_chunk(Cx{}, Ta{}, std::integral_constant<int, 4>{}); epi_chunk(Cx{}, Ta{}, std::integral_constant<int, 5>{}); }
        if (x == 3) { epi_chunk(Cx{}, Ta{}, std::integral_constant<int, 6>{}); epi_chunk(Cx{}, Ta{}, std::integral_constant<int, 7>{}); }
        if (x == 4) { epi_chunk(Cx{}, Tb{}, std::integral_constant<int, 0>{}); epi_chunk(Cx{}, Tb{}, std::integral_constant<int, 1>{}); }
        if (x == 5) { epi_chunk(Cx{}, Tb{}, std::integral_constant<int, 2>{}); epi_chunk(Cx{}, Tb{}, std::integral_constant<int, 3>{}); }
        if (x == 6) { epi_chunk(Cx{}, Tb{}, std::integral_constant<int, 4>{}); epi_chunk(Cx{}, Tb{}, std::integral_constant<int, 5>{}); }
        if (x == 7) { epi_chunk(Cx{}, Tb{}, std::integral_constant<int, 6>{}); epi_chunk(Cx{}, Tb{}, std::integral_constant<int, 7>{}); }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using F = std::integral_constant<bool, false>;
  using NoT = std::integral_constant<int, -1>;

  // prologue: stages 0 and 1 in flight, stage 0 landed, its first fragments,
  // stage 2 in flight
  {
    const Src s0 = stage_src(0), s1 = stage_src(1);
#pragma unroll
    for (int d = 0; d < ND; ++d) issue_one(s0, d);
#pragma unroll
    for (int d = 0; d < ND; ++d) issue_one(s1, d);
    wait_vm<ND>();
    lds_barrier();
#pragma unroll
    for (int f = 0; f < WM + WN; ++f) {
      if constexpr (FP8) read_frag8(f, lds, 0, af8, bf8);
      else read_frag(f, lds, 0, af[0], bfr[0]);
    }
    const Src s2 = stage_src(2);
#pragma unroll
    for (int d = 0; d < ND; ++d) issue_one(s2, d);
  }

  // stage S of the current item; the epilogue of the previous item runs in
  // stages q < EPI_STAGES (task 4q + k-step)
  auto stage = [&](auto CC, auto QQ, int S) __attribute__((always_inline)) {
    constexpr int C = decltype(CC)::value;
    constexpr int Q = decltype(QQ)::value;  // < 0: a stage without epilogue work
    const char* cur = lds + (S % NST) * STAGE;
    if constexpr (FP8) {
      // two k-steps of 64: tasks 4Q, 4Q+1 before the hand-over, 4Q+2, 4Q+3 after
      using Z = std::integral_constant<bool, Q == 0>;
      using T0 = std::integral_constant<int, Q >= 0 ? 4 * Q : -1>;
      using T2 = std::integral_constant<int, Q >= 0 ? 4 * Q + 2 : -1>;
      kstep8(CC, Z{}, T0{}, cur, 1, false, 0);
      wait_vm<ND>();  // stage S+1 landed; stage S+2 may be in flight
      lds_barrier();  // every wave is done with slot S
      kstep8(CC, F{}, T2{}, lds + ((S + 1) % NST) * STAGE, 0, true, S + 3);
    } else if constexpr (Q >= 0) {
      using Z = std::integral_constant<bool, Q == 0>;
      kstep(C0{}, CC, Z{}, std::integral_constant<int, 4 * Q + 0>{}, cur, 1, false, 0);
      kstep(C1{}, CC, F{}, std::integral_constant<int, 4 * Q + 1>{}, cur, 2, false, 0);
      kstep(C0{}, CC, F{}, std::integral_constant<int, 4 * Q + 2>{}, cur, 3, false, 0);
      wait_vm<ND>();  // stage S+1 landed; stage S+2 may be in flight
      lds_barrier();  // every wave is done with slot S
      kstep(C1{}, CC, F{}, std::integral_constant<int, 4 * Q + 3>{}, lds + ((S + 1) % NST) * STAGE, 0, true, S + 3);
    } else {
      kstep(C0{}, CC, F{}, NoT{}, cur, 1, false, 0);
      kstep(C1{}, CC, F{}, NoT{}, cur, 2, false, 0);
      kstep(C0{}, CC, F{}, NoT{}, cur, 3, false, 0);
      wait_vm<ND>();
      lds_barrier();
      kstep(C1{}, CC, F{}, NoT{}, lds + ((S + 1) % NST) * STAGE, 0, true, S + 3);
    }
  };
  auto item = [&](auto CC, int n) __attribute__((always_inline)) {
    const int S0 = n * nq;
    stage(CC, std::integral_constant<int, 0>{}, S0 + 0);
    stage(CC, std::integral_constant<int, 1>{}, S0 + 1);
    stage(CC, std::integral_constant<int, 2>{}, S0 + 2);
    stage(CC, std::integral_constant<int, 3>{}, S0 + 3);
    stage(CC, std::integral_constant<int, 4>{}, S0 + 4);
    for (int q = EPI_STAGES; q < nq; ++q) stage(CC, NoT{}, S0 + q);
    // this item is the one finalized during the next
    e_live = true;
    item_of(n, e_ct, e_vt);
    e_par = n % NBUF;
  };

  for (int n = 0; n < n_items; n += 2) {
    item(C0{}, n);
    if (n + 1 < n_items) item(C1{}, n + 1);
  }
  // the last item's epilogue, with no MFMAs to hide it under
  auto drain = [&](auto EE) __attribute__((always_inline)) {
#define RNNT_E3(T)                                                                                      \
  epi_chunk(EE, std::integral_constant<int, T>{}, std::integral_constant<int, 0>{});                 \
  epi_chunk(EE, std::integral_constant<int, T>{}, std::integral_constant<int, 1>{});                 \
  epi_chunk(EE, std::integral_constant<int, T>{}, std::integral_constant<int, 2>{});                 \
  epi_chunk(EE, std::integral_constant<int, T>{}, std::integral_constant<int, 3>{});                 \
  epi_chunk(EE, std::integral_constant<int, T>{}, std::integral_constant<int, 4>{});                 \
  epi_chunk(EE, std::integral_constant<int, T>{}, std::integral_constant<int, 5>{});                 \
  epi_chunk(EE, std::integral_constant<int, T>{}, std::integral_constant<int, 6>{});                 \
  epi_chunk(EE, std::integral_constant<int, T>{}, std::integral_constant<int, 7>{});
    RNNT_E3(0) RNNT_E3(1) RNNT_E3(2) RNNT_E3(3) RNNT_E3(4) RNNT_E3(5) RNNT_E3(6) RNNT_E3(7)
    RNNT_E3(8) RNNT_E3(9) RNNT_E3(10) RNNT_E3(11) RNNT_E3(12) RNNT_E3(13) RNNT_E3(14) RNNT_E3(15)
    RNNT_E3(16) RNNT_E3(17) RNNT_E3(18)
    lds_barrier();
    RNNT_E3(19)
#undef RNNT_E3
  };
  if (n_items & 1) drain(C0{});
  else drain(C1{});
  wait_vm<0>();  // dma past the end must land before the workgroup's LDS is released
}

hipError_t launch_scores3(const Scores3Args& a, bool bwd, hipStream_t st) {
  if (a.n_ct == 0) return hipSuccess;
  dim3 grid(256), block(256);
  const bool fp8 = a.WO8 != nullptr;
  // at least EPI_STAGES stages per item; fp8 rows are whole stages of 128 bytes
  if (fp8 ? (a.H8 % 128 != 0 || a.H8 / 128 < s3::EPI_STAGES || a.z8_ld % 128 != 0 || !a.z8 || !a.ew)
          : (a.H_pad % 64 != 0 || a.H_pad / 64 < 8))
    return hipErrorInvalidValue;
  if (a.logits && (bwd || fp8)) return hipErrorInvalidValue;  // only the bf16 forward stores the scores
  if (fp8) {
    if (bwd) hipLaunchKernelGGL((scores3_kernel<true, true, false>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((scores3_kernel<false, true, false>), grid, block, 0, st, a);
  } else if (bwd) {
    hipLaunchKernelGGL((scores3_kernel<true, false, false>), grid, block, 0, st, a);
  } else if (a.logits) {
    hipLaunchKernelGGL((scores3_kernel<false, false, true>), grid, block, 0, st, a);
  } else {
    hipLaunchKernelGGL((scores3_kernel<false, false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

// ============================================================================ helpers
// Zero-padded copy of W^O: [nvt*256][H_pad], 0 for v >= V or k >= H.
__global__ void pad_wo_kernel(const bf16* __restrict__ WO, bf16* __restrict__ WOp, int V, int H, int H_pad,
                              int rows) {
  const int64_t n = (int64_t)rows * H_pad;
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < n; x += (int64_t)gridDim.x * blockDim.x) {
    const int v = (int)(x / H_pad), k = (int)(x - (int64_t)v * H_pad);
    WOp[x] = (v < V && k < H) ? WO[(int64_t)v * H + k] : (bf16)0.0f;
  }
}
// bl[v] = b^O[v] log2 e for v < V, -1e30 up to nvt*256 (those rows drop out of
// the max and the sum)
__global__ void bias_table_kernel(const bf16* __restrict__ bO, float* __restrict__ bl, int V, int rows) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v < rows) bl[v] = v < V ? (float)bO[v] * kLog2e : -1e30f;
}

hipError_t launch_bias_table(const void* bO, float* bl, int V, int nvt, hipStream_t st) {
  const int rows = nvt * 256;
  hipLaunchKernelGGL(bias_table_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, reinterpret_cast<const bf16*>(bO),
                     bl, V, rows);
  return hipGetLastError();
}

hipError_t launch_score_tables(const void* WO, const void* bO, void* WOp, float* bl, int V, int H, int H_pad,
                               int nvt, hipStream_t st) {
  const int rows = nvt * 256;
  hipLaunchKernelGGL(pad_wo_kernel, dim3(512), dim3(256), 0, st, reinterpret_cast<const bf16*>(WO),
                     reinterpret_cast<bf16*>(WOp), V, H, H_pad, rows);
  hipLaunchKernelGGL(bias_table_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, reinterpret_cast<const bf16*>(bO),
                     bl, V, rows);
  return hipGetLastError();
}

// fp8 output layer: the scale exponent of W^O, one workgroup. |x| of a bf16
// orders like its bits with the sign cleared, so the largest magnitude is the
// largest such bit pattern (NaN and infinity are clamped to the largest
// finite value). e is the largest integer with amax 2^e <= 448 = 0.875 2^9:
// with amax = m 2^x, m in [0.5, 1), e = 9 - x if m <= 0.875, else 8 - x.
__global__ void __launch_bounds__(1024) wo_scale_kernel(const u32x4* __restrict__ WO, int64_t n16, int* ew) {
  __shared__ uint32_t red[16];
  uint32_t m = 0;
  for (int64_t i = threadIdx.x; i < n16; i += 1024) {
    const u32x4 v = WO[i];
#pragma unroll
    for (int q = 0; q < 4; ++q) m = max(m, max(v[q] & 0x7fffu, (v[q] >> 16) & 0x7fffu));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int i = 0; i < 16; ++i) a = max(a, red[i]);
    a = min(a, 0x7f7fu);
    int e = 0;
    if (a != 0) {
      int x = 0;
      const float mnt = __builtin_frexpf(__uint_as_float(a << 16), &x);
      e = mnt <= 0.875f ? 9 - x : 8 - x;
    }
    *ew = e;
  }
}

// WO8[v][k] = E4M3(W^O[v][k] 2^e) for v < V, k < H (the product is exact in
// fp32), 0 elsewhere up to [nvt*256][H8]; four bytes per thread.
__global__ void pad_wo8_kernel(const bf16* __restrict__ WO, uint32_t* __restrict__ WO8, const int* __restrict__ ew,
                               int V, int H, int H8, int rows) {
  const int e = *ew;
  const int q4 = H8 / 4;
  const int64_t n = (int64_t)rows * q4;
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < n; x += (int64_t)gridDim.x * blockDim.x) {
    const int v = (int)(x / q4), k = 4 * (int)(x - (int64_t)v * q4);
    uint32_t w = 0;
    if (v < V && k < H) {  // H % 4 == 0: the four values are all inside or all outside
      const bf16* src = WO + (int64_t)v * H + k;
      int r = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf((float)src[0], e), __builtin_ldexpf((float)src[1], e),
                                              0, false);
      r = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf((float)src[2], e), __builtin_ldexpf((float)src[3], e), r,
                                          true);
      w = (uint32_t)r;
    }
    WO8[x] = w;
  }
}

hipError_t launch_score_tables8(const void* WO, const void* bO, void* WO8, float* bl, int* ew, int V, int H, int H8,
                                int nvt, hipStream_t st) {
  const int rows = nvt * 256;
  if (H % 8 != 0 || H8 % 4 != 0 || H8 < H) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wo_scale_kernel, dim3(1), dim3(1024), 0, st, reinterpret_cast<const u32x4*>(WO),
                     (int64_t)V * H / 8, ew);
  hipLaunchKernelGGL(pad_wo8_kernel, dim3(512), dim3(256), 0, st, reinterpret_cast<const bf16*>(WO),
                     reinterpret_cast<uint32_t*>(WO8), ew, V, H, H8, rows);
  hipLaunchKernelGGL(bias_table_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, reinterpret_cast<const bf16*>(bO),
                     bl, V, rows);
  return hipGetLastError();
}

// Per buffer row (cell) of a wave, the backward coefficients of Eq. (10):
// coefA = (lse log2 e, g alpha beta / P), coefB = (g alpha phi beta' / P,
// g alpha psi beta'' / P, label, 0); zeros (label -1) on padding rows.
// One workgroup per 32 t x 32 u block of a tile: the lattice values are read
// group of four diagonals by group in (row, diagonal) order (each wave reads
// the 16-byte pieces of consecutive rows) into LDS, beta with one more t and
// u for the neighbours, and the coefficients are written in row order. The workgroup past the last tile clears the
// rows between the wave's last row and the 128-row padding.
constexpr int kCB = 32, kCS = 34;  // block edge, LDS row stride (conflict-free both ways)
__global__ void __launch_bounds__(256) coef_kernel(Scores3Args p) {
  __shared__ float sm[4][kCB * kCS];        // alpha, phi, psi, lse at [u][t]
  __shared__ float sb[(kCB + 1) * kCS];     // beta at [u][t], u, t <= 32
  f32x2* coefA = reinterpret_cast<f32x2*>(p.coefA);
  f32x4* coefB = reinterpret_cast<f32x4*>(p.coefB);
  if ((int)blockIdx.x == p.tile_end - p.tile_begin) {
    if (blockIdx.y == 0 && blockIdx.z == 0)
      for (int rr = p.n_rows + threadIdx.x; rr < p.n_ct * s3::BN; rr += 256) {
        coefA[rr] = f32x2{kPosInf, 0.0f};
        coefB[rr] = f32x4{0.0f, 0.0f, -1.0f, 0.0f};
      }
    return;
  }
  const Tile tl = p.tiles[p.tile_begin + blockIdx.x];
  const int tb = blockIdx.y * kCB, ub = blockIdx.z * kCB;
  if (tb >= tl.ht || ub >= tl.wu) return;
  const int nt = min(kCB, tl.ht - tb), nu = min(kCB, tl.wu - ub);
  const int b = tl.b, Tb = p.T_len[b], Ub = p.U_len[b];
  const int t0 = tl.t0 + tb, u0 = tl.u0 + ub;
  const LatGeo geo = lat_geo(p.lat_off, p.U_len, b);
  // lattice -> LDS for the (33 x 33) region, whose diagonals t0 + u0 ..
  // t0 + u0 + 64 lie in 17 groups from q0 on; all loads of the thread are
  // issued before any is stored (masked slots read entry 0)
  constexpr int kRows = kCB + 1, kGroups = (2 * kCB + 3) / 4 + 1;
  constexpr int kSlots = kGroups * kRows * 4, kIt = (kSlots + 255) / 256;
  const int q0 = (t0 + u0) >> 2;
  auto slot_of = [&](int i, int& ul, int& tt) {
    const int e = i & 3, gq = (i >> 2) / kRows;
    ul = (i >> 2) - gq * kRows;
    tt = 4 * (q0 + gq) + e - t0 - u0 - ul;
  };
  float va[kIt], vb[kIt], vp[kIt], vs[kIt], vl[kIt];
#pragma unroll
  for (int q = 0; q < kIt; ++q) {
    const int i = threadIdx.x + 256 * q;
    int ul, tt;
    slot_of(i, ul, tt);
    const bool okb = i < kSlots && tt >= 0 && tt <= kCB && t0 + tt < Tb && u0 + ul <= Ub;
    const bool oka = okb && tt < nt && ul < nu;
    const size_t idx = okb ? (size_t)lat_at(geo, t0 + tt, u0 + ul) : 0;
    const size_t ia = oka ? idx : 0;
    vb[q] = p.beta[idx];
    va[q] = p.alpha[ia];
    vp[q] = p.phi[ia];
    vs[q] = p.psi[ia];
    vl[q] = p.lse[ia];
  }
#pragma unroll
  for (int q = 0; q < kIt; ++q) {
    const int i = threadIdx.x + 256 * q;
    int ul, tt;
    slot_of(i, ul, tt);
    const bool okb = i < kSlots && tt >= 0 && tt <= kCB && t0 + tt < Tb && u0 + ul <= Ub;
    if (!okb) continue;
    sb[ul * kCS + tt] = vb[q];
    if (tt < nt && ul < nu) {
      sm[0][ul * kCS + tt] = va[q];
      sm[1][ul * kCS + tt] = vp[q];
      sm[2][ul * kCS + tt] = vs[q];
      sm[3][ul * kCS + tt] = vl[q];
    }
  }
  __syncthreads();
  const float lp = p.lnP[b];
  const float gb = p.dcosts ? p.dcosts[b] : 1.0f;
#pragma unroll
  for (int i = threadIdx.x; i < kCB * kCB; i += 256) {
    const int ul = i / kCB, tt = i % kCB;
    if (ul >= nu) continue;
    const int rr = tl.row0 + (ub + ul) * tl.htp + tb + tt - p.buf_row_base;
    // rows past ht (up to htp) are padding: lse = +inf makes the exponent of
    // every score -inf there, so their dh is exactly 0 however large the
    // score (0 x inf would be NaN)
    float ls = kPosInf, co = 0.0f, cb = 0.0f, cl = 0.0f, lab = -1.0f;
    if (tt < nt) {
      const int t = t0 + tt, u = u0 + ul;
      const float A = sm[0][ul * kCS + tt], Bt = sb[ul * kCS + tt];
      ls = sm[3][ul * kCS + tt];
      const float bn = (t + 1 < Tb) ? sb[ul * kCS + tt + 1] : (u == Ub ? 0.0f : kNegInf);
      co = gb * fexp2((A + Bt - lp) * kLog2e);
      cb = gb * fexp2((A + sm[1][ul * kCS + tt] + bn - lp) * kLog2e);
      if (u < Ub) {
        cl = gb * fexp2((A + sm[2][ul * kCS + tt] + sb[(ul + 1) * kCS + tt] - lp) * kLog2e);
        lab = (float)p.labels[(size_t)b * p.U1 + u + 1];
      }
    }
    coefA[rr] = f32x2{ls * kLog2e, co};
    coefB[rr] = f32x4{cb, cl, lab, 0.0f};
  }
}

// dh[row, blank] -= cb, dh[row, label] -= cl (in fp32, rounded once more to bf16)
__global__ void dh_fix_kernel(Scores3Args p) {
  const int rr = blockIdx.x * blockDim.x + threadIdx.x;
  if (rr >= p.n_rows) return;
  const f32x4 c = reinterpret_cast<const f32x4*>(p.coefB)[rr];
  bf16* row = reinterpret_cast<bf16*>(p.dh) + (int64_t)rr * p.V_pad;
  if (c[0] != 0.0f) row[p.blank] = (bf16)((float)row[p.blank] - c[0]);
  const int lab = (int)c[2];
  if (lab >= 0 && c[1] != 0.0f) row[lab] = (bf16)((float)row[lab] - c[1]);
}

hipError_t launch_coef(const Scores3Args& a, int tile_t, int tile_u, hipStream_t st) {
  if (a.n_ct == 0) return hipSuccess;
  const dim3 grid(a.tile_end - a.tile_begin + 1, (tile_t + kCB - 1) / kCB, (tile_u + kCB - 1) / kCB);
  hipLaunchKernelGGL(coef_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_dh_fix(const Scores3Args& a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(dh_fix_kernel, dim3((a.n_rows + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Untiled mode: dh from the products the forward kept ((W^O z) log2 e as
// fp16, rows of V_pad), written in place as bf16 (Eq. (10)): with
// y = product + b^O log2 e (in fp32), dh = occ 2^(y - lse log2 e), minus the
// blank and label terms of the row's coefficients. Eight consecutive scores
// (16 bytes) per thread, their b^O log2 e from the bias table (two 16-byte
// loads); past V the table holds -1e30, so dh is 0.
__global__ void __launch_bounds__(256) dh_logits_kernel(Scores3Args p) {
  const int per_row = p.V_pad / 8;
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= (int64_t)p.n_rows * per_row) return;
  const int rr = (int)(x / per_row);
  const int v0 = (int)(x - (int64_t)rr * per_row) * 8;
  const f32x2 ca = reinterpret_cast<const f32x2*>(p.coefA)[rr];
  const f32x4 cb = reinterpret_cast<const f32x4*>(p.coefB)[rr];
  const int lab = (int)cb[2];
  // b^O log2 e, and -1e30 past V (2^(w - 1e30 - lse) is exactly 0 there)
  const f32x4 bl0 = reinterpret_cast<const f32x4*>(p.bl + v0)[0];
  const f32x4 bl1 = reinterpret_cast<const f32x4*>(p.bl + v0)[1];
  char* row = reinterpret_cast<char*>(p.logits) + ((int64_t)rr * p.V_pad + v0) * 2;
  const f16x8 w = *reinterpret_cast<const f16x8*>(row);
  bf16x8 out;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int v = v0 + k;
    const float yb = k < 4 ? bl0[k] : bl1[k - 4];
    float d = ca[1] * fexp2((float)w[k] + yb - ca[0]);
    if (v == p.blank) d -= cb[0];
    if (v == lab) d -= cb[1];
    out[k] = (bf16)d;
  }
  *reinterpret_cast<bf16x8*>(row) = out;
}

hipError_t launch_dh_logits(const Scores3Args& a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  if (a.V_pad % 8 != 0 || !a.logits || !a.coefA || !a.coefB || !a.bl) return hipErrorInvalidValue;
  const int64_t n = (int64_t)a.n_rows * (a.V_pad / 8);
  hipLaunchKernelGGL(dh_logits_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace rnnt
