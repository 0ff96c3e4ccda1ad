// Work and address mapping of the persistent score kernels (scores3.hip),
// written as constexpr functions so that the kernel and host-side checks
// compute item and byte offsets with the same code (constexpr functions are
// callable from device code). No HIP headers: plain C++ can include this.
//
// A launch has 256 workgroups, one per CU: xcd = blockIdx % 8 (the XCD the
// hardware dispatches it to), slot = blockIdx / 8. The wave's rows form
// n_ct cell tiles of 128 rows; a work item is (cell tile ct, 256-score V
// tile vt). Cell tiles ct = 8 c + xcd belong to XCD xcd; its 32 slots walk
// items idx = slot + 32 n (n = 0, 1, ...), idx = c0 * nvt + vt, so the V
// tiles of one cell tile run on neighbouring slots of one XCD (their z rows
// shared in that XCD's L2). Cell tiles are taken from the end of the wave
// backwards (c = nctl - 1 - c0): the z rows the z-row kernel wrote last are
// still in the last-level cache when they are read first.
#pragma once

#include <stdint.h>

namespace rnnt {
namespace s3map {

constexpr int kGrid = 256;   // workgroups per launch
constexpr int kThreads = 256;
constexpr int BN = 128;      // cells per item
constexpr int BK = 64;       // k per stage
constexpr int NST = 3;       // stages in flight
constexpr int A_BYTES = 256 * BK * 2;
constexpr int B_BYTES = BN * BK * 2;
constexpr int NDA = A_BYTES / (kThreads * 16);  // 16-byte dma per thread per stage
constexpr int NDB = B_BYTES / (kThreads * 16);

constexpr int imax(int a, int b) { return a > b ? a : b; }
constexpr int imin(int a, int b) { return a < b ? a : b; }

// LDS chunk swizzle of a 128-byte operand row (same as swz in common.hpp)
constexpr int swz_row(int row) { return (row ^ (row >> 3)) & 7; }

// cell tiles of this XCD
constexpr int nctl_of(int n_ct, int xcd) { return (n_ct - xcd + 7) / 8; }
// items of workgroup (xcd, slot)
constexpr int items_of(int n_ct, int nvt, int xcd, int slot) {
  return imax(0, (nctl_of(n_ct, xcd) * nvt - slot + 31) / 32);
}

struct Item {
  int ct, vt;
};
// item n of workgroup (xcd, slot); n is clamped to the last item (the
// pipeline's dma past the end re-reads the last item's operands)
constexpr Item item_of(int n, int n_items, int nctl, int nvt, int xcd, int slot) {
  const int nn = imin(n, n_items - 1);
  const int idx = slot + 32 * nn;
  const int c0 = idx / nvt;
  return Item{(nctl - 1 - c0) * 8 + xcd, idx - c0 * nvt};
}

// Byte offsets of stage S's sources (S = n * nq + q, nq = H_pad / BK stages
// per item) from the base of each buffer: A = padded W^O rows of V tile vt,
// B = z rows of cell tile ct, the V tile's 256 bias values, the cell tile's
// 128 backward coefficient pairs. Row lengths H_pad and z_ld count 2-byte
// units: a stage moves 128 bytes of each row (64 bf16, or 128 fp8 values
// with the row lengths halved).
struct StageSrc {
  int64_t a, b, bias, coef;
  int par;  // (clamped) item index mod nbuf: which LDS bias / coefficient buffer
};
constexpr StageSrc stage_src(int S, int nq, int n_items, int nctl, int nvt, int xcd, int slot, int H_pad,
                             int64_t z_ld, int nbuf = 2) {
  const int n = S / nq, q = S - (S / nq) * nq;
  const Item it = item_of(n, n_items, nctl, nvt, xcd, slot);
  return StageSrc{((int64_t)it.vt * 256 * H_pad + q * BK) * 2, ((int64_t)it.ct * BN * z_ld + q * BK) * 2,
                  (int64_t)it.vt * 256 * 4, (int64_t)it.ct * BN * 8, imin(n, n_items - 1) % nbuf};
}

// Per-thread part of the operand dma: instruction d of an operand (d < NDA
// for A, d < NDB for B) of thread (wave, lane) moves the 16 bytes of chunk
// (lane % 8) ^ swizzle of row 64 (d / 2) + 8 (4 (d % 2) + wave) + lane / 8.
// dma_thread_off(i, ...) is the thread's offset for d % 2 = i; step32 is the
// byte offset of 32 rows.
constexpr uint32_t dma_thread_off(int i, int wave, int lane, int ld_elems) {
  const int row = (i * 4 + wave) * 8 + (lane >> 3);
  return (uint32_t)(row * ld_elems * 2 + (((lane & 7) ^ swz_row(row)) << 4));
}
constexpr int64_t dma_off(int d_in_operand, uint32_t off0, uint32_t off1, int64_t step32) {
  return (int64_t)(d_in_operand >> 1) * 2 * step32 + ((d_in_operand & 1) ? off1 : off0);
}

}  // namespace s3map
}  // namespace rnnt
