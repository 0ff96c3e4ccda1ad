// Shared device definitions for the gfx950 RNN-T kernels: operand types,
// MFMA fragment conventions, LDS swizzle, fast transcendentals and the tile
// plan records that the host builds and the kernels read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common_host.hpp"

namespace rnnt {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();
constexpr float kF16Max = 65504.0f;

// ---------------------------------------------------------------- plan records
// A tile is a t x u block of one sample's lattice, clipped to t < T_b,
// u <= U_b. Its cells occupy rows [row0, row0 + wu*htp) of the row space,
// u-major with t fastest: row = row0 + (u-u0)*htp + (t-t0). htp is ht rounded
// up to 32; rows with t-t0 >= ht are padding (their scores/gradients are 0).
// Tiles are listed in plan order; row0 and strip0 (32-row strips along t:
// strip0 + (t-t0)/32) are prefix sums over that order.
struct Tile {
  int32_t b, t0, u0, ht, wu, htp, row0, strip0;
};

// Rows of gA (group kind A: same sample and t0) or gL (kind L: same sample
// and u0) that receive contributions from tiles idx[first .. first+count) of
// one wave. len = ht (A) or wu (L); start = t0 (A) or u0 (L).
struct Group {
  int32_t b, start, len, first, count, pad0, pad1, pad2;
};

// Sample b's block in the packed lattice arrays of `saved` (lat_off: the
// block offsets, U_len: the label counts, both in `saved`).
__device__ inline LatGeo lat_geo(const int64_t* lat_off, const int32_t* U_len, int b) {
  return lat_geo_packed(lat_off[b], U_len[b]);
}

// ---------------------------------------------------------------- MFMA conventions
// Both operand fragments are 16 bytes per lane. A lane holds row (A) or column
// (B) `lane % ROWS` of a ROWS x ROWS output block and k-elements
// [KPL*g, KPL*g + KPL) of a KSTEP-wide k slab, g = lane / ROWS. Using the same
// (g, element) -> k assignment for A and B makes each product sum over all k.
struct MfmaBf16 {  // v_mfma_f32_32x32x16_bf16
  using CT = bf16;
  static constexpr int ROWS = 32, KPL = 8, GROUPS = 2, KSTEP = 16, NACC = 16;
  using Frag = bf16x8;
  using Acc = f32x16;
  __device__ static inline Acc mma(Frag a, Frag b, Acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // output element e of `lane` is (row_of(e, lane), col_of(lane))
  __device__ static inline int row_of(int e, int lane) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }
  __device__ static inline int col_of(int lane) { return lane & 31; }
};

struct MfmaF32 {  // four v_mfma_f32_16x16x4_f32 per fragment
  using CT = float;
  static constexpr int ROWS = 16, KPL = 4, GROUPS = 4, KSTEP = 16, NACC = 4;
  using Frag = f32x4;
  using Acc = f32x4;
  __device__ static inline Acc mma(Frag a, Frag b, Acc c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
  __device__ static inline int row_of(int e, int lane) { return 4 * (lane >> 4) + e; }
  __device__ static inline int col_of(int lane) { return lane & 15; }
};

template <class CT> struct MfmaFor;
template <> struct MfmaFor<bf16> { using type = MfmaBf16; };
template <> struct MfmaFor<float> { using type = MfmaF32; };

// ---------------------------------------------------------------- LDS tiles
// An LDS operand tile is rows x 128 bytes (8 chunks of 16 bytes). Chunk c of
// row r is stored at physical chunk c ^ swz(r), which keeps both the MFMA
// fragment reads (8 consecutive rows, same chunk) and the transposing stores
// (rows 8 apart) free of bank conflicts.
__device__ inline int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ inline int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }

// ---------------------------------------------------------------- math
__device__ inline float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float flog2(float x) { return __builtin_amdgcn_logf(x); }
__device__ inline float frcp(float x) { return __builtin_amdgcn_rcpf(x); }

// tanh from one exp2 and one reciprocal: tanh|x| = (1-e)/(1+e), e = exp(-2|x|).
// Absolute error ~1e-7, far below bf16 rounding of the result.
// z = tanh(x) from s = x * kTanhArgScale (the pre-projections of the bf16
// path are stored scaled): 2 / (1 + 2^s) - 1
constexpr float kTanhArgScale = -2.0f * 1.4426950408889634f;
__device__ inline float tanh_from_scaled(float s) { return __builtin_fmaf(2.0f, frcp(1.0f + fexp2(s)), -1.0f); }
__device__ inline float tanh_fast(float x) {
  // tanh x = 2 / (1 + e^-2x) - 1; for x -> -inf, e^-2x overflows to +inf and
  // the reciprocal to 0, giving -1
  return __builtin_fmaf(2.0f, frcp(1.0f + fexp2(-2.0f * kLog2e * x)), -1.0f);
}

template <class CT> __device__ inline float joint_act(float x);
template <> __device__ inline float joint_act<bf16>(float x) { return tanh_fast(x); }
template <> __device__ inline float joint_act<float>(float x) { return tanhf(x); }

// log(exp(a) + exp(b)); -inf when both are -inf.
__device__ inline float log_add_exp(float a, float b) {
  float m = __builtin_fmaxf(a, b);
  float n = __builtin_fminf(a, b);
  float r = m + kLn2 * flog2(1.0f + fexp2((n - m) * kLog2e));
  return m == kNegInf ? kNegInf : r;
}

template <class T> __device__ inline T to_ct(float x);
template <> __device__ inline float to_ct<float>(float x) { return x; }
template <> __device__ inline bf16 to_ct<bf16>(float x) { return (bf16)x; }

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(bf16 x) { return (float)x; }

// Plain 16-byte global load/store helpers.
template <class T> __device__ inline T ldg(const void* p) { return *reinterpret_cast<const T*>(p); }

}  // namespace rnnt
