// Kernel argument records and launcher declarations (host <-> device glue).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace rnnt {

// Fused joint + output layer (forward statistics or backward dh).
struct JointArgs {
  const Tile* tiles;
  int tile_begin, tile_end;  // tiles of this launch, in plan order
  int row_begin;             // global row of tiles[tile_begin]
  int n_chunks;              // ROWS-row chunks covered by the launch
  const int32_t* T_len;
  const int32_t* U_len;
  const int32_t* labels;  // [B, U1]
  const int64_t* lat_off;  // packed lattice blocks (lat_geo)
  const int32_t* band_lo;  // pruned lattice: [B, T] band starts (null: not pruned)
  int band_S;
  int T, U1, V, H, H_pad, V_pad, blank;
  const float* a;  // [B*T, H_pad]  W^A h^A + b^Z
  const float* l;  // [B*U1, H_pad] W^L h^L
  const void* WO;  // [V, H]
  const void* bO;  // [V]
  // forward outputs, packed lattice layout
  float* lse_out;
  float* phi_out;
  float* psi_out;
  int store;           // forward: also store scores and z (untiled mode)
  void* logits_out;    // scores (forward store) or dh (backward), [rows, V_pad]
  void* z_out;         // z transposed, [H_pad, z_ld] (element (row, h) at h*z_ld + row)
  int64_t z_ld;
  int buf_row_base;    // buffer row = global row - buf_row_base
  // backward inputs
  const float* lse;
  const float* phi;
  const float* psi;
  const float* alpha;
  const float* beta;
  const float* lnP;
  const float* dcosts;
  // fp32 mode: alpha, beta, ln P in fp64 (null: the fp32 arrays above)
  const double* alpha64;
  const double* beta64;
  const double* lnP64;
};

struct DhInplaceArgs {
  const Tile* tiles;
  int tile_begin, tile_end, row_begin;
  int64_t n_rows;
  const int32_t* T_len;
  const int32_t* U_len;
  const int32_t* labels;
  const int64_t* lat_off;  // packed lattice blocks
  int T, U1, V, V_pad, blank;
  void* logits;
  int buf_row_base;
  const float* lse;
  const float* phi;
  const float* psi;
  const float* alpha;
  const float* beta;
  const float* lnP;
  const float* dcosts;
  const double* alpha64;  // as in JointArgs
  const double* beta64;
  const double* lnP64;
};

// Writes out = labels with every label of columns 1..U_len[b] outside [0, V)
// (and every other column) set to blank; status = (count of such labels,
// flat index of the first or -1). One workgroup.
hipError_t launch_labels_check(const int32_t* labels, const int32_t* U_len, int B, int U1, int V, int blank,
                               int32_t* out, int32_t* status, hipStream_t st);

// (H_pad = 16 * joint_ks_for(H), declared in plan.hpp)
hipError_t launch_joint(const JointArgs& a, bool bf16_mode, bool bwd, hipStream_t st);
hipError_t launch_dh_inplace(const DhInplaceArgs& a, hipStream_t st);  // fp32 untiled mode

// Forward-backward variables over each sample's lattice.
struct LatticeArgs {
  const int32_t* T_len;
  const int32_t* U_len;
  const float* phi;  // packed layout (lat_off non-null) or padded layout (lat_ix)
  const float* psi;
  float* alpha;
  float* beta;
  float* lnP;   // [B] (may be null)
  float* costs; // [B] (may be null)
  int B, T, U1;
  double* alpha64;  // fp64 sweep only: alpha, beta (lattice layout) and ln P [B]
  const int64_t* lat_off;  // packed blocks [B] (saved); null: the padded layout
  double* beta64;
  double* lnP64;
  // fp32 sweep: a cell's two terms may both be -inf (a pruned lattice's
  // cells outside the band, or caller-given log-probs); false for the loss's
  // own full lattice, whose log-probs are finite
  bool clamp;
  // [2 B] (may be null): the paired sweep's workgroup j runs alpha of sample
  // pair[2 j] and beta of sample pair[2 j + 1]; each sample appears once in
  // each role
  const int32_t* pair;
};
hipError_t launch_lattice(const LatticeArgs& a, int U1max, hipStream_t st);
// Pruned lattice: phi = psi = -inf on every lattice cell (t < T_b, u <= U_b)
// outside its frame's band lo[b, t] <= u < lo[b, t] + S (packed layout).
hipError_t launch_band_fill(const int32_t* T_len, const int32_t* U_len, const int64_t* lat_off,
                            const int32_t* band_lo, int S, int B, int T, int U1, float* phi, float* psi,
                            hipStream_t st);
// The same recursions in fp64 from fp32 phi, psi: writes alpha64, beta64,
// lnP64 and (when non-null) lnP and costs rounded to fp32.
hipError_t launch_lattice64(const LatticeArgs& a, hipStream_t st);

// ---------------------------------------------------------------- GEMMs
// C[m, n] = sum_k A[m, k] * B[n, k] over a K range, 128 x 128 workgroup tiles.
// Operand access: "kc" = element (m, k) at base + m*ld + k (k contiguous);
// "mn" = element (m, k) at base + k*ld + m (m contiguous). kvalid (optional)
// masks whole k rows of an mn operand: k is valid iff
// (k % kv_T) < kv_len[k / kv_T] (+ kv_add), used to skip padded time/label
// rows of h^A / h^L.
struct Operand {
  const void* base;
  int64_t ld;
  int rows;          // valid m (or n) extent
  const int32_t* kv_len;
  int kv_T, kv_add;  // see above
};

struct GemmArgs {
  Operand A, B;
  int M, N, K;
  int k_per_split;   // K range per blockIdx.z
  // epilogue
  float* C;          // output (or partials base)
  int64_t ldc;
  int64_t split_stride;  // elements between split partials (0 = no split)
  int c_cols;        // columns to write (cols in [N, c_cols) get 0)
  const void* bias;  // optional bias over n
  int bias_bf16;
  float out_scale;   // C = (acc + bias) * out_scale; 0 means 1
  // optional column sums of A over k (sum over k of A[m, k]) for n-tile 0
  float* colsum;     // [splits, M] partials
};

enum GemmKind { GEMM_KC_KC = 0, GEMM_KC_MN = 1, GEMM_MN_MN = 2, GEMM_MN_KC = 3 };
// compute: 0 = bf16 MFMA (operands bf16), 1 = f32 MFMA; src_bf16 flags give the
// storage type of A and B.
hipError_t launch_gemm(const GemmArgs& g, GemmKind kind, bool bf16_compute, bool a_bf16,
                       bool b_bf16, int splits, hipStream_t st);

// dz = dh . W^O with dtanh and the per-tile sums over u (gA) and t (gL).
struct DzArgs {
  const Tile* tiles;
  int tile_begin, tile_end;
  int strip_begin;       // strip0 of tiles[tile_begin]
  int n_strips;
  int wave_row_base;     // buffer row = global row - wave_row_base
  const void* dh;        // [rows, V_pad]
  const void* z;         // z transposed, [H_pad, z_ld]
  int64_t z_ld;
  const void* WOT;       // W^O transposed, [H, V_pad] (zero for v >= V)
  int V, V_pad, H, H_pad;
  float* PA;             // [tiles_in_wave, tile_tp, H]
  float* PL;             // [tiles_in_wave, tile_tp/32, tile_u, H]
  int tile_tp, tile_u;
};
hipError_t launch_dz(const DzArgs& a, bool bf16_mode, hipStream_t st);

// Deterministic sums of the per-tile partials into gA / gL.
struct GroupReduceArgs {
  const Tile* tiles;
  const Group* groups;
  int n_groups;
  const int32_t* idx;    // tile ids (plan order)
  int tile_begin;        // partial slot = tile id - tile_begin
  const float* P;        // PA or PL
  int64_t tile_stride;   // floats per tile slot
  int n_sub;             // 1: sum the tile's htp/32 strips (PL); 0: one slot (PA)
  int64_t sub_stride;    // floats between strips
  float* G;              // gA [B*T, H] or gL [B*U1, H]
  int Gdim;              // T (for gA) or U1 (for gL)
  int H;
  int max_len;
};
hipError_t launch_group_reduce(const GroupReduceArgs& a, hipStream_t st);

// out[i] (+)= sum_s P[s*stride + i]
// dst[i] = bf16(src[i]) (round to nearest even), n a multiple of 4
hipError_t launch_to_bf16(const float* src, void* dst, int64_t n, hipStream_t st);
hipError_t launch_split_reduce(float* out, const float* P, int64_t n, int splits, int64_t stride,
                               bool accumulate, hipStream_t st);
hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t st);

// ---------------------------------------------------------------- bf16 large-tile path
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct DwoArgs {  // dW^O = dh^T z (split-K partials), db^O from a column of ones
  const void* dh;
  int64_t dh_ld;
  const void* z;
  int64_t z_ld;
  int V, H, K, k_per_split, splits;
  float* PW;  // [splits, V, H]
  float* PB;  // [splits, V]
};

struct ZArgs {  // z rows and (hb != null) the blank / label scores of a wave's strips
  const Tile* tiles;
  int tile_begin, tile_end, strip_begin, n_strips, n_ug, buf_row_base;
  const int32_t* U_len;
  const int32_t* labels;
  int T, U1, H, H_pad, blank;
  const float* a;
  const float* l;
  const void* WO;
  const void* bO;
  void* z;  // [rows, z_ld] bf16 (null: not written)
  int64_t z_ld;
  float* hb;
  float* hy;
  // fp8 output layer: z8 [rows, z8_ld] = E4M3(z 2^8) (null: not written);
  // with hb, the blank / label scores are those of the E4M3 operands (W^O
  // rows from WO8 scaled by 2^-(8+e))
  void* z8;
  int64_t z8_ld;
  const void* WO8;
  int H8;
  const int* ew;
};
hipError_t launch_zrow(const ZArgs& a, hipStream_t st);

// C[m, n] = (sum_k A[m, k] B[n, k] + bias[n]) * scale for n < N, 0 for
// N <= n < c_cols; A [M, lda] and B [N, ldb] bf16 with k contiguous, bias
// bf16 or null; fp32 C [M, ldc]. The bf16 joint pre-projections.
struct RowGemmArgs {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  const void* bias;
  float scale;
  float* C;
  int64_t ldc;
  int M, N, K, c_cols;
};
hipError_t launch_rowgemm(const RowGemmArgs& a, hipStream_t st);
// dst[r] = src[r] for rows r = b*Tdim + t with t < len[b] + add, else 0 (bf16
// rows of `cols` elements; cols % 8 == 0)
hipError_t launch_mask_rows(void* dst, const void* src, int64_t rows, int cols, int Tdim, const int32_t* len, int add,
                            hipStream_t st);
hipError_t launch_dz_dwo(const DzArgs& a, const DwoArgs& w, hipStream_t st);

struct ScoresArgs {  // scores^T tiles: forward statistics or backward dh
  const Tile* tiles;
  int tile_begin, tile_end, row_begin, n_rows, buf_row_base;
  const int32_t* T_len;
  const int32_t* U_len;
  const int32_t* labels;
  const int64_t* lat_off;
  int T, U1, V, H, V_pad, blank;
  const void* WO;
  const void* bO;
  const void* z;
  int64_t z_ld;
  f32x2* stats;   // forward: [rows, V tiles] (max, sum)
  void* logits;   // forward, untiled: fp16 (W^O z) log2 e [rows, V_pad] (global rows)
  void* dh;       // backward: [rows, V_pad]
  const float* lse;
  const float* phi;
  const float* psi;
  const float* alpha;
  const float* beta;
  const float* lnP;
  const float* dcosts;
};
hipError_t launch_scores(const ScoresArgs& a, bool bwd, hipStream_t st);

// Persistent 256-score x 128-cell tiles of the bf16 tiled path (one wave of
// tiles): forward (max, sum) statistics or backward dh without the blank /
// label terms; coef_kernel fills coefA / coefB, dh_fix subtracts the terms.
struct Scores3Args {
  const Tile* tiles;
  int tile_begin, tile_end, n_rows, n_ct, buf_row_base;  // n_ct = ceil(n_rows / 128)
  const int32_t* T_len;
  const int32_t* U_len;
  const int32_t* labels;
  const int64_t* lat_off;
  int T, U1, V, H_pad, V_pad, nvt, blank;
  const void* WOp;   // [nvt*256][H_pad] bf16, zero-padded W^O
  const float* bl;   // [nvt*256] b^O log2 e, -1e30 past V
  const void* z;     // [n_ct*128][z_ld] bf16
  int64_t z_ld;
  f32x2* stats;      // forward: [n_ct*128][nvt]
  void* dh;          // backward: [n_ct*128][V_pad] bf16
  void* logits;      // untiled mode: [n_rows][V_pad] fp16 (W^O z) log2 e (forward; null: not stored), dh in place (backward)
  void* coefA;       // [n_ct*128] (lse log2 e, occupancy)
  void* coefB;       // [n_ct*128] (cb, cl, label, 0)
  // fp8 output layer (WO8 non-null): E4M3 operands, rows of H8 bytes
  const void* WO8;   // [nvt*256][H8] W^O 2^e, zero-padded
  const void* z8;    // [n_ct*128][z8_ld] z 2^8
  int64_t z8_ld;
  int H8;
  const int* ew;     // the scale exponent e of W^O
  const float* lse;
  const float* phi;
  const float* psi;
  const float* alpha;
  const float* beta;
  const float* lnP;
  const float* dcosts;
};
hipError_t launch_scores3(const Scores3Args& a, bool bwd, hipStream_t st);
hipError_t launch_score_tables(const void* WO, const void* bO, void* WOp, float* bl, int V, int H, int H_pad,
                               int nvt, hipStream_t st);
// The bias table alone: bl[v] = b^O[v] log2 e for v < V, -1e30 up to nvt * 256.
hipError_t launch_bias_table(const void* bO, float* bl, int V, int nvt, hipStream_t st);
// fp8 output layer: ew = the largest e with max|W^O| 2^e <= 448 (0 if W^O is
// all zero), WO8 = E4M3(W^O 2^e) as [nvt*256][H8] bytes (0 past V and H), the
// bias table bl as launch_score_tables writes it.
hipError_t launch_score_tables8(const void* WO, const void* bO, void* WO8, float* bl, int* ew, int V, int H, int H8,
                                int nvt, hipStream_t st);
// grid over the wave's tiles x 32 x 32 blocks (+1 for the padding rows)
hipError_t launch_coef(const Scores3Args& a, int tile_t, int tile_u, hipStream_t st);
hipError_t launch_dh_fix(const Scores3Args& a, hipStream_t st);
// untiled mode: dh in place of the stored scores a.logits [n_rows][V_pad],
// from the coefficients coefA / coefB of launch_coef
hipError_t launch_dh_logits(const Scores3Args& a, hipStream_t st);

struct MergeArgs {
  const Tile* tiles;
  int tile_begin, tile_end, n_rows, buf_row_base, nvt;
  const int32_t* U_len;
  const int64_t* lat_off;
  const int32_t* band_lo;  // pruned lattice: [B, T] band starts (null: not pruned)
  int band_S;
  int T, U1;
  const f32x2* stats;
  const float* hb;
  const float* hy;
  float* lse;
  float* phi;
  float* psi;
};
// grid over the wave's tiles x 32 x 32 blocks: tile_t x tile_u bound every tile
hipError_t launch_lse_merge(const MergeArgs& a, int tile_t, int tile_u, hipStream_t st);
// dst[h, v] = src[v, h] for v < V (0 for V <= v < V_pad), element size 2 or 4
hipError_t launch_transpose_wo(void* dst, const void* src, int V, int H, int V_pad, bool bf16, hipStream_t st);
hipError_t launch_fill_bytes(void* p, int64_t nbytes, hipStream_t st);

}  // namespace rnnt
