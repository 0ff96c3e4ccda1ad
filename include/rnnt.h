/*
 * rnnt.h - C ABI of the MI355X (gfx950) RNN-T joint + loss library.
 *
 * The library computes, for a batch of B utterances, the RNN-T loss and its
 * gradients through the joint network and output layer:
 *
 *   joint network   z[b,t,u] = tanh(W^A h^A[b,t] + W^L h^L[b,u] + b^Z)
 *   output layer    h[b,t,u] = W^O z[b,t,u] + b^O              (V scores)
 *   two log-probs   phi = h[blank] - logsumexp(h), psi = h[y[u+1]] - logsumexp(h)
 *   lattice         alpha/beta forward-backward variables over t < T_b, u <= U_b
 *   loss            cost_b = -ln P(y_b | x_b) = -(alpha(T_b-1,U_b) + phi(T_b-1,U_b))
 *
 * Definitions: "Neural transducer training: reduced memory consumption with
 * sample-wise computation", section "Transducer training", Eqs. (3)-(10)
 * (joint network f^J, output layer f^O, loss sub-functions f^W_1..4; the
 * extraction lost Eq. (4), and tanh with a single bias b^Z is the reading this
 * library implements). Tiled recompute, the fused joint kernel, the
 * two-probability reduction, in-place gradients and the untiled mode follow
 * "Flash RNN-T: making room to train speech recognition", sections "Compute
 * it, use it, make room" and "Making each operation more efficient".
 *
 * Conventions shared by every entry point
 *  - All device buffers are allocated and owned by the caller. The library
 *    never allocates device memory; the bytes it needs beyond inputs and
 *    outputs are exactly what rnnt_loss_query reports.
 *  - Length arrays T_len_host / U_len_host are HOST int32 arrays [B], read
 *    during the call and not retained (the forward copies them, with the tile
 *    plan, into `saved`). 1 <= T_len[b] <= T, 0 <= U_len[b] <= U.
 *  - Float inputs (h^A, h^L, W^A, W^L, b^Z, W^O, b^O) all have the dtype of
 *    desc->dtype (fp32, or bf16 for RNNT_BF16 and RNNT_BF16_FP8), row-major,
 *    densely packed:
 *      hA [B,T,HA], hL [B,U+1,HL], WA [H,HA], WL [H,HL], bZ [H], WO [V,H], bO [V].
 *    labels is int32 [B,U+1] on the device; column 0 is the blank id, column
 *    u+1 (u < U_len[b]) is the label emitted from lattice row u. Entries past
 *    U_len[b] (and column 0) are never read. Label values must lie in [0,V):
 *    the forward copies the labels into `saved` and every kernel reads that
 *    copy, in which a label outside [0,V) is replaced by the blank id, so a
 *    bad label cannot address memory outside the output layer; it does make
 *    the results those of the replaced label. After the forward, the first two
 *    int32 of `saved` hold the number of such labels (0 if all are in range)
 *    and the flat index b*(U+1)+u+1 of the first one (-1 if none).
 *    Padded positions (t >= T_len[b], u > U_len[b]) of hA and hL may be read
 *    (the joint pre-projections run over all B*T and B*(U+1) rows) but never
 *    affect any cost or gradient: any values there, NaN and infinities
 *    included, give the same results.
 *  - costs, dcosts and every gradient output are fp32. Gradients are
 *    overwritten, not accumulated; padded rows of dhA/dhL are written as 0.
 *  - `stream` is a hipStream_t (NULL = the null stream). Every call enqueues
 *    work on that stream and returns without synchronizing the device. The
 *    forward's only host-to-device copy (the tile plan, a few hundred bytes
 *    to a few hundred KB) goes through a ring of pinned staging slots, each
 *    reused once its previous copy has completed; new slots are added while
 *    all are in flight, so a call waits on the host only if 16 forward calls'
 *    copies are still queued.
 *  - The calls can be captured into a HIP graph (stream capture): a forward
 *    called while its stream is capturing copies the plan from a host buffer
 *    the library keeps until the process ends, so every replay of the graph
 *    copies that call's plan.
 *  - Results are deterministic: every reduction (over tiles, waves, splits
 *    and samples) runs in a fixed order with no floating-point atomics, so
 *    repeated calls on the same inputs give identical bits.
 *  - Errors: every entry point validates its arguments on the host before
 *    launching anything and returns a status; no exception or exit crosses
 *    the ABI. rnnt_last_error() gives a thread-local description of the last
 *    failure. Calls are reentrant given distinct saved/workspace buffers.
 */
#ifndef RNNT_MI355_H
#define RNNT_MI355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RNNT_OK = 0,
  RNNT_E_INVALID = -1,     /* bad dims, lengths, pointers or tile settings   */
  RNNT_E_WORKSPACE = -2,   /* saved/workspace smaller than rnnt_loss_query   */
  RNNT_E_HIP = -3,         /* a HIP runtime call or kernel launch failed      */
  RNNT_E_UNSUPPORTED = -4  /* valid request outside the library's limits      */
} rnnt_status;

/* RNNT_BF16_FP8: bf16 inputs as in RNNT_BF16, with the output layer's product
 * W^O z in the score kernels (forward and the backward's recompute) taken on
 * OCP FP8 E4M3 operands: z scaled by 2^8 and W^O by 2^e (e the largest
 * integer with max|W^O| 2^e <= 448), each rounded to nearest even, the fp32
 * product scaled back by 2^-(8+e). The backward products dz = dh W^O and
 * dW^O = dh^T z stay bf16. An approximation of the bf16 result: "Neural
 * transducer training ...", Introduction and Conclusion, name reduced and
 * mixed precision without defining them; this is the library's reading.
 * Tiled mode only (RNNT_E_UNSUPPORTED in untiled mode). */
typedef enum { RNNT_F32 = 0, RNNT_BF16 = 1, RNNT_BF16_FP8 = 2 } rnnt_dtype;

/* Tiled: the joint/output intermediates exist one wave of tiles at a time and
 * are recomputed in the backward. Untiled: the forward keeps z and the scores
 * for every valid lattice cell in `saved` and the backward reuses them. */
typedef enum { RNNT_TILED = 0, RNNT_UNTILED = 1 } rnnt_mode;

typedef struct {
  int32_t B, T, U, V, HA, HL, H; /* lattice per sample is T x (U+1)           */
  int32_t blank;                 /* blank id, 0 <= blank < V                   */
  int32_t dtype;                 /* rnnt_dtype of all float inputs             */
  int32_t mode;                  /* rnnt_mode                                  */
  int32_t tile_t, tile_u;        /* tile extent in t and u (tiled mode), > 0   */
  int32_t tiles_per_wave;        /* tiles whose buffers coexist; 0 = default   */
  int32_t reserved;              /* must be 0. (No "deterministic" switch is
                                    needed: every call is deterministic.)    */
} rnnt_desc;

/* Limits of this library (RNNT_E_UNSUPPORTED beyond them): H, HA, HL multiples
 * of 8; H <= 768; U+1 <= 1024; V <= 65536; B*4*NQ*US <= 2^30 and
 * 4*NQ*US <= 2^29 with NQ = ceil((T+U)/4) and US = U+1 rounded up to a
 * multiple of 32 (the entries of the lattice arrays, see rnnt_lattice). Any tile size
 * is accepted; a tile's t extent is padded to a multiple of 32 rows inside the
 * library, so tile_t values that are multiples of 32 waste nothing. The
 * padded rows of all tiles, sum over tiles of (tile's u extent) x (its t
 * extent rounded up to 32), must not exceed 2^31 - 257 (row numbers are
 * 32-bit); very small tile_t on large batches can exceed it. */

/* Bytes of `saved` (lives from rnnt_loss_fwd to rnnt_loss_bwd, must not be
 * modified in between) and of `workspace` (scratch, reusable after each call)
 * for this descriptor and these lengths. Host-only; launches nothing.
 * Either output pointer may be NULL. */
rnnt_status rnnt_loss_query(const rnnt_desc* desc, const int32_t* T_len_host,
                            const int32_t* U_len_host, size_t* saved_bytes,
                            size_t* workspace_bytes);

/* Wave size from a memory budget (tiled mode): the largest tiles_per_wave
 * for which saved + workspace bytes (as rnnt_loss_query reports them for this
 * descriptor with that tiles_per_wave) fit in budget_bytes; desc's own
 * tiles_per_wave is ignored. Host-only. With tile_t >= T and tile_u >= U+1 a
 * tile is a whole sample, so the result is the number of samples computed
 * together: the sample-wise computation with batch splitting of "Neural
 * transducer training ...", section "Sample-wise method" (Alg. 1), whose
 * memory hardly grows with the batch size. RNNT_E_WORKSPACE if one tile per
 * wave already exceeds the budget; RNNT_E_INVALID in untiled mode or for a
 * null pointer; descriptor and length errors as rnnt_loss_query. */
rnnt_status rnnt_waves_for_budget(const rnnt_desc* desc, const int32_t* T_len_host,
                                  const int32_t* U_len_host, size_t budget_bytes,
                                  int32_t* tiles_per_wave);

/* Forward: per-sample costs[b] = -ln P(y_b | x_b) (fp32 [B], device).
 * Fills `saved` with the tile plan, the joint pre-activations, the per-cell
 * log-softmax denominators and two log-probs, alpha, beta and ln P (fp32 in
 * bf16 mode, fp64 in fp32 mode, where the backward pass needs
 * alpha + beta - ln P to better than fp32's spacing at these magnitudes) and,
 * in untiled mode, z and the scores. bf16 mode uses `workspace` (at least
 * rnnt_loss_query's workspace_bytes) for one wave of z rows and per-tile
 * statistics; fp32 mode does not use it (it may be NULL). */
rnnt_status rnnt_loss_fwd(const rnnt_desc* desc, const void* hA, const void* hL,
                          const int32_t* labels, const int32_t* T_len_host,
                          const int32_t* U_len_host, const void* WA, const void* WL,
                          const void* bZ, const void* WO, const void* bO, float* costs,
                          void* saved, size_t saved_bytes, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Pruned lattice (an approximation). "Neural transducer training ...",
 * Introduction and Conclusion, name pruning (its reference 14) among the ways
 * to cut the memory of the output tensor but do not define it; this library's
 * reading: frame t of sample b keeps the label positions
 *   lo_host[b*T + t] <= u < lo_host[b*T + t] + width
 * and every other cell of the lattice is removed (its two log-probs are -inf),
 * so the loss sums the alignments whose every cell lies in the band, pruned
 * cells get no gradient, and tiles holding no kept cell are not computed at
 * all (the saving). The bands are the caller's (computing them, e.g. from a
 * cheaper model, is outside this library). A band must hold an alignment:
 * width >= 1, lo[b, 0] = 0, lo non-decreasing in t with steps of at most
 * width - 1, 0 <= lo <= U_len[b], lo[b, T_len[b]-1] + width - 1 >= U_len[b];
 * otherwise RNNT_E_INVALID. Frames t >= T_len[b] are not read. lo_host is a
 * HOST int32 array [B, T], read during the call and copied into `saved`. */
typedef struct {
  const int32_t* lo_host;
  int32_t width;
} rnnt_band;

/* rnnt_loss_query, rnnt_loss_fwd and rnnt_loss_bwd on the pruned lattice of
 * `band` (the same band for the three calls; saved, workspace and results
 * are those of the pruned lattice). Every mode and dtype is supported. */
rnnt_status rnnt_loss_query_pruned(const rnnt_desc* desc, const int32_t* T_len_host,
                                   const int32_t* U_len_host, const rnnt_band* band,
                                   size_t* saved_bytes, size_t* workspace_bytes);
rnnt_status rnnt_loss_fwd_pruned(const rnnt_desc* desc, const void* hA, const void* hL,
                                 const int32_t* labels, const int32_t* T_len_host,
                                 const int32_t* U_len_host, const rnnt_band* band, const void* WA,
                                 const void* WL, const void* bZ, const void* WO, const void* bO,
                                 float* costs, void* saved, size_t saved_bytes, void* workspace,
                                 size_t workspace_bytes, void* stream);
rnnt_status rnnt_loss_bwd_pruned(const rnnt_desc* desc, const void* hA, const void* hL,
                                 const int32_t* labels, const int32_t* T_len_host,
                                 const int32_t* U_len_host, const rnnt_band* band, const void* WA,
                                 const void* WL, const void* bZ, const void* WO, const void* bO,
                                 const float* dcosts, void* saved, size_t saved_bytes,
                                 void* workspace, size_t workspace_bytes, float* dhA, float* dhL,
                                 float* dWA, float* dWL, float* dbZ, float* dWO, float* dbO,
                                 void* stream);

/* Bytes of the static device array rnnt_loss_fwd_noalloc uses as its workspace. */
#define RNNT_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/* Allocation-free forward, for callers that cannot allocate device memory
 * (code under stream capture, tight serving or evaluation loops, harnesses
 * that forbid allocation). Same arguments, results and `saved` contents as
 * rnnt_loss_fwd, without the workspace: the forward's working buffers live
 * in a static device array of RNNT_NOALLOC_SCRATCH_BYTES (256 MiB) that the
 * library holds on each GPU it runs on until the process ends. It calls no
 * device or pinned-host allocation: the tile plan is copied from pageable
 * host memory (so the call may wait for that copy to be staged). Every call
 * on one GPU shares that GPU's array, so calls that overlap on one GPU (two
 * streams, two threads) race and must be serialized by the caller. The
 * forward's workspace need grows with tiles_per_wave x tile area; a request
 * that needs more than the array returns RNNT_E_WORKSPACE before launching
 * anything (a smaller tiles_per_wave fits). fp32 mode needs no workspace. */
rnnt_status rnnt_loss_fwd_noalloc(const rnnt_desc* desc, const void* hA, const void* hL,
                                  const int32_t* labels, const int32_t* T_len_host,
                                  const int32_t* U_len_host, const void* WA, const void* WL,
                                  const void* bZ, const void* WO, const void* bO, float* costs,
                                  void* saved, size_t saved_bytes, void* stream);

/* Backward: gradients of L = sum_b dcosts[b] * cost_b (dcosts fp32 [B] on the
 * device; NULL means all ones, i.e. L = sum of costs) with respect to every
 * input: dhA [B,T,HA], dhL [B,U+1,HL], dWA [H,HA], dWL [H,HL], dbZ [H],
 * dWO [V,H], dbO [V], all fp32 on the device. The inputs must be the ones
 * given to rnnt_loss_fwd, and `saved` the buffer it filled. In untiled mode
 * the backward overwrites the scores kept in `saved` with their gradients
 * (in place, as the scores are not needed afterwards), so it may run once
 * per forward; in tiled mode `saved` is only read. The labels are read from
 * the forward's checked copy in `saved` (labels must still be non-null). */
rnnt_status rnnt_loss_bwd(const rnnt_desc* desc, const void* hA, const void* hL,
                          const int32_t* labels, const int32_t* T_len_host,
                          const int32_t* U_len_host, const void* WA, const void* WL,
                          const void* bZ, const void* WO, const void* bO,
                          const float* dcosts, void* saved, size_t saved_bytes,
                          void* workspace, size_t workspace_bytes, float* dhA, float* dhL,
                          float* dWA, float* dWL, float* dbZ, float* dWO, float* dbO,
                          void* stream);

/* The lattice step alone (forward-backward variables, "Transducer training"
 * Eqs. (8)-(9)) on caller-given two log-probs, for testing and for callers
 * that produce phi/psi themselves. T_len_dev / U_len_dev are DEVICE int32
 * arrays [B] (same ranges as above, not checked here). phi, psi, alpha, beta
 * are fp32 device arrays, 16-byte aligned, in the lattice layout of groups of
 * four anti-diagonals: with NQ = ceil((T + U) / 4) and US = U + 1 rounded up
 * to a multiple of 32, cell (t, u) of sample b, on diagonal d = t + u, is
 * element ((b * NQ + d / 4) * US + u) * 4 + d % 4 (B * NQ * US * 4 elements
 * per array; the four diagonals of one group and row are one aligned 16-byte
 * piece). Elements that are not cells of a sample's lattice may hold any
 * value, NaN and infinities included, and do not affect the results; psi
 * at u = U_len[b] likewise. costs[b] = -(alpha(T_b-1,U_b) + phi(T_b-1,U_b)).
 * Only the lattice cells of alpha and beta are written. desc supplies B, T,
 * U (other fields are ignored). RNNT_E_INVALID for a null or misaligned
 * pointer, RNNT_E_UNSUPPORTED beyond the limits above. */
rnnt_status rnnt_lattice(const rnnt_desc* desc, const int32_t* T_len_dev,
                         const int32_t* U_len_dev, const float* phi, const float* psi,
                         float* alpha, float* beta, float* costs, void* stream);

/* Launch timing (tracing). rnnt_profile_start() clears previous records and
 * makes every later launch record a hipEvent pair on its stream;
 * rnnt_profile_stop() waits for those events, turns them into per-kernel
 * totals (launch count and summed milliseconds, keyed by kernel name such as
 * "joint_fwd", "joint_bwd", "dz", "dWO_gemm", "lattice") and sets
 * *n_kernels; rnnt_profile_get(i, ...) reads entry i (0 <= i < n_kernels;
 * the name stays valid until the next rnnt_profile_start). Process-global;
 * not meant to be toggled while another thread is launching. */
rnnt_status rnnt_profile_start(void);
rnnt_status rnnt_profile_stop(int32_t* n_kernels);
rnnt_status rnnt_profile_get(int32_t i, const char** name, int32_t* launches, double* total_ms);

const char* rnnt_status_string(rnnt_status status);
const char* rnnt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RNNT_MI355_H */
