// C ABI of the RNN-T joint + loss library: argument checks, the tile plan,
// buffer layout and the launch sequence of the forward and backward passes.
//
// Forward ("Flash RNN-T", section "Compute it, use it, make room"; "Neural
// transducer training ...", section "Transducer training", Eqs. (3)-(9)):
//   1. a = W^A h^A + b^Z and l = W^L h^L              (MFMA GEMMs)
//   2. per lattice cell: z, scores, logsumexp, phi, psi (fused kernel; scores
//      and z kept only in untiled mode)
//   3. alpha, beta, ln P and the costs                  (lattice kernel)
// Backward (Eq. (10) and the gradient accumulation of the sample-wise
// method, section "Sample-wise method"), one wave of tiles at a time:
//   4. recompute scores, dh in place of them, z          (fused kernel)
//   5. dz = dh W^O, ds = dz (1 - z^2), sums over u / t  (dz kernel)
//   6. gA += sums over u, gL += sums over t             (ordered reductions)
//   7. dW^O += dh^T z, db^O += sum dh                    (split-K GEMM)
// then dh^A = gA W^A, dh^L = gL W^L, dW^A = gA^T h^A, dW^L = gL^T h^L,
// db^Z = sum gA.
#include <hip/hip_runtime.h>

#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/rnnt.h"
#include "common.hpp"
#include "kernels.hpp"
#include "plan.hpp"
#include "staging.hpp"

static_assert(sizeof(rnnt::Tile) == sizeof(rnnt::TileH), "tile record layout");
static_assert(sizeof(rnnt::Group) == sizeof(rnnt::GroupH), "group record layout");

namespace {

thread_local std::string g_last_error;

rnnt_status fail(rnnt_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

#define RNNT_HIP(call)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess)                                                              \
      return fail(RNNT_E_HIP, std::string(#call) + ": " + hipGetErrorString(e_));     \
  } while (0)

#define RNNT_STATUS(call)              \
  do {                                 \
    rnnt_status s_ = (call);           \
    if (s_ != RNNT_OK) return s_;      \
  } while (0)

rnnt_status to_dims(const rnnt_desc* desc, rnnt::Dims& d) {
  if (!desc) return fail(RNNT_E_INVALID, "desc is null");
  if (desc->dtype != RNNT_F32 && desc->dtype != RNNT_BF16 && desc->dtype != RNNT_BF16_FP8)
    return fail(RNNT_E_INVALID, "unknown dtype");
  if (desc->mode != RNNT_TILED && desc->mode != RNNT_UNTILED) return fail(RNNT_E_INVALID, "unknown mode");
  if (desc->reserved != 0) return fail(RNNT_E_INVALID, "reserved field must be 0");
  d = rnnt::Dims{desc->B, desc->T, desc->U, desc->V, desc->HA, desc->HL, desc->H, desc->blank,
                 desc->dtype != RNNT_F32, desc->mode == RNNT_UNTILED, desc->dtype == RNNT_BF16_FP8,
                 desc->tile_t, desc->tile_u, desc->tiles_per_wave};
  std::string err;
  int st = 0;
  if (!rnnt::check_dims(d, err, st)) return fail((rnnt_status)st, err);
  return RNNT_OK;
}

// band: null, or the bands of a pruned lattice (validated here).
rnnt_status prepare(const rnnt_desc* desc, const int32_t* T_len, const int32_t* U_len, rnnt::Plan& p,
                    rnnt::Layout& L, const rnnt_band* band = nullptr) {
  rnnt::Dims d;
  rnnt_status s = to_dims(desc, d);
  if (s != RNNT_OK) return s;
  std::string err;
  if (!rnnt::check_lengths(d, T_len, U_len, err)) return fail(RNNT_E_INVALID, err);
  rnnt::Band bd;
  if (band) {
    bd.lo = band->lo_host;
    bd.S = band->width;
    if (!rnnt::check_band(d, T_len, U_len, bd, err)) return fail(RNNT_E_INVALID, err);
  }
  int ks = rnnt::joint_ks_for(d.H);
  if (ks < 0) return fail(RNNT_E_UNSUPPORTED, "H too large for the fused joint kernel");
  rnnt::build_plan(d, T_len, U_len, ks * 16, p, bd);
  if (!rnnt::check_plan(p, err)) return fail(RNNT_E_UNSUPPORTED, err);
  L = rnnt::make_layout(p);
  return RNNT_OK;
}

// Pinned staging for the host -> device plan copy: a ring of slots, each
// reused once its previous copy has completed (staging.hpp), so no call
// waits on the host in steady state.
struct HipStagingBackend {
  using Event = hipEvent_t;
  using Stream = hipStream_t;
  void* alloc(size_t n) {
    void* p = nullptr;
    return hipHostMalloc(&p, n, hipHostMallocDefault) == hipSuccess ? p : nullptr;
  }
  hipEvent_t make_event() {
    hipEvent_t e = nullptr;
    return hipEventCreateWithFlags(&e, hipEventDisableTiming) == hipSuccess ? e : nullptr;
  }
  bool done(hipEvent_t e) { return hipEventQuery(e) == hipSuccess; }
  bool wait(hipEvent_t e) { return hipEventSynchronize(e) == hipSuccess; }
  bool copy(void* dst, const void* src, size_t n, hipStream_t st) {
    return hipMemcpyAsync(dst, src, n, hipMemcpyHostToDevice, st) == hipSuccess;
  }
  bool record(hipEvent_t e, hipStream_t st) { return hipEventRecord(e, st) == hipSuccess; }
};
rnnt::StagingRing<HipStagingBackend> g_staging;

rnnt_status upload(void* dst, const std::vector<char>& src, hipStream_t st) {
  const char* what = nullptr;
  if (!g_staging.upload(dst, src.data(), src.size(), st, &what))
    return fail(RNNT_E_HIP, std::string("plan upload: ") + (what ? what : "failed") + ": " +
                                hipGetErrorString(hipGetLastError()));
  return RNNT_OK;
}

// Under stream capture the copy becomes a graph node that reads its host
// source at every replay, so a captured forward copies its plan from a host
// buffer of its own, kept unchanged until the process ends (one per captured
// call: a staging slot is reused by later calls, and its event is not
// recorded during a capture). Ordinary heap memory: no pinned allocation.
std::mutex g_captured_mu;
std::vector<std::unique_ptr<char[]>> g_captured_plans;

rnnt_status plan_copy(void* dst, const std::vector<char>& src, hipStream_t st, bool scratch_mode) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  RNNT_HIP(hipStreamIsCapturing(st, &cs));
  if (cs == hipStreamCaptureStatusActive) {
    std::unique_ptr<char[]> buf(new char[src.size()]);
    std::memcpy(buf.get(), src.data(), src.size());
    RNNT_HIP(hipMemcpyAsync(dst, buf.get(), src.size(), hipMemcpyHostToDevice, st));
    std::lock_guard<std::mutex> lk(g_captured_mu);
    g_captured_plans.push_back(std::move(buf));
    return RNNT_OK;
  }
  if (scratch_mode) {
    // pageable source: the runtime has consumed it when the call returns
    RNNT_HIP(hipMemcpyAsync(dst, src.data(), src.size(), hipMemcpyHostToDevice, st));
    return RNNT_OK;
  }
  return upload(dst, src, st);
}

// ---------------------------------------------------------------- launch timing
// When enabled, every launch site records a hipEvent pair on the launch
// stream; rnnt_profile_stop() resolves them into per-kernel totals.
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<ProfRec> recs;
  std::vector<std::string> names;
  std::vector<int> launches;
  std::vector<double> total_ms;
};
Profiler g_prof;

struct ProfScope {
  hipStream_t st;
  hipEvent_t b = nullptr;
  ProfScope(const char* name, hipStream_t s) : st(s) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (!g_prof.on) return;
    hipEvent_t a;
    if (hipEventCreate(&a) != hipSuccess) return;
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      b = nullptr;
      return;
    }
    (void)hipEventRecord(a, st);
    g_prof.recs.push_back(ProfRec{name, a, b});
  }
  ~ProfScope() {
    if (b) (void)hipEventRecord(b, st);
  }
};

template <class T> T* at(void* base, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(base) + off); }
template <class T> const T* at(const void* base, size_t off) {
  return reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}

struct Saved {
  int32_t* status;
  int32_t* labels;  // the range-checked labels every kernel reads
  const int64_t* lat_off;  // packed lattice blocks
  const int32_t* lat_pair;  // lattice sweep pairing [2 B]
  const int32_t* band_lo;  // pruned lattice bands [B, T], else null
  const int32_t* Tlen;
  const int32_t* Ulen;
  const rnnt::Tile* tiles;
  const rnnt::Group* groups;
  const int32_t* gidx;
  float *a, *l, *lse, *phi, *psi, *alpha, *beta, *lnP;
  double *alpha64, *beta64, *lnP64;  // fp32 mode (the same memory as alpha, beta, lnP), else null
  void* logits;
  void* z;
};

Saved saved_view(void* s, const rnnt::Layout& L) {
  Saved v;
  v.status = at<int32_t>(s, L.off_status);
  v.labels = at<int32_t>(s, L.off_labels);
  v.lat_off = at<int64_t>(s, L.off_latoff);
  v.lat_pair = at<int32_t>(s, L.off_latpair);
  v.band_lo = L.off_band ? at<int32_t>(s, L.off_band) : nullptr;
  v.Tlen = at<int32_t>(s, L.off_Tlen);
  v.Ulen = at<int32_t>(s, L.off_Ulen);
  v.tiles = at<rnnt::Tile>(s, L.off_tiles);
  v.groups = at<rnnt::Group>(s, L.off_groups);
  v.gidx = at<int32_t>(s, L.off_gidx);
  v.a = at<float>(s, L.off_a);
  v.l = at<float>(s, L.off_l);
  v.lse = at<float>(s, L.off_lse);
  v.phi = at<float>(s, L.off_phi);
  v.psi = at<float>(s, L.off_psi);
  v.alpha = at<float>(s, L.off_alpha);
  v.beta = at<float>(s, L.off_beta);
  v.lnP = at<float>(s, L.off_lnP);
  v.alpha64 = L.lat64 ? at<double>(s, L.off_alpha) : nullptr;
  v.beta64 = L.lat64 ? at<double>(s, L.off_beta) : nullptr;
  v.lnP64 = L.lat64 ? at<double>(s, L.off_lnP) : nullptr;
  v.logits = L.off_logits ? at<char>(s, L.off_logits) : nullptr;
  v.z = L.off_z ? at<char>(s, L.off_z) : nullptr;
  return v;
}

rnnt::JointArgs joint_args(const rnnt::Plan& p, const Saved& sv, const void* WO, const void* bO) {
  rnnt::JointArgs a{};
  a.tiles = sv.tiles;
  a.T_len = sv.Tlen;
  a.U_len = sv.Ulen;
  a.labels = sv.labels;
  a.lat_off = sv.lat_off;
  a.band_lo = sv.band_lo;
  a.band_S = p.band_S;
  a.T = p.d.T;
  a.U1 = p.U1;
  a.V = p.d.V;
  a.H = p.d.H;
  a.H_pad = p.H_pad;
  a.V_pad = p.V_pad;
  a.blank = p.d.blank;
  a.a = sv.a;
  a.l = sv.l;
  a.WO = WO;
  a.bO = bO;
  a.lse = sv.lse;
  a.phi = sv.phi;
  a.psi = sv.psi;
  a.alpha = sv.alpha;
  a.beta = sv.beta;
  a.lnP = sv.lnP;
  a.alpha64 = sv.alpha64;
  a.beta64 = sv.beta64;
  a.lnP64 = sv.lnP64;
  return a;
}

inline int rows_per_chunk(bool bf16) { return bf16 ? 32 : 16; }

}  // namespace

// Workspace of rnnt_loss_fwd_noalloc: a static device array, one per GPU the
// library runs on, held until the process ends. Host code never uses its
// name as an address: the per-device address comes from hipGetSymbolAddress.
static constexpr size_t kScratchBytes = RNNT_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

struct ScratchAddrs {
  std::mutex mu;
  std::vector<void*> ptr;  // by device id
};
ScratchAddrs g_scratch;

// The current device's copy of `scratch`, looked up once per device.
rnnt_status scratch_for_current_device(void** out) {
  int dev = 0;
  RNNT_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(g_scratch.mu);
  if ((int)g_scratch.ptr.size() <= dev) g_scratch.ptr.resize(dev + 1, nullptr);
  if (!g_scratch.ptr[dev]) {
    void* p = nullptr;
    RNNT_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(RNNT_E_HIP, "hipGetSymbolAddress returned a null address for the scratch array");
    g_scratch.ptr[dev] = p;
  }
  *out = g_scratch.ptr[dev];
  return RNNT_OK;
}

}  // namespace

extern "C" {

const char* rnnt_status_string(rnnt_status s) {
  switch (s) {
    case RNNT_OK: return "ok";
    case RNNT_E_INVALID: return "invalid argument";
    case RNNT_E_WORKSPACE: return "saved or workspace buffer too small";
    case RNNT_E_HIP: return "HIP runtime error";
    case RNNT_E_UNSUPPORTED: return "outside the limits of this library";
  }
  return "unknown status";
}

const char* rnnt_last_error(void) { return g_last_error.c_str(); }

rnnt_status rnnt_loss_query(const rnnt_desc* desc, const int32_t* T_len_host, const int32_t* U_len_host,
                            size_t* saved_bytes, size_t* workspace_bytes) {
  rnnt::Plan p;
  rnnt::Layout L;
  rnnt_status s = prepare(desc, T_len_host, U_len_host, p, L);
  if (s != RNNT_OK) return s;
  if (saved_bytes) *saved_bytes = L.saved_bytes;
  if (workspace_bytes) *workspace_bytes = L.workspace_bytes;
  return RNNT_OK;
}

rnnt_status rnnt_loss_query_pruned(const rnnt_desc* desc, const int32_t* T_len_host, const int32_t* U_len_host,
                                   const rnnt_band* band, size_t* saved_bytes, size_t* workspace_bytes) {
  if (!band) return fail(RNNT_E_INVALID, "band is null");
  rnnt::Plan p;
  rnnt::Layout L;
  rnnt_status s = prepare(desc, T_len_host, U_len_host, p, L, band);
  if (s != RNNT_OK) return s;
  if (saved_bytes) *saved_bytes = L.saved_bytes;
  if (workspace_bytes) *workspace_bytes = L.workspace_bytes;
  return RNNT_OK;
}

rnnt_status rnnt_waves_for_budget(const rnnt_desc* desc, const int32_t* T_len_host, const int32_t* U_len_host,
                                  size_t budget_bytes, int32_t* tiles_per_wave) {
  if (!desc || !tiles_per_wave) return fail(RNNT_E_INVALID, "null descriptor or output pointer");
  if (desc->mode != RNNT_TILED) return fail(RNNT_E_INVALID, "waves are chosen in tiled mode only");
  rnnt_desc d = *desc;
  auto bytes = [&](int tpw, size_t& total, int& n_tiles) -> rnnt_status {
    d.tiles_per_wave = tpw;
    rnnt::Plan p;
    rnnt::Layout L;
    const rnnt_status s = prepare(&d, T_len_host, U_len_host, p, L);
    if (s != RNNT_OK) return s;
    total = L.saved_bytes + L.workspace_bytes;
    n_tiles = (int)p.tiles.size();
    return RNNT_OK;
  };
  size_t total = 0;
  int n_tiles = 0;
  rnnt_status s = bytes(1, total, n_tiles);
  if (s != RNNT_OK) return s;
  if (total > budget_bytes) return fail(RNNT_E_WORKSPACE, "one tile per wave already exceeds the budget");
  // the working set grows with tiles_per_wave up to the tile count
  int lo = 1, hi = std::max(n_tiles, 1);
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    int n = 0;
    s = bytes(mid, total, n);
    if (s != RNNT_OK) return s;
    if (total <= budget_bytes) lo = mid; else hi = mid - 1;
  }
  *tiles_per_wave = lo;
  return RNNT_OK;
}

// The forward pass. scratch_mode: the workspace is the static scratch array
// (rnnt_loss_fwd_noalloc): its regions follow the forward-only layout and
// the plan is copied from pageable memory, so nothing is allocated.
static rnnt_status forward_impl(const rnnt_desc* desc, const void* hA, const void* hL, const int32_t* labels,
                                const int32_t* T_len_host, const int32_t* U_len_host, const void* WA,
                                const void* WL, const void* bZ, const void* WO, const void* bO, float* costs,
                                void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                                void* stream, bool scratch_mode, const rnnt_band* band) {
  rnnt::Plan p;
  rnnt::Layout L;
  rnnt_status s = prepare(desc, T_len_host, U_len_host, p, L, band);
  if (s != RNNT_OK) return s;
  if (scratch_mode) L = rnnt::make_forward_layout(p);  // same saved layout, packed forward workspace
  if (!hA || !hL || !labels || !WA || !WL || !bZ || !WO || !bO || !costs || !saved)
    return fail(RNNT_E_INVALID, "null input, output or saved pointer");
  if (saved_bytes < L.saved_bytes) return fail(RNNT_E_WORKSPACE, "saved buffer smaller than rnnt_loss_query");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool bf = p.d.bf16;
  const rnnt::Dims& d = p.d;
  if (bf) {
    if (!workspace) return fail(RNNT_E_INVALID, "bf16 mode needs the workspace in the forward");
    if (workspace_bytes < L.workspace_bytes) {
      if (scratch_mode)
        return fail(RNNT_E_WORKSPACE, "the forward needs " + std::to_string(L.workspace_bytes) +
                                          " bytes of scratch, more than the " + std::to_string(workspace_bytes) +
                                          " of rnnt_loss_fwd_noalloc (fewer tiles per wave need less)");
      return fail(RNNT_E_WORKSPACE, "workspace buffer smaller than rnnt_loss_query");
    }
  }

  std::vector<char> host_plan;
  rnnt::serialize_plan(p, L, T_len_host, U_len_host, host_plan);
  s = plan_copy(saved, host_plan, st, scratch_mode);
  if (s != RNNT_OK) return s;
  Saved sv = saved_view(saved, L);
  {
    ProfScope ps_("labels_check", st);
    RNNT_HIP(rnnt::launch_labels_check(labels, sv.Ulen, d.B, p.U1, d.V, d.blank, sv.labels, sv.status, st));
  }
  if (sv.band_lo) {
    ProfScope ps_("band_fill", st);
    RNNT_HIP(rnnt::launch_band_fill(sv.Tlen, sv.Ulen, sv.lat_off, sv.band_lo, p.band_S, d.B, d.T, p.U1, sv.phi, sv.psi,
                                    st));
  }

  // 1. joint pre-activations (bf16: large-tile row GEMM, scaled for the z-row
  // kernel's base-2 exponential, the only reader of a and l in this mode)
  if (bf) {
    rnnt::RowGemmArgs r{};
    r.A = hA;
    r.lda = d.HA;
    r.B = WA;
    r.ldb = d.HA;
    r.bias = bZ;
    r.scale = rnnt::kTanhArgScale;
    r.C = sv.a;
    r.ldc = p.H_pad;
    r.M = d.B * d.T;
    r.N = d.H;
    r.K = d.HA;
    r.c_cols = p.H_pad;
    {
      ProfScope ps_("preproj_gemm", st);
      RNNT_HIP(rnnt::launch_rowgemm(r, st));
    }
    r.A = hL;
    r.lda = d.HL;
    r.B = WL;
    r.ldb = d.HL;
    r.bias = nullptr;
    r.C = sv.l;
    r.M = d.B * p.U1;
    r.K = d.HL;
    {
      ProfScope ps_("preproj_gemm", st);
      RNNT_HIP(rnnt::launch_rowgemm(r, st));
    }
  } else {
    rnnt::GemmArgs g{};
    g.A = rnnt::Operand{hA, d.HA, d.B * d.T, nullptr, 1, 0};
    g.B = rnnt::Operand{WA, d.HA, d.H, nullptr, 1, 0};
    g.M = d.B * d.T;
    g.N = d.H;
    g.K = d.HA;
    g.k_per_split = d.HA;
    g.C = sv.a;
    g.ldc = p.H_pad;
    g.c_cols = p.H_pad;
    g.bias = bZ;
    g.bias_bf16 = bf;
    // bf16 mode: a and l are read only by the z-row kernel, which wants the
    // tanh argument already scaled for its base-2 exponential
    g.out_scale = bf ? rnnt::kTanhArgScale : 0.0f;
    {
      ProfScope ps_("preproj_gemm", st);
      RNNT_HIP(rnnt::launch_gemm(g, rnnt::GEMM_KC_KC, bf, bf, bf, 1, st));
    }
    g.A = rnnt::Operand{hL, d.HL, d.B * p.U1, nullptr, 1, 0};
    g.B = rnnt::Operand{WL, d.HL, d.H, nullptr, 1, 0};
    g.M = d.B * p.U1;
    g.K = d.HL;
    g.k_per_split = d.HL;
    g.C = sv.l;
    g.bias = nullptr;
    {
      ProfScope ps_("preproj_gemm", st);
      RNNT_HIP(rnnt::launch_gemm(g, rnnt::GEMM_KC_KC, bf, bf, bf, 1, st));
    }
  }
  // 2. joint + output layer + log-softmax statistics
  if (bf) {
    // bf16: per wave of tiles, z rows (and the blank / label scores), then
    // 256 x 256 score tiles with per-tile (max, sum), then the merge
    void* zbuf = d.untiled ? sv.z : at<char>(workspace, L.w_z);
    auto* stats = at<rnnt::f32x2>(workspace, L.w_stats);
    float* hb = at<float>(workspace, L.w_hb);
    float* hy = at<float>(workspace, L.w_hy);
    const bool s3 = rnnt::persistent_scores(p);
    char* z8buf = d.fp8 ? at<char>(workspace, L.w_z8) : nullptr;
    int* ew = d.fp8 ? at<int>(workspace, L.w_ew) : nullptr;
    if (d.fp8) {
      ProfScope ps_("score_tables", st);
      RNNT_HIP(rnnt::launch_score_tables8(WO, bO, at<char>(workspace, L.w_WO8), at<float>(workspace, L.w_bl), ew, d.V,
                                          d.H, p.H8, p.nvt, st));
    } else if (s3) {
      ProfScope ps_("score_tables", st);
      RNNT_HIP(rnnt::launch_score_tables(WO, bO, at<char>(workspace, L.w_WOp), at<float>(workspace, L.w_bl), d.V,
                                         d.H, p.H_pad, p.nvt, st));
    }
    if (d.fp8 && p.H8 > p.H_pad) {
      // the z-row kernel writes H_pad columns; the score kernels read H8
      ProfScope ps_("fill", st);
      RNNT_HIP(rnnt::launch_fill_bytes(z8buf, (int64_t)((p.max_wave_rows + 127) / 128 * 128) * p.H8, st));
    }
    for (const rnnt::WaveInfo& wv : p.waves) {
      const int wrows = wv.row_end - wv.row_begin;
      const int base = d.untiled ? 0 : wv.row_begin;  // buffer row = global row - base
      rnnt::ZArgs z{};
      z.tiles = sv.tiles;
      z.tile_begin = wv.tile_begin;
      z.tile_end = wv.tile_end;
      z.strip_begin = wv.strip_begin;
      z.n_strips = wv.strip_end - wv.strip_begin;
      z.n_ug = (d.tile_u + 7) / 8;
      z.buf_row_base = base;
      z.U_len = sv.Ulen;
      z.labels = sv.labels;
      z.T = d.T;
      z.U1 = p.U1;
      z.H = d.H;
      z.H_pad = p.H_pad;
      z.blank = d.blank;
      z.a = sv.a;
      z.l = sv.l;
      z.WO = WO;
      z.bO = bO;
      z.z = d.fp8 ? nullptr : zbuf;  // fp8: the forward reads only the E4M3 rows
      z.z_ld = p.H_pad;
      z.hb = hb - (wv.row_begin - base);  // hb/hy indexed by wave-relative row
      z.hy = hy - (wv.row_begin - base);
      if (d.fp8) {
        z.z8 = z8buf;
        z.z8_ld = p.H8;
        z.WO8 = at<char>(workspace, L.w_WO8);
        z.H8 = p.H8;
        z.ew = ew;
      }
      {
        ProfScope ps_("zrow", st);
        RNNT_HIP(rnnt::launch_zrow(z, st));
      }
      rnnt::ScoresArgs sc{};
      sc.tiles = sv.tiles;
      sc.tile_begin = wv.tile_begin;
      sc.tile_end = wv.tile_end;
      sc.row_begin = wv.row_begin;
      sc.n_rows = wrows;
      sc.buf_row_base = wv.row_begin;
      sc.T = d.T;
      sc.U1 = p.U1;
      sc.V = d.V;
      sc.H = d.H;
      sc.V_pad = p.V_pad;
      sc.blank = d.blank;
      sc.WO = WO;
      sc.bO = bO;
      sc.z = at<char>(zbuf, (size_t)(wv.row_begin - base) * p.H_pad * 2);
      sc.z_ld = p.H_pad;
      sc.stats = stats;
      sc.logits = d.untiled ? sv.logits : nullptr;
      if (s3) {
        rnnt::Scores3Args a3{};
        a3.n_rows = wrows;
        a3.n_ct = (wrows + 127) / 128;
        a3.V = d.V;
        a3.H_pad = p.H_pad;
        a3.V_pad = p.V_pad;
        a3.nvt = p.nvt;
        a3.blank = d.blank;
        a3.WOp = d.fp8 ? nullptr : at<char>(workspace, L.w_WOp);
        a3.bl = at<float>(workspace, L.w_bl);
        a3.z = d.fp8 ? nullptr : sc.z;
        a3.z_ld = p.H_pad;
        a3.stats = stats;
        // untiled: the scores are kept for the backward (the wave's rows)
        a3.logits = d.untiled ? at<char>(sv.logits, (size_t)wv.row_begin * p.V_pad * 2) : nullptr;
        if (d.fp8) {
          a3.WO8 = at<char>(workspace, L.w_WO8);
          a3.z8 = z8buf;
          a3.z8_ld = p.H8;
          a3.H8 = p.H8;
          a3.ew = ew;
        }
        ProfScope ps_("scores_fwd", st);
        RNNT_HIP(rnnt::launch_scores3(a3, false, st));
      } else {
        ProfScope ps_("scores_fwd", st);
        RNNT_HIP(rnnt::launch_scores(sc, false, st));
      }
      rnnt::MergeArgs mg{};
      mg.tiles = sv.tiles;
      mg.tile_begin = wv.tile_begin;
      mg.tile_end = wv.tile_end;
      mg.n_rows = wrows;
      mg.buf_row_base = wv.row_begin;
      mg.nvt = p.nvt;
      mg.U_len = sv.Ulen;
      mg.lat_off = sv.lat_off;
      mg.band_lo = sv.band_lo;
      mg.band_S = p.band_S;
      mg.T = d.T;
      mg.U1 = p.U1;
      mg.stats = stats;
      mg.hb = hb;
      mg.hy = hy;
      mg.lse = sv.lse;
      mg.phi = sv.phi;
      mg.psi = sv.psi;
      {
        ProfScope ps_("lse_merge", st);
        RNNT_HIP(rnnt::launch_lse_merge(mg, d.tile_t, d.tile_u, st));
      }
    }
  } else {
    rnnt::JointArgs a = joint_args(p, sv, WO, bO);
    a.tile_begin = 0;
    a.tile_end = (int)p.tiles.size();
    a.row_begin = 0;
    a.n_chunks = (int)(p.total_rows / rows_per_chunk(bf));
    a.lse_out = sv.lse;
    a.phi_out = sv.phi;
    a.psi_out = sv.psi;
    a.store = d.untiled ? 1 : 0;
    a.logits_out = sv.logits;
    a.z_out = sv.z;
    a.z_ld = p.total_rows;
    a.buf_row_base = 0;
    {
      ProfScope ps_("joint_fwd", st);
      RNNT_HIP(rnnt::launch_joint(a, bf, false, st));
    }
  }
  // 3. lattice
  {
    rnnt::LatticeArgs la{sv.Tlen, sv.Ulen, sv.phi, sv.psi, sv.alpha, sv.beta, sv.lnP, costs, d.B, d.T, p.U1};
    la.lat_off = sv.lat_off;
    la.pair = sv.lat_pair;
    la.clamp = sv.band_lo != nullptr;
    ProfScope ps_("lattice", st);
    if (L.lat64) {
      // fp32 mode: the fp64 arrays share the fp32 ones' memory, so the fp32
      // ln P is not written
      la.alpha = la.beta = la.lnP = nullptr;
      la.alpha64 = sv.alpha64;
      la.beta64 = sv.beta64;
      la.lnP64 = sv.lnP64;
      RNNT_HIP(rnnt::launch_lattice64(la, st));
    } else {
      RNNT_HIP(rnnt::launch_lattice(la, p.U1, st));
    }
  }
  return RNNT_OK;
}

rnnt_status rnnt_loss_fwd(const rnnt_desc* desc, const void* hA, const void* hL, const int32_t* labels,
                          const int32_t* T_len_host, const int32_t* U_len_host, const void* WA,
                          const void* WL, const void* bZ, const void* WO, const void* bO, float* costs,
                          void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return forward_impl(desc, hA, hL, labels, T_len_host, U_len_host, WA, WL, bZ, WO, bO, costs, saved, saved_bytes,
                      workspace, workspace_bytes, stream, false, nullptr);
}

rnnt_status rnnt_loss_fwd_pruned(const rnnt_desc* desc, const void* hA, const void* hL, const int32_t* labels,
                                 const int32_t* T_len_host, const int32_t* U_len_host, const rnnt_band* band,
                                 const void* WA, const void* WL, const void* bZ, const void* WO, const void* bO,
                                 float* costs, void* saved, size_t saved_bytes, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!band) return fail(RNNT_E_INVALID, "band is null");
  return forward_impl(desc, hA, hL, labels, T_len_host, U_len_host, WA, WL, bZ, WO, bO, costs, saved, saved_bytes,
                      workspace, workspace_bytes, stream, false, band);
}

rnnt_status rnnt_loss_fwd_noalloc(const rnnt_desc* desc, const void* hA, const void* hL, const int32_t* labels,
                                  const int32_t* T_len_host, const int32_t* U_len_host, const void* WA,
                                  const void* WL, const void* bZ, const void* WO, const void* bO, float* costs,
                                  void* saved, size_t saved_bytes, void* stream) {
  void* ws = nullptr;
  const rnnt_status s = scratch_for_current_device(&ws);
  if (s != RNNT_OK) return s;
  return forward_impl(desc, hA, hL, labels, T_len_host, U_len_host, WA, WL, bZ, WO, bO, costs, saved, saved_bytes,
                      ws, kScratchBytes, stream, true, nullptr);
}

static rnnt_status backward_impl(const rnnt_desc* desc, const void* hA, const void* hL, const int32_t* labels,
                                 const int32_t* T_len_host, const int32_t* U_len_host, const void* WA,
                                 const void* WL, const void* bZ, const void* WO, const void* bO,
                                 const float* dcosts, void* saved, size_t saved_bytes, void* workspace,
                                 size_t workspace_bytes, float* dhA, float* dhL, float* dWA, float* dWL,
                                 float* dbZ, float* dWO, float* dbO, void* stream, const rnnt_band* band);

rnnt_status rnnt_loss_bwd(const rnnt_desc* desc, const void* hA, const void* hL, const int32_t* labels,
                          const int32_t* T_len_host, const int32_t* U_len_host, const void* WA,
                          const void* WL, const void* bZ, const void* WO, const void* bO,
                          const float* dcosts, void* saved, size_t saved_bytes, void* workspace,
                          size_t workspace_bytes, float* dhA, float* dhL, float* dWA, float* dWL,
                          float* dbZ, float* dWO, float* dbO, void* stream) {
  return backward_impl(desc, hA, hL, labels, T_len_host, U_len_host, WA, WL, bZ, WO, bO, dcosts, saved, saved_bytes,
                       workspace, workspace_bytes, dhA, dhL, dWA, dWL, dbZ, dWO, dbO, stream, nullptr);
}

rnnt_status rnnt_loss_bwd_pruned(const rnnt_desc* desc, const void* hA, const void* hL, const int32_t* labels,
                                 const int32_t* T_len_host, const int32_t* U_len_host, const rnnt_band* band,
                                 const void* WA, const void* WL, const void* bZ, const void* WO, const void* bO,
                                 const float* dcosts, void* saved, size_t saved_bytes, void* workspace,
                                 size_t workspace_bytes, float* dhA, float* dhL, float* dWA, float* dWL,
                                 float* dbZ, float* dWO, float* dbO, void* stream) {
  if (!band) return fail(RNNT_E_INVALID, "band is null");
  return backward_impl(desc, hA, hL, labels, T_len_host, U_len_host, WA, WL, bZ, WO, bO, dcosts, saved, saved_bytes,
                       workspace, workspace_bytes, dhA, dhL, dWA, dWL, dbZ, dWO, dbO, stream, band);
}

static rnnt_status backward_impl(const rnnt_desc* desc, const void* hA, const void* hL, const int32_t* labels,
                                 const int32_t* T_len_host, const int32_t* U_len_host, const void* WA,
                                 const void* WL, const void* bZ, const void* WO, const void* bO,
                                 const float* dcosts, void* saved, size_t saved_bytes, void* workspace,
                                 size_t workspace_bytes, float* dhA, float* dhL, float* dWA, float* dWL,
                                 float* dbZ, float* dWO, float* dbO, void* stream, const rnnt_band* band) {
  (void)bZ;
  rnnt::Plan p;
  rnnt::Layout L;
  rnnt_status s = prepare(desc, T_len_host, U_len_host, p, L, band);
  if (s != RNNT_OK) return s;
  if (!hA || !hL || !labels || !WA || !WL || !WO || !bO || !saved || !workspace || !dhA || !dhL || !dWA ||
      !dWL || !dbZ || !dWO || !dbO)
    return fail(RNNT_E_INVALID, "null input, output, saved or workspace pointer");
  if (saved_bytes < L.saved_bytes) return fail(RNNT_E_WORKSPACE, "saved buffer smaller than rnnt_loss_query");
  if (workspace_bytes < L.workspace_bytes)
    return fail(RNNT_E_WORKSPACE, "workspace buffer smaller than rnnt_loss_query");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool bf = p.d.bf16;
  const rnnt::Dims& d = p.d;
  Saved sv = saved_view(saved, L);
  float* gA = at<float>(workspace, L.w_gA);
  float* gL = at<float>(workspace, L.w_gL);
  float* PA = at<float>(workspace, L.w_PA);
  float* PL = at<float>(workspace, L.w_PL);
  float* PW = at<float>(workspace, L.w_PW);
  float* PB = at<float>(workspace, L.w_PB);
  void* dh_buf = d.untiled ? sv.logits : at<char>(workspace, L.w_dh);
  void* z_buf = d.untiled ? sv.z : at<char>(workspace, L.w_z);
  const int64_t z_ld = d.untiled ? p.total_rows : p.max_wave_rows;
  void* WOT = at<char>(workspace, L.w_WOT);
  {
    ProfScope ps_("transpose_wo", st);
    RNNT_HIP(rnnt::launch_transpose_wo(WOT, WO, d.V, d.H, p.V_pad, bf, st));
  }
  const bool s3 = rnnt::persistent_scores(p);
  char* z8buf = d.fp8 ? at<char>(workspace, L.w_z8) : nullptr;
  int* ew = d.fp8 ? at<int>(workspace, L.w_ew) : nullptr;
  if (d.fp8) {
    ProfScope ps_("score_tables", st);
    RNNT_HIP(rnnt::launch_score_tables8(WO, bO, at<char>(workspace, L.w_WO8), at<float>(workspace, L.w_bl), ew, d.V,
                                        d.H, p.H8, p.nvt, st));
  } else if (s3) {
    ProfScope ps_("score_tables", st);
    RNNT_HIP(rnnt::launch_score_tables(WO, bO, at<char>(workspace, L.w_WOp), at<float>(workspace, L.w_bl), d.V, d.H,
                                       p.H_pad, p.nvt, st));
  } else if (d.untiled && bf) {
    ProfScope ps_("score_tables", st);
    RNNT_HIP(rnnt::launch_bias_table(bO, at<float>(workspace, L.w_bl), d.V, p.nvt, st));
  }
  if (d.fp8 && p.H8 > p.H_pad) {
    ProfScope ps_("fill", st);
    RNNT_HIP(rnnt::launch_fill_bytes(z8buf, (int64_t)((p.max_wave_rows + 127) / 128 * 128) * p.H8, st));
  }

  {
    ProfScope ps_("fill", st);
    RNNT_HIP(rnnt::launch_fill(gA, (int64_t)d.B * d.T * d.H, 0.0f, st));
  }
  {
    ProfScope ps_("fill", st);
    RNNT_HIP(rnnt::launch_fill(gL, (int64_t)d.B * p.U1 * d.H, 0.0f, st));
  }
  {
    ProfScope ps_("fill", st);
    RNNT_HIP(rnnt::launch_fill(dWO, (int64_t)d.V * d.H, 0.0f, st));
  }
  {
    ProfScope ps_("fill", st);
    RNNT_HIP(rnnt::launch_fill(dbO, d.V, 0.0f, st));
  }

  for (const rnnt::WaveInfo& wv : p.waves) {
    const int wrows = wv.row_end - wv.row_begin;
    const int buf_base = d.untiled ? 0 : wv.row_begin;
    // 4. dh (and z) for the wave's cells
    if (d.untiled && bf) {
      // dh in place of the kept scores, from the per-row coefficients
      rnnt::Scores3Args a3{};
      a3.tiles = sv.tiles;
      a3.tile_begin = wv.tile_begin;
      a3.tile_end = wv.tile_end;
      a3.n_rows = wrows;
      a3.n_ct = (wrows + 127) / 128;
      a3.buf_row_base = wv.row_begin;
      a3.T_len = sv.Tlen;
      a3.U_len = sv.Ulen;
      a3.labels = sv.labels;
      a3.lat_off = sv.lat_off;
      a3.T = d.T;
      a3.U1 = p.U1;
      a3.V = d.V;
      a3.V_pad = p.V_pad;
      a3.blank = d.blank;
      a3.logits = at<char>(sv.logits, (size_t)wv.row_begin * p.V_pad * 2);
      a3.bl = at<float>(workspace, L.w_bl);
      a3.coefA = at<char>(workspace, L.w_coefA);
      a3.coefB = at<char>(workspace, L.w_coefB);
      a3.lse = sv.lse;
      a3.phi = sv.phi;
      a3.psi = sv.psi;
      a3.alpha = sv.alpha;
      a3.beta = sv.beta;
      a3.lnP = sv.lnP;
      a3.dcosts = dcosts;
      {
        ProfScope ps_("coef", st);
        RNNT_HIP(rnnt::launch_coef(a3, d.tile_t, d.tile_u, st));
      }
      {
        ProfScope ps_("dh_logits", st);
        RNNT_HIP(rnnt::launch_dh_logits(a3, st));
      }
    } else if (d.untiled) {
      rnnt::DhInplaceArgs a{};
      a.tiles = sv.tiles;
      a.tile_begin = wv.tile_begin;
      a.tile_end = wv.tile_end;
      a.row_begin = wv.row_begin;
      a.n_rows = wrows;
      a.T_len = sv.Tlen;
      a.U_len = sv.Ulen;
      a.labels = sv.labels;
      a.lat_off = sv.lat_off;
      a.T = d.T;
      a.U1 = p.U1;
      a.V = d.V;
      a.V_pad = p.V_pad;
      a.blank = d.blank;
      a.logits = sv.logits;
      a.buf_row_base = 0;
      a.lse = sv.lse;
      a.phi = sv.phi;
      a.psi = sv.psi;
      a.alpha = sv.alpha;
      a.beta = sv.beta;
      a.lnP = sv.lnP;
      a.alpha64 = sv.alpha64;
      a.beta64 = sv.beta64;
      a.lnP64 = sv.lnP64;
      a.dcosts = dcosts;
      {
        ProfScope ps_("dh_inplace", st);
        RNNT_HIP(rnnt::launch_dh_inplace(a, st));
      }
    } else if (bf) {
      // z rows for the wave, then dh from 256 x 256 score tiles
      rnnt::ZArgs z{};
      z.tiles = sv.tiles;
      z.tile_begin = wv.tile_begin;
      z.tile_end = wv.tile_end;
      z.strip_begin = wv.strip_begin;
      z.n_strips = wv.strip_end - wv.strip_begin;
      z.n_ug = (d.tile_u + 7) / 8;
      z.buf_row_base = buf_base;
      z.U_len = sv.Ulen;
      z.labels = sv.labels;
      z.T = d.T;
      z.U1 = p.U1;
      z.H = d.H;
      z.H_pad = p.H_pad;
      z.blank = d.blank;
      z.a = sv.a;
      z.l = sv.l;
      z.WO = WO;
      z.bO = bO;
      z.z = z_buf;
      z.z_ld = p.H_pad;
      z.hb = nullptr;  // the backward needs z only
      z.hy = nullptr;
      if (d.fp8) {  // and the E4M3 rows of the recomputed scores
        z.z8 = z8buf;
        z.z8_ld = p.H8;
        z.WO8 = at<char>(workspace, L.w_WO8);
        z.H8 = p.H8;
        z.ew = ew;
      }
      {
        ProfScope ps_("zrow", st);
        RNNT_HIP(rnnt::launch_zrow(z, st));
      }
      rnnt::ScoresArgs sc{};
      sc.tiles = sv.tiles;
      sc.tile_begin = wv.tile_begin;
      sc.tile_end = wv.tile_end;
      sc.row_begin = wv.row_begin;
      sc.n_rows = wrows;
      sc.buf_row_base = wv.row_begin;
      sc.T_len = sv.Tlen;
      sc.U_len = sv.Ulen;
      sc.labels = sv.labels;
      sc.lat_off = sv.lat_off;
      sc.T = d.T;
      sc.U1 = p.U1;
      sc.V = d.V;
      sc.H = d.H;
      sc.V_pad = p.V_pad;
      sc.blank = d.blank;
      sc.WO = WO;
      sc.bO = bO;
      sc.z = z_buf;
      sc.z_ld = p.H_pad;
      sc.dh = dh_buf;
      sc.lse = sv.lse;
      sc.phi = sv.phi;
      sc.psi = sv.psi;
      sc.alpha = sv.alpha;
      sc.beta = sv.beta;
      sc.lnP = sv.lnP;
      sc.dcosts = dcosts;
      if (s3) {
        rnnt::Scores3Args a3{};
        a3.tiles = sv.tiles;
        a3.tile_begin = wv.tile_begin;
        a3.tile_end = wv.tile_end;
        a3.n_rows = wrows;
        a3.n_ct = (wrows + 127) / 128;
        a3.buf_row_base = wv.row_begin;
        a3.T_len = sv.Tlen;
        a3.U_len = sv.Ulen;
        a3.labels = sv.labels;
        a3.lat_off = sv.lat_off;
        a3.T = d.T;
        a3.U1 = p.U1;
        a3.V = d.V;
        a3.H_pad = p.H_pad;
        a3.V_pad = p.V_pad;
        a3.nvt = p.nvt;
        a3.blank = d.blank;
        a3.WOp = d.fp8 ? nullptr : at<char>(workspace, L.w_WOp);
        a3.bl = at<float>(workspace, L.w_bl);
        a3.z = d.fp8 ? nullptr : z_buf;
        a3.z_ld = p.H_pad;
        a3.dh = dh_buf;
        if (d.fp8) {
          a3.WO8 = at<char>(workspace, L.w_WO8);
          a3.z8 = z8buf;
          a3.z8_ld = p.H8;
          a3.H8 = p.H8;
          a3.ew = ew;
        }
        a3.coefA = at<char>(workspace, L.w_coefA);
        a3.coefB = at<char>(workspace, L.w_coefB);
        a3.lse = sv.lse;
        a3.phi = sv.phi;
        a3.psi = sv.psi;
        a3.alpha = sv.alpha;
        a3.beta = sv.beta;
        a3.lnP = sv.lnP;
        a3.dcosts = dcosts;
        {
          ProfScope ps_("coef", st);
          RNNT_HIP(rnnt::launch_coef(a3, d.tile_t, d.tile_u, st));
        }
        {
          ProfScope ps_("scores_bwd", st);
          RNNT_HIP(rnnt::launch_scores3(a3, true, st));
        }
        {
          ProfScope ps_("dh_fix", st);
          RNNT_HIP(rnnt::launch_dh_fix(a3, st));
        }
      } else {
        ProfScope ps_("scores_bwd", st);
        RNNT_HIP(rnnt::launch_scores(sc, true, st));
      }
    } else {
      rnnt::JointArgs a = joint_args(p, sv, WO, bO);
      a.tile_begin = wv.tile_begin;
      a.tile_end = wv.tile_end;
      a.row_begin = wv.row_begin;
      a.n_chunks = wrows / rows_per_chunk(bf);
      a.logits_out = dh_buf;
      a.z_out = z_buf;
      a.z_ld = z_ld;
      a.buf_row_base = buf_base;
      a.dcosts = dcosts;
      {
        ProfScope ps_("joint_bwd", st);
        RNNT_HIP(rnnt::launch_joint(a, bf, true, st));
      }
    }
    // bf16: dW^O / db^O split-K partials, launched together with dz (step 5)
    rnnt::DwoArgs w{};
    if (bf) {
      w.dh = dh_buf;
      w.dh_ld = p.V_pad;
      w.z = z_buf;
      w.z_ld = p.H_pad;
      w.V = d.V;
      w.H = d.H;
      w.K = wrows;
      w.splits = p.s6;
      w.k_per_split = ((wrows + p.s6 - 1) / p.s6 + 63) / 64 * 64;
      w.PW = PW;
      w.PB = PB;
    }
    // 5. dz, dtanh and per-tile sums
    {
      rnnt::DzArgs a{};
      a.tiles = sv.tiles;
      a.tile_begin = wv.tile_begin;
      a.tile_end = wv.tile_end;
      a.strip_begin = wv.strip_begin;
      a.n_strips = wv.strip_end - wv.strip_begin;
      a.wave_row_base = buf_base;
      a.dh = dh_buf;
      a.z = z_buf;
      a.z_ld = z_ld;
      a.WOT = WOT;
      a.V = d.V;
      a.V_pad = p.V_pad;
      a.H = d.H;
      a.H_pad = p.H_pad;
      a.PA = PA;
      a.PL = PL;
      a.tile_tp = p.tile_tp;
      a.tile_u = d.tile_u;
      if (bf) {
        a.z_ld = p.H_pad;  // bf16 path: z rows are row-major
        ProfScope ps_("dz_dwo", st);
        RNNT_HIP(rnnt::launch_dz_dwo(a, w, st));
      } else {
        ProfScope ps_("dz", st);
        RNNT_HIP(rnnt::launch_dz(a, bf, st));
      }
    }
    // 6. gA / gL
    {
      rnnt::GroupReduceArgs r{};
      r.tiles = sv.tiles;
      r.groups = sv.groups + wv.gA_begin;
      r.n_groups = wv.gA_end - wv.gA_begin;
      r.idx = sv.gidx;
      r.tile_begin = wv.tile_begin;
      r.P = PA;
      r.tile_stride = (int64_t)p.tile_tp * d.H;
      r.n_sub = 0;
      r.sub_stride = 0;
      r.G = gA;
      r.Gdim = d.T;
      r.H = d.H;
      r.max_len = wv.maxA_len;
      {
        ProfScope ps_("group_reduce", st);
        RNNT_HIP(rnnt::launch_group_reduce(r, st));
      }
      r.groups = sv.groups + wv.gL_begin;
      r.n_groups = wv.gL_end - wv.gL_begin;
      r.P = PL;
      r.tile_stride = (int64_t)(p.tile_tp / 32) * d.tile_u * d.H;
      r.n_sub = 1;
      r.sub_stride = (int64_t)d.tile_u * d.H;
      r.G = gL;
      r.Gdim = p.U1;
      r.max_len = wv.maxL_len;
      {
        ProfScope ps_("group_reduce", st);
        RNNT_HIP(rnnt::launch_group_reduce(r, st));
      }
    }
    // 7. dW^O and db^O (the bf16 partials came with dz)
    if (bf) {
      {
        ProfScope ps_("split_reduce", st);
        RNNT_HIP(rnnt::launch_split_reduce(dWO, PW, (int64_t)d.V * d.H, p.s6, (int64_t)d.V * d.H, true, st));
      }
      {
        ProfScope ps_("split_reduce", st);
        RNNT_HIP(rnnt::launch_split_reduce(dbO, PB, d.V, p.s6, d.V, true, st));
      }
    } else {
      rnnt::GemmArgs g{};
      g.A = rnnt::Operand{dh_buf, p.V_pad, d.V, nullptr, 1, 0};
      g.B = rnnt::Operand{z_buf, z_ld, d.H, nullptr, 1, 0};  // z^T: k (row) contiguous
      g.M = d.V;
      g.N = d.H;
      g.K = wrows;
      const int kst = bf ? 64 : 32;
      g.k_per_split = (int)(((wrows + p.s6 - 1) / p.s6 + kst - 1) / kst * kst);
      g.C = PW;
      g.ldc = d.H;
      g.split_stride = (int64_t)d.V * d.H;
      g.c_cols = d.H;
      g.colsum = PB;
      // rows of the dh/z buffers start at the wave's first row
      {
        ProfScope ps_("dWO_gemm", st);
        RNNT_HIP(rnnt::launch_gemm(g, rnnt::GEMM_MN_KC, bf, bf, bf, p.s6, st));
      }
      {
        ProfScope ps_("split_reduce", st);
        RNNT_HIP(rnnt::launch_split_reduce(dWO, PW, (int64_t)d.V * d.H, p.s6, (int64_t)d.V * d.H, true, st));
      }
      {
        ProfScope ps_("split_reduce", st);
        RNNT_HIP(rnnt::launch_split_reduce(dbO, PB, d.V, p.s6, d.V, true, st));
      }
    }
  }

  // 8. encodings and joint weights. bf16 mode: gA and gL (complete only after
  // the last wave) are rounded to bf16 once and the four products run on bf16
  // MFMA with fp32 accumulation; fp32 mode: fp32 MFMA.
  const void* gA_op = gA;
  const void* gL_op = gL;
  if (bf) {
    char* gb = at<char>(workspace, L.w_gb);
    {
      ProfScope ps_("to_bf16", st);
      RNNT_HIP(rnnt::launch_to_bf16(gA, gb, (int64_t)d.B * d.T * d.H, st));
      RNNT_HIP(rnnt::launch_to_bf16(gL, gb + 2 * (size_t)d.B * d.T * d.H, (int64_t)d.B * p.U1 * d.H, st));
    }
    gA_op = gb;
    gL_op = gb + 2 * (size_t)d.B * d.T * d.H;
  }
  const int kst = bf ? 64 : 32;  // split-K granule of the GEMM engine
  if (bf) {
    // dh^A = gA W^A, dh^L = gL W^L on the large-tile row GEMM, with the
    // weights transposed so that both operands run along H
    char* WAT = at<char>(workspace, L.w_WAT);
    char* WLT = at<char>(workspace, L.w_WLT);
    {
      ProfScope ps_("transpose_wo", st);
      RNNT_HIP(rnnt::launch_transpose_wo(WAT, WA, d.H, d.HA, d.H, true, st));
      RNNT_HIP(rnnt::launch_transpose_wo(WLT, WL, d.H, d.HL, d.H, true, st));
    }
    rnnt::RowGemmArgs r{};
    r.A = gA_op;
    r.lda = d.H;
    r.B = WAT;
    r.ldb = d.H;
    r.bias = nullptr;
    r.scale = 1.0f;
    r.C = dhA;
    r.ldc = d.HA;
    r.M = d.B * d.T;
    r.N = d.HA;
    r.K = d.H;
    r.c_cols = d.HA;
    {
      ProfScope ps_("dh_enc_gemm", st);
      RNNT_HIP(rnnt::launch_rowgemm(r, st));
    }
    r.A = gL_op;
    r.B = WLT;
    r.C = dhL;
    r.ldc = d.HL;
    r.M = d.B * p.U1;
    r.N = d.HL;
    r.c_cols = d.HL;
    {
      ProfScope ps_("dh_enc_gemm", st);
      RNNT_HIP(rnnt::launch_rowgemm(r, st));
    }
  } else {
    rnnt::GemmArgs g{};
    g.A = rnnt::Operand{gA_op, d.H, d.B * d.T, nullptr, 1, 0};
    g.B = rnnt::Operand{WA, d.HA, d.HA, nullptr, 1, 0};
    g.M = d.B * d.T;
    g.N = d.HA;
    g.K = d.H;
    g.k_per_split = d.H;
    g.C = dhA;
    g.ldc = d.HA;
    g.c_cols = d.HA;
    {
      ProfScope ps_("dh_enc_gemm", st);
      RNNT_HIP(rnnt::launch_gemm(g, rnnt::GEMM_KC_MN, bf, bf, bf, 1, st));
    }
    g.A = rnnt::Operand{gL_op, d.H, d.B * p.U1, nullptr, 1, 0};
    g.B = rnnt::Operand{WL, d.HL, d.HL, nullptr, 1, 0};
    g.M = d.B * p.U1;
    g.N = d.HL;
    g.C = dhL;
    g.ldc = d.HL;
    g.c_cols = d.HL;
    {
      ProfScope ps_("dh_enc_gemm", st);
      RNNT_HIP(rnnt::launch_gemm(g, rnnt::GEMM_KC_MN, bf, bf, bf, 1, st));
    }
  }
  if (bf) {
    // dW^A = gA^T h^A (db^Z from the ones column) and dW^L = gL^T h^L on the
    // dW^O role of the dz_dwo kernel (256 x 256 tiles, split-K over the rows,
    // whole splits per XCD), on copies of h^A, h^L with the padding rows zeroed
    float* PWA = at<float>(workspace, L.w_PWA);
    float* PBZ = at<float>(workspace, L.w_PBZ);
    float* PWL = at<float>(workspace, L.w_PWL);
    char* hsA = at<char>(workspace, L.w_hs);
    char* hsL = hsA + 2 * (size_t)d.B * d.T * d.HA;
    {
      ProfScope ps_("mask_rows", st);
      RNNT_HIP(rnnt::launch_mask_rows(hsA, hA, (int64_t)d.B * d.T, d.HA, d.T, sv.Tlen, 0, st));
      RNNT_HIP(rnnt::launch_mask_rows(hsL, hL, (int64_t)d.B * p.U1, d.HL, p.U1, sv.Ulen, 1, st));
    }
    // out_b null: the ones column's sums (PB) are scratch
    auto dw = [&](const void* gop, const void* hs, int Hin, int64_t rows, int s_max, float* PW, float* PB,
                  float* out_W, float* out_b) -> rnnt_status {
      const int tiles = ((d.H + 255) / 256) * ((Hin + 1 + 255) / 256);
      const int splits = std::max(1, std::min(s_max, 8 * std::max(1, 32 / tiles)));
      rnnt::DwoArgs w{};
      w.dh = gop;
      w.dh_ld = d.H;
      w.z = hs;
      w.z_ld = Hin;
      w.V = d.H;
      w.H = Hin;
      w.K = (int)rows;
      w.splits = splits;
      w.k_per_split = (int)(((rows + splits - 1) / splits + 63) / 64 * 64);
      w.PW = PW;
      w.PB = PB;
      rnnt::DzArgs none{};
      {
        ProfScope ps_("dW_enc_gemm", st);
        RNNT_HIP(rnnt::launch_dz_dwo(none, w, st));
      }
      {
        ProfScope ps_("split_reduce", st);
        RNNT_HIP(rnnt::launch_split_reduce(out_W, PW, (int64_t)d.H * Hin, splits, (int64_t)d.H * Hin, false, st));
      }
      if (out_b) {
        ProfScope ps_("split_reduce", st);
        RNNT_HIP(rnnt::launch_split_reduce(out_b, PB, d.H, splits, d.H, false, st));
      }
      return RNNT_OK;
    };
    // PWA / PBZ hold s7a splits, PWL s7l
    rnnt_status s2 = dw(gA_op, hsA, d.HA, (int64_t)d.B * d.T, p.s7a, PWA, PBZ, dWA, dbZ);
    if (s2 != RNNT_OK) return s2;
    // dW^L has no bias: its ones column goes to PBZ, free once db^Z is reduced
    s2 = dw(gL_op, hsL, d.HL, (int64_t)d.B * p.U1, std::min(p.s7l, p.s7a), PWL, PBZ, dWL, nullptr);
    if (s2 != RNNT_OK) return s2;
    return RNNT_OK;
  }
  {
    float* PWA = at<float>(workspace, L.w_PWA);
    float* PBZ = at<float>(workspace, L.w_PBZ);
    float* PWL = at<float>(workspace, L.w_PWL);
    rnnt::GemmArgs g{};
    g.A = rnnt::Operand{gA_op, d.H, d.H, nullptr, 1, 0};
    g.B = rnnt::Operand{hA, d.HA, d.HA, sv.Tlen, d.T, 0};
    g.M = d.H;
    g.N = d.HA;
    g.K = d.B * d.T;
    g.k_per_split = (int)(((g.K + p.s7a - 1) / p.s7a + kst - 1) / kst * kst);
    g.C = PWA;
    g.ldc = d.HA;
    g.split_stride = (int64_t)d.H * d.HA;
    g.c_cols = d.HA;
    g.colsum = PBZ;
    {
      ProfScope ps_("dW_enc_gemm", st);
      RNNT_HIP(rnnt::launch_gemm(g, rnnt::GEMM_MN_MN, bf, bf, bf, p.s7a, st));
    }
    {
      ProfScope ps_("split_reduce", st);
      RNNT_HIP(rnnt::launch_split_reduce(dWA, PWA, (int64_t)d.H * d.HA, p.s7a, (int64_t)d.H * d.HA, false, st));
    }
    {
      ProfScope ps_("split_reduce", st);
      RNNT_HIP(rnnt::launch_split_reduce(dbZ, PBZ, d.H, p.s7a, d.H, false, st));
    }
    g.A = rnnt::Operand{gL_op, d.H, d.H, nullptr, 1, 0};
    g.B = rnnt::Operand{hL, d.HL, d.HL, sv.Ulen, p.U1, 1};
    g.N = d.HL;
    g.K = d.B * p.U1;
    g.k_per_split = (int)(((g.K + p.s7l - 1) / p.s7l + kst - 1) / kst * kst);
    g.C = PWL;
    g.ldc = d.HL;
    g.split_stride = (int64_t)d.H * d.HL;
    g.c_cols = d.HL;
    g.colsum = nullptr;
    {
      ProfScope ps_("dW_enc_gemm", st);
      RNNT_HIP(rnnt::launch_gemm(g, rnnt::GEMM_MN_MN, bf, bf, bf, p.s7l, st));
    }
    {
      ProfScope ps_("split_reduce", st);
      RNNT_HIP(rnnt::launch_split_reduce(dWL, PWL, (int64_t)d.H * d.HL, p.s7l, (int64_t)d.H * d.HL, false, st));
    }
  }
  return RNNT_OK;
}

rnnt_status rnnt_profile_start(void) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (auto& r : g_prof.recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.recs.clear();
  g_prof.names.clear();
  g_prof.launches.clear();
  g_prof.total_ms.clear();
  g_prof.on = true;
  return RNNT_OK;
}

rnnt_status rnnt_profile_stop(int32_t* n_kernels) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = false;
  rnnt_status st = RNNT_OK;
  for (auto& r : g_prof.recs) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) st = fail(RNNT_E_HIP, std::string("profile events: ") + hipGetErrorString(e));
    size_t k = 0;
    while (k < g_prof.names.size() && g_prof.names[k] != r.name) ++k;
    if (k == g_prof.names.size()) {
      g_prof.names.push_back(r.name);
      g_prof.launches.push_back(0);
      g_prof.total_ms.push_back(0.0);
    }
    g_prof.launches[k] += 1;
    g_prof.total_ms[k] += ms;
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.recs.clear();
  if (n_kernels) *n_kernels = (int32_t)g_prof.names.size();
  return st;
}

rnnt_status rnnt_profile_get(int32_t i, const char** name, int32_t* launches, double* total_ms) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (i < 0 || i >= (int32_t)g_prof.names.size()) return fail(RNNT_E_INVALID, "profile index out of range");
  if (name) *name = g_prof.names[i].c_str();
  if (launches) *launches = g_prof.launches[i];
  if (total_ms) *total_ms = g_prof.total_ms[i];
  return RNNT_OK;
}

rnnt_status rnnt_lattice(const rnnt_desc* desc, const int32_t* T_len_dev, const int32_t* U_len_dev,
                         const float* phi, const float* psi, float* alpha, float* beta, float* costs,
                         void* stream) {
  if (!desc) return fail(RNNT_E_INVALID, "desc is null");
  if (desc->B <= 0 || desc->T <= 0 || desc->U < 0) return fail(RNNT_E_INVALID, "need B, T > 0 and U >= 0");
  if (desc->U + 1 > 1024) return fail(RNNT_E_UNSUPPORTED, "this library supports U + 1 <= 1024");
  if (!T_len_dev || !U_len_dev || !phi || !psi || !alpha || !beta || !costs)
    return fail(RNNT_E_INVALID, "null pointer");
  for (const void* q : {(const void*)phi, (const void*)psi, (const void*)alpha, (const void*)beta})
    if (reinterpret_cast<uintptr_t>(q) % 16 != 0)
      return fail(RNNT_E_INVALID, "phi, psi, alpha and beta must be 16-byte aligned");
  if (rnnt::lat_cells(desc->B, desc->T, desc->U + 1) > ((int64_t)1 << 30) ||
      rnnt::lat_sample(desc->T, desc->U + 1) > ((int64_t)1 << 29))
    return fail(RNNT_E_UNSUPPORTED, "the lattice arrays exceed B*4*NQ*US <= 2^30 or 4*NQ*US <= 2^29 entries");
  rnnt::LatticeArgs la{T_len_dev, U_len_dev, phi, psi, alpha, beta, nullptr, costs, desc->B, desc->T, desc->U + 1};
  la.clamp = true;  // the caller's log-probs may hold -inf anywhere
  RNNT_HIP(rnnt::launch_lattice(la, desc->U + 1, reinterpret_cast<hipStream_t>(stream)));
  return RNNT_OK;
}

}  // extern "C"
