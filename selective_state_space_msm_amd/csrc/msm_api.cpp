// C ABI of the Momentum-Mamba selective scan: argument checks, launch planning, workspace
// layout.  Every check happens before anything is enqueued; nothing here allocates memory.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "../../include/msm.h"
#include "msm_internal.h"

namespace {

using msm::kMaxChunks;
using msm::kTile;
using msm::kWave;

constexpr int64_t kTargetWaves = 1024;  // one wavefront per SIMD on 256 CUs x 4 SIMDs
constexpr int64_t kMaxWorkgroups = 4096;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

int padded_states(int64_t N) { return N <= 4 ? 4 : (N <= 16 ? 16 : (N <= 32 ? 32 : 64)); }

bool shape_ok(int64_t Bt, int64_t L, int64_t D, int64_t N) {
  if (Bt < 1 || L < 1 || D < 1 || N < 1) return false;
  const int64_t lim = (int64_t)1 << 40;
  if (Bt > lim || L > lim || D > lim) return false;
  // tile row offsets are 32-bit byte offsets: kTile rows of D fp32 values must fit
  if (D > ((int64_t)1 << 24)) return false;
  // element counts must stay far inside int64 and the grid inside 2^31 workgroups
  if (Bt * L > lim || Bt * L * D > ((int64_t)1 << 50)) return false;
  if (ceil_div(D, kWave) * Bt * kMaxChunks > ((int64_t)1 << 31) - 1) return false;
  return true;
}

msm_status check_common(int64_t Bt, int64_t L, int64_t D, int64_t N, float beta, float alpha,
                        msm_dtype io) {
  if (io != MSM_F32 && io != MSM_BF16) return MSM_ERR_UNSUPPORTED;
  if (Bt < 1 || L < 1 || D < 1 || N < 1) return MSM_ERR_INVALID_ARG;
  if (N > msm::kMaxN) return MSM_ERR_UNSUPPORTED;
  if (!shape_ok(Bt, L, D, N)) return MSM_ERR_INVALID_ARG;
  if (!(beta >= 0.0f && beta < 1.0f)) return MSM_ERR_INVALID_ARG;  // also rejects NaN
  if (!(alpha >= 0.0f) || !isfinite(alpha)) return MSM_ERR_INVALID_ARG;
  return MSM_OK;
}

// ---- forward planning ----
// Chunks a plan may ask for: enough workgroups to fill the GPU, at most kMaxChunks.
int64_t fwd_plan_chunks(int64_t Bt, int64_t L, int64_t D) {
  const int64_t wg_per_chunk = Bt * ceil_div(D, kWave);
  int64_t g = ceil_div(kMaxWorkgroups, wg_per_chunk);
  if (g > kMaxChunks) g = kMaxChunks;
  const int64_t tiles = ceil_div(L, kTile);
  if (g > tiles) g = tiles;
  return g < 1 ? 1 : g;
}

// Chunks every launch needs at least: the kernels address one chunk of one batch row of an
// (Bt, L, D) array with 32-bit byte offsets, so a chunk must stay below 2^31 bytes (with room
// for rounding the chunk length up to a whole tile).
int64_t fwd_min_chunks(int64_t L, int64_t D, int64_t es) {
  const int64_t max_rows = (((int64_t)1 << 31) - 1) / (D * es) - kTile;
  return ceil_div(L, max_rows);
}

// Chunks the workspace is sized for: the most any plan or the offset limit can need.
int64_t fwd_max_chunks(int64_t Bt, int64_t L, int64_t D, int64_t es) {
  const int64_t a = fwd_plan_chunks(Bt, L, D), b = fwd_min_chunks(L, D, es);
  return a > b ? a : b;
}

bool allowed_k(int NP, int K) {
  switch (NP) {
    case 4: return K == 1 || K == 2 || K == 4;
    case 16: return K == 1 || K == 2 || K == 4 || K == 8 || K == 16;
    case 32: return K == 4 || K == 8;
    case 64: return K == 4 || K == 8 || K == 16;
    default: return false;
  }
}

// Launch plan.  Measured on MI355X: the scan is VALU-bound, and two wavefronts per SIMD hide
// each other's LDS, memory and scalar instructions, so the preferred plan keeps S = NP/K
// wavefronts of few states each per 64-channel block when the channels alone give at least
// one wavefront per SIMD.  Otherwise the sequence is cut into chunks until there are a few
// wavefronts per SIMD: shorter chunks shorten the sequential path of every wavefront, and the
// extra summary work is small.  Measured on MI355X (Bt=1): L=65536 D=2048 N=16, 2 states per
// wavefront: 16 chunks 0.804 ms, 8 chunks 0.886 ms, 24 chunks 0.906 ms, 32 chunks 0.956 ms
// (4 states, 16 chunks: 0.840 ms; chunk counts that leave the workgroups unevenly spread over
// the CUs, 12 or 20, are slower still); L=16384 D=1024 N=16: 32 chunks best; N=4 and N=64 are
// best at about two wavefronts per SIMD.
msm_plan auto_fwd_plan(int64_t Bt, int64_t L, int64_t D, int64_t N) {
  const int NP = padded_states(N);
  const int64_t chan_blocks = Bt * ceil_div(D, kWave);
  msm_plan pl{0, 1};
  const int kpref = NP == 4 ? 1 : (NP == 16 ? 2 : (NP == 32 ? 4 : 8));
  if (chan_blocks * (NP / kpref) >= kTargetWaves) {
    pl.states_per_wave = kpref;
    return pl;
  }
  const int kchunk = NP == 4 ? 2 : (NP == 16 ? 2 : (NP == 32 ? 4 : 8));
  const int64_t waves = chan_blocks * (NP / kchunk);
  const int per_simd = NP == 16 ? 4 : 2;
  int64_t G = ceil_div(per_simd * kTargetWaves, waves);
  const int64_t gmax = fwd_plan_chunks(Bt, L, D);
  if (G > gmax) G = gmax;
  // Chunk k composes the maps of the k chunks before it in its prologue, so chunks are kept at
  // least 2G rows long (README shape, Bt=2 L=512 D=256 N=16: 16 chunks 20.0 us, 32 chunks
  // 24.2 us).  Below about a million state updates the summary pass's launch costs more than
  // its parallelism gains (Bt=1 L=64 D=4 N=4: one chunk 14.9 us, four chunks 16.9 us).
  while (G > 1 && ceil_div(L, G) < 2 * G) --G;
  if (Bt * L * D * N < ((int64_t)1 << 20)) G = 1;
  if (G < 1) G = 1;
  pl.states_per_wave = kchunk;
  pl.chunks = (int32_t)G;
  return pl;
}

// The half-wavefront layout of the forward's main pass (32 channels per workgroup, twice the
// workgroups of the full layout, two per CU with independent barriers) for unchunked plans.
// Measured on MI355X, 16 states, 2 per wavefront: Bt=4 L=4096 D=4096 bf16 0.335 ms against
// 0.345 ms in the full layout; Bt=8 L=2048 D=1536 fp32 0.169 against 0.177 ms.  Chunked plans
// already fill the CUs with several workgroups each and keep the full layout (Bt=1 L=65536
// D=2048 in 16 chunks: 0.92 ms half-wavefront against 0.79 ms).
bool fwd_half_wave(int64_t G) { return G == 1; }

struct FwdLayout {
  size_t off_bv, off_bh, off_q, off_sd, total;
};

// Chunk summaries for G chunks: (bv, bh, q) [Bt][G][N][D] and the delta sums [Bt][G][D], fp32.
FwdLayout fwd_layout_g(int64_t Bt, int64_t G, int64_t D, int64_t N) {
  FwdLayout l{};
  if (G <= 1) return l;
  const size_t per = align_up(sizeof(float) * (size_t)(Bt * G * N * D));
  l.off_bv = 0;
  l.off_bh = per;
  l.off_q = 2 * per;
  l.off_sd = 3 * per;
  l.total = 3 * per + align_up(sizeof(float) * (size_t)(Bt * G * D));
  return l;
}

// The workspace a caller passes is sized for the most chunks any plan can use.
FwdLayout fwd_layout(int64_t Bt, int64_t L, int64_t D, int64_t N, int64_t es) {
  return fwd_layout_g(Bt, fwd_max_chunks(Bt, L, D, es), D, N);
}

// ---- backward planning ----
// channels per backward workgroup: 64 for the full-wavefront kernel (64 padded states with
// K = 4), kBwdChans for the half-wavefront one
int64_t bwd_chans(int NP, int K) { return (NP == 64 && K == 4) ? kWave : msm::kBwdChans; }

// The half-wavefront backward addresses one tile's checkpoints ([2][N][D] fp32) through one
// buffer resource, whose extent is at most 2^31 - 1 bytes: 8 N D must stay below 2^31.
constexpr int64_t kBwdMaxL = (int64_t)1 << 30;

bool bwd_ckpt_ok(int64_t N, int64_t D) { return 8 * N * D < ((int64_t)1 << 31); }

// 64 padded states as two halves of the 32-state plan address a tile of the first half's
// fp64 sums ([L][2][D] per batch row) with 32-bit offsets: kBwdTile rows of 16 D bytes; the
// checkpoints keep their N-state layout
bool bwd_split_ok(int64_t N, int64_t D) {
  return (int64_t)msm::kBwdTile * 16 * D < ((int64_t)1 << 31) && bwd_ckpt_ok(N, D);
}

bool bwd_allowed_k(int NP, int K) {
  switch (NP) {
    case 4: return K == 1 || K == 2;
    case 16: return K == 1 || K == 2 || K == 4;
    case 32: return K == 2;  // 8 wavefronts of 2 states per half
    // two halves of the 32-state plan (K = 2), or the full-wavefront backward (K = 4)
    case 64: return K == 2 || K == 4;
    default: return false;
  }
}

// For 4, 16 or 32 padded states a backward workgroup holds 2K states of kBwdChans channels per
// wavefront and NP / (2K) wavefronts (32 states: always K = 2, 8 wavefronts).  A wavefront
// alone on its SIMD stalls on every non-VALU instruction and on LDS and fp64 latencies, so the
// plan asks for two wavefronts per SIMD: the largest K (at most 2: K = 4 needs more registers
// than two wavefronts leave) that still gives 2 * 1024 wavefronts, else K = 1.  64 padded states
// take K = 2, two launches of the 32-state plan, or K = 4, the full-wavefront kernel, when the
// first half's sums would exceed 32-bit offsets (D >= 2^23).
msm_plan auto_bwd_plan(int64_t Bt, int64_t L, int64_t D, int64_t N, int ext = 0) {
  const int NP = padded_states(N);
  msm_plan pl{0, 1};
  if (NP == 64 || NP == 32) {
    // 64 states: two launches of the 32-state plan (measured at Bt=4, L=2048, D=2048, N=64:
    // the full-wavefront kernel, which spills, takes 12.5 ms)
    pl.states_per_wave = (NP == 64 && !bwd_split_ok(N, D)) ? 4 : 2;
    return pl;
  }
  const int64_t chan_blocks = Bt * ceil_div(D, msm::kBwdChans);
  pl.states_per_wave = 1;
  if (bwd_allowed_k(NP, 2) && chan_blocks * (NP / 4) >= 2 * kTargetWaves) pl.states_per_wave = 2;
  // the zero-order hold carries more registers per state: at 16 padded states it runs with two
  // states per lane (measured at Bt=4, L=2048, D=2048: 0.99 ms against 2.52 ms with one, which
  // spills); the fused variant without it takes the default (0.504 ms with one state per lane
  // against 0.577 ms with two)
  if (ext == 2 && NP == 16) pl.states_per_wave = 2;
  return pl;
}

struct BwdLayout {
  size_t off_ckpt, off_dbc, off_dA, off_dD, off_dbias, off_accq, off_accz, total;
};

BwdLayout bwd_layout(int64_t Bt, int64_t L, int64_t D, int64_t N) {
  const int64_t NT = ceil_div(L, msm::kBwdTile);
  // sized for the narrower channel blocks, which have the most partial sums
  const int64_t ncb = ceil_div(D, msm::kBwdChans);
  const int NP = padded_states(N);
  BwdLayout l{};
  l.off_ckpt = 0;
  l.off_dbc = align_up(sizeof(float) * (size_t)(Bt * NT * 2 * N * D));
  l.off_dA = l.off_dbc + align_up(sizeof(float) * (size_t)(Bt * ncb * L * 2 * NP));
  l.off_dD = l.off_dA + align_up(sizeof(float) * (size_t)(Bt * N * D));
  l.off_dbias = l.off_dD + align_up(sizeof(float) * (size_t)(Bt * D));
  l.off_accq = l.off_dbias + align_up(sizeof(float) * (size_t)(Bt * D));
  l.off_accz = l.off_accq;
  l.total = l.off_accq;
  if (NP == 64 && bwd_split_ok(N, D)) {
    // the first half's sums when 64 states run as two halves
    l.off_accz = l.off_accq + align_up(sizeof(double) * 2 * (size_t)(Bt * L * D));
    l.total = l.off_accz + align_up(sizeof(float) * (size_t)(Bt * L * D));
  }
  return l;
}

// ---- overlap checks ----
struct Range {
  uintptr_t lo, hi;
};
Range rng(const void* p, size_t bytes) {
  Range r{(uintptr_t)p, (uintptr_t)p + bytes};
  return r;
}
bool overlaps(Range a, Range b) {
  if (a.lo == 0 || b.lo == 0 || a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}
bool any_overlap(const Range* outs, int nout, const Range* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlaps(outs[i], ins[j])) return true;
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(outs[i], outs[j])) return true;
  }
  return false;
}


// ---- complex scan ----
// The complex kernels address a tile of the state history ((kTile + 1) rows of N * D complex
// fp32 values) with 32-bit byte offsets.
bool complex_shape_ok(int64_t Bt, int64_t L, int64_t D, int64_t N) {
  if (!shape_ok(Bt, L, D, N)) return false;
  if ((int64_t)(kTile + 1) * N * D * 8 > ((int64_t)1 << 31) - 1) return false;
  if (ceil_div(D, msm::kBwdChans) * Bt > ((int64_t)1 << 31) - 1) return false;
  return true;
}

struct CBwdLayout {
  size_t off_hist, off_dbc, off_dA, off_dD, off_acc, total;
};

CBwdLayout cbwd_layout(int64_t Bt, int64_t L, int64_t D, int64_t N) {
  const int64_t ncb = ceil_div(D, msm::kBwdChans);
  const int NP = msm::complex_padded_states(N);
  CBwdLayout l{};
  l.off_hist = 0;
  l.off_dbc = align_up(sizeof(float) * 2 * (size_t)(Bt * (L + 1) * N * D));
  l.off_dA = l.off_dbc + align_up(sizeof(float) * 4 * (size_t)(Bt * ncb * L * NP));
  l.off_dD = l.off_dA + align_up(sizeof(float) * 2 * (size_t)(Bt * D * N));
  l.off_acc = l.off_dD + align_up(sizeof(float) * (size_t)(Bt * D));
  l.total = l.off_acc;
  // more than 16 states: the backward runs in launches of 16 states that sum dx, ddelta here
  if (NP > 16) l.total += align_up(sizeof(double) * 2 * (size_t)(Bt * L * D));
  return l;
}

// The complex kernels load B and C as whole (re, im) pairs and read the workspace's partial
// sums as 16-byte vectors.
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

msm_status check_complex(int64_t Bt, int64_t L, int64_t D, int64_t N, float beta, float alpha,
                         msm_dtype io) {
  msm_status st = check_common(Bt, L, D, N, beta, alpha, io);
  if (st != MSM_OK) return st;
  if (!complex_shape_ok(Bt, L, D, N)) return MSM_ERR_INVALID_ARG;
  // the complex kernels index rows and tiles of a sequence in 32 bits
  if (L >= kBwdMaxL) return MSM_ERR_UNSUPPORTED;
  return MSM_OK;
}

}  // namespace

extern "C" {

int32_t msm_version(void) { return 10000; }

const char* msm_status_string(msm_status s) {
  switch (s) {
    case MSM_OK: return "MSM_OK";
    case MSM_ERR_INVALID_ARG: return "MSM_ERR_INVALID_ARG: invalid argument";
    case MSM_ERR_UNSUPPORTED: return "MSM_ERR_UNSUPPORTED: unsupported by this build";
    case MSM_ERR_WORKSPACE: return "MSM_ERR_WORKSPACE: workspace too small";
    case MSM_ERR_LAUNCH: return "MSM_ERR_LAUNCH: kernel launch failed";
    default: return "MSM_ERR_UNKNOWN";
  }
}

size_t msm_scan_fwd_workspace_bytes(int64_t Bt, int64_t L, int64_t D, int64_t N, msm_dtype io) {
  if (check_common(Bt, L, D, N, 0.f, 1.f, io) != MSM_OK) return 0;
  if (fwd_min_chunks(L, D, io == MSM_BF16 ? 2 : 4) > kMaxChunks) return 0;
  return fwd_layout(Bt, L, D, N, io == MSM_BF16 ? 2 : 4).total;
}

size_t msm_scan_bwd_workspace_bytes(int64_t Bt, int64_t L, int64_t D, int64_t N, msm_dtype io) {
  if (check_common(Bt, L, D, N, 0.f, 1.f, io) != MSM_OK) return 0;
  return bwd_layout(Bt, L, D, N).total;
}

msm_status msm_scan_fwd_plan(int64_t Bt, int64_t L, int64_t D, int64_t N, msm_dtype io,
                             float beta, msm_plan* plan) {
  msm_status st = check_common(Bt, L, D, N, beta, 1.f, io);
  if (st != MSM_OK) return st;
  if (!plan) return MSM_ERR_INVALID_ARG;
  *plan = auto_fwd_plan(Bt, L, D, N);
  return MSM_OK;
}

msm_status msm_scan_bwd_plan(int64_t Bt, int64_t L, int64_t D, int64_t N, msm_dtype io,
                             float beta, msm_plan* plan) {
  msm_status st = check_common(Bt, L, D, N, beta, 1.f, io);
  if (st != MSM_OK) return st;
  if (!plan) return MSM_ERR_INVALID_ARG;
  *plan = auto_bwd_plan(Bt, L, D, N);
  return MSM_OK;
}

}  // extern "C"

namespace {

// The forward behind every forward entry point.  noalloc: ignore workspace / workspace_bytes
// and place the chunk summaries of this call's plan in the library's static device scratch
// (msm_scan_fwd_noalloc).
msm_status fwd_impl(const void* x, const void* delta, const float* A, const void* B,
                    const void* C, const float* Dskip, const void* z, const float* delta_bias,
                    int32_t delta_softplus, int32_t zero_order_hold, const float* h0,
                    const float* v0, void* y, float* last_h, float* last_v, int64_t Bt,
                    int64_t L, int64_t D, int64_t N, float beta, float alpha, msm_dtype io,
                    void* workspace, size_t workspace_bytes, void* stream, const msm_plan* plan,
                    bool noalloc) {
  msm_status st = check_common(Bt, L, D, N, beta, alpha, io);
  if (st != MSM_OK) return st;
  if (!x || !delta || !A || !B || !C || !y) return MSM_ERR_INVALID_ARG;
  if (delta_softplus != 0 && delta_softplus != 1) return MSM_ERR_INVALID_ARG;
  if (zero_order_hold != 0 && zero_order_hold != 1) return MSM_ERR_INVALID_ARG;
  const int ext = zero_order_hold ? 2 : (z || delta_bias || delta_softplus ? 1 : 0);

  msm_plan pl = auto_fwd_plan(Bt, L, D, N);
  const int NP = padded_states(N);
  if (plan) {
    if (plan->states_per_wave != 0) {
      if (!allowed_k(NP, plan->states_per_wave)) return MSM_ERR_UNSUPPORTED;
      pl.states_per_wave = plan->states_per_wave;
    }
    if (plan->chunks != 0) {
      if (plan->chunks < 1 || plan->chunks > fwd_plan_chunks(Bt, L, D)) return MSM_ERR_INVALID_ARG;
      pl.chunks = plan->chunks;
    }
  }

  const size_t es = io == MSM_BF16 ? 2 : 4;
  const size_t nxd = (size_t)(Bt * L * D), nbc = (size_t)(Bt * L * N);
  // a batch row's array may span at most kMaxChunks chunks of 2 GiB
  if (fwd_min_chunks(L, D, (int64_t)es) > kMaxChunks) return MSM_ERR_INVALID_ARG;

  // chunk length: a multiple of the tile, so only the final chunk can end mid-tile.  The
  // kernels address a chunk with 32-bit byte offsets: keep every chunk of every (Bt,L,D)
  // array below 2^31 bytes.
  int64_t G = pl.chunks;
  const int64_t gmin = fwd_min_chunks(L, D, (int64_t)es);
  if (G < gmin) G = gmin;  // within the workspace: fwd_layout is sized for it
  const int64_t Tc = ceil_div(ceil_div(L, G), kTile) * kTile;
  G = ceil_div(L, Tc);  // rounding Tc up can leave fewer non-empty chunks

  FwdLayout lay{};
  if (noalloc) {
    // the summaries of exactly this call's chunks, in the static scratch
    lay = fwd_layout_g(Bt, G, D, N);
    if (G > 1 && lay.total > msm::kNoAllocScratchBytes) return MSM_ERR_WORKSPACE;
    workspace = nullptr;
    workspace_bytes = 0;
  } else {
    lay = fwd_layout(Bt, L, D, N, (int64_t)es);
    if (workspace_bytes < lay.total || (lay.total > 0 && !workspace)) return MSM_ERR_WORKSPACE;
  }
  const size_t nst = (size_t)(Bt * D * N) * 4;
  const Range ins[] = {rng(x, nxd * es),        rng(delta, nxd * es),
                       rng(A, (size_t)(D * N) * 4), rng(B, nbc * es),
                       rng(C, nbc * es),        rng(Dskip, Dskip ? (size_t)D * 4 : 0),
                       rng(h0, h0 ? nst : 0),   rng(v0, v0 ? nst : 0),
                       rng(z, z ? nxd * es : 0), rng(delta_bias, delta_bias ? (size_t)D * 4 : 0)};
  const Range outs[] = {rng(y, nxd * es), rng(last_h, last_h ? nst : 0),
                        rng(last_v, last_v ? nst : 0), rng(workspace, noalloc ? 0 : lay.total)};
  if (any_overlap(outs, 4, ins, 10)) return MSM_ERR_INVALID_ARG;
  if (noalloc && G > 1) {
    // the scratch's device address on the current device (no allocation)
    if (msm::noalloc_scratch(&workspace) != hipSuccess) return MSM_ERR_LAUNCH;
  }

  msm::FwdArgs a{};
  a.x = x;
  a.delta = delta;
  a.A = A;
  a.B = B;
  a.C = C;
  a.Dskip = Dskip;
  a.h0 = h0;
  a.v0 = v0;
  a.y = y;
  a.last_h = last_h;
  a.last_v = last_v;
  a.z = z;
  a.delta_bias = delta_bias;
  a.delta_softplus = delta_softplus;
  char* ws = static_cast<char*>(workspace);
  a.s_bv = G > 1 ? reinterpret_cast<float*>(ws + lay.off_bv) : nullptr;
  a.s_bh = G > 1 ? reinterpret_cast<float*>(ws + lay.off_bh) : nullptr;
  a.s_q = G > 1 ? reinterpret_cast<float*>(ws + lay.off_q) : nullptr;
  a.s_sd = G > 1 ? reinterpret_cast<float*>(ws + lay.off_sd) : nullptr;
  a.Bt = Bt;
  a.L = L;
  a.D = D;
  a.N = N;
  a.Tc = Tc;
  a.G = (int32_t)G;
  a.ncb = (int32_t)ceil_div(D, kWave);
  a.ncb_hw = 2 * a.ncb;
  a.half_wave = fwd_half_wave(G) ? 1 : 0;
  a.beta = beta;
  a.alpha = alpha;
  a.beta_pow_tc = (float)pow((double)beta, (double)Tc);
  // rows after which the velocity's share beta^rows is below 2^-kWinLog2 (beta = 0: none)
  a.win_rows = beta > 0.f ? (int64_t)ceil(msm::kWinLog2 / -log2((double)beta)) : 0;
  if (a.win_rows < 0 || a.win_rows > L) a.win_rows = L;
  a.cus = 256;  // MI355X; replaced by the current device's count when the runtime reports it
  {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus > 0)
      a.cus = cus;
  }

  hipError_t e = msm::launch_fwd(a, io == MSM_BF16, pl.states_per_wave, beta == 0.0f, ext,
                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSM_OK : MSM_ERR_LAUNCH;
}

}  // namespace

extern "C" {

msm_status msm_selective_scan_fwd(const void* x, const void* delta, const float* A,
                                  const void* B, const void* C, const float* Dskip, const void* z,
                                  const float* delta_bias, int32_t delta_softplus,
                                  int32_t zero_order_hold, const float* h0, const float* v0,
                                  void* y, float* last_h,
                                  float* last_v, int64_t Bt, int64_t L, int64_t D, int64_t N,
                                  float beta, float alpha, msm_dtype io, void* workspace,
                                  size_t workspace_bytes, void* stream, const msm_plan* plan) {
  return fwd_impl(x, delta, A, B, C, Dskip, z, delta_bias, delta_softplus, zero_order_hold, h0,
                  v0, y, last_h, last_v, Bt, L, D, N, beta, alpha, io, workspace,
                  workspace_bytes, stream, plan, false);
}

msm_status msm_scan_fwd_noalloc(const void* x, const void* delta, const float* A, const void* B,
                                const void* C, const float* Dskip, void* y, float* last_h,
                                float* last_v, int64_t Bt, int64_t L, int64_t D, int64_t N,
                                float beta, float alpha, msm_dtype io, void* stream) {
  return fwd_impl(x, delta, A, B, C, Dskip, nullptr, nullptr, 0, 0, nullptr, nullptr, y, last_h,
                  last_v, Bt, L, D, N, beta, alpha, io, nullptr, 0, stream, nullptr, true);
}

msm_status msm_scan_fwd_state(const void* x, const void* delta, const float* A, const void* B,
                              const void* C, const float* Dskip, const float* h0,
                              const float* v0, void* y, float* last_h, float* last_v, int64_t Bt,
                              int64_t L, int64_t D, int64_t N, float beta, float alpha,
                              msm_dtype io, void* workspace, size_t workspace_bytes, void* stream,
                              const msm_plan* plan) {
  return msm_selective_scan_fwd(x, delta, A, B, C, Dskip, nullptr, nullptr, 0, 0, h0, v0, y,
                                last_h, last_v, Bt, L, D, N, beta, alpha, io, workspace,
                                workspace_bytes, stream, plan);
}

msm_status msm_scan_fwd_with_plan(const void* x, const void* delta, const float* A,
                                  const void* B, const void* C, const float* Dskip, void* y,
                                  float* last_h, float* last_v, int64_t Bt, int64_t L, int64_t D,
                                  int64_t N, float beta, float alpha, msm_dtype io,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  const msm_plan* plan) {
  return msm_scan_fwd_state(x, delta, A, B, C, Dskip, nullptr, nullptr, y, last_h, last_v, Bt, L,
                            D, N, beta, alpha, io, workspace, workspace_bytes, stream, plan);
}

msm_status msm_scan_fwd(const void* x, const void* delta, const float* A, const void* B,
                        const void* C, const float* Dskip, void* y, float* last_h,
                        float* last_v, int64_t Bt, int64_t L, int64_t D, int64_t N, float beta,
                        float alpha, msm_dtype io, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return msm_scan_fwd_with_plan(x, delta, A, B, C, Dskip, y, last_h, last_v, Bt, L, D, N, beta,
                                alpha, io, workspace, workspace_bytes, stream, nullptr);
}

msm_status msm_selective_scan_bwd(const void* x, const void* delta, const float* A,
                                  const void* B, const void* C, const float* Dskip, const void* z,
                                  const float* delta_bias, int32_t delta_softplus,
                                  int32_t zero_order_hold, const void* dy,
                                  const float* h0, const float* v0, const float* dlast_h,
                                  const float* dlast_v, void* dx, void* ddelta, float* dA,
                                  void* dB, void* dC, float* dDskip, void* dz,
                                  float* ddelta_bias, float* dh0, float* dv0, int64_t Bt,
                                  int64_t L, int64_t D, int64_t N, float beta, float alpha,
                                  msm_dtype io, void* workspace, size_t workspace_bytes,
                                  void* stream, const msm_plan* plan) {
  msm_status st = check_common(Bt, L, D, N, beta, alpha, io);
  if (st != MSM_OK) return st;
  if (!x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dA || !dB || !dC)
    return MSM_ERR_INVALID_ARG;
  if ((Dskip != nullptr) != (dDskip != nullptr)) return MSM_ERR_INVALID_ARG;
  if ((z != nullptr) != (dz != nullptr)) return MSM_ERR_INVALID_ARG;
  if ((delta_bias != nullptr) != (ddelta_bias != nullptr)) return MSM_ERR_INVALID_ARG;
  if (delta_softplus != 0 && delta_softplus != 1) return MSM_ERR_INVALID_ARG;
  if (zero_order_hold != 0 && zero_order_hold != 1) return MSM_ERR_INVALID_ARG;
  const int ext = zero_order_hold ? 2 : (z || delta_bias || delta_softplus ? 1 : 0);

  msm_plan pl = auto_bwd_plan(Bt, L, D, N, ext);
  const int NP = padded_states(N);
  if (plan) {
    if (plan->states_per_wave != 0) {
      if (!bwd_allowed_k(NP, plan->states_per_wave)) return MSM_ERR_UNSUPPORTED;
      if (NP == 64 && plan->states_per_wave == 2 && !bwd_split_ok(N, D)) return MSM_ERR_UNSUPPORTED;
      pl.states_per_wave = plan->states_per_wave;
    }
    if (plan->chunks != 0 && plan->chunks != 1) return MSM_ERR_UNSUPPORTED;
  }
  // up to 32 states the backward runs only in the half-wavefront kernel (64 states take the
  // full-wavefront one when the checkpoints are too large, see auto_bwd_plan)
  if (NP <= 32 && !bwd_ckpt_ok(N, D)) return MSM_ERR_UNSUPPORTED;
  // the backward kernels index rows and tiles of a sequence in 32 bits, and address a step of
  // their forward pass (4 tiles of (Bt, L, D) rows) with 32-bit offsets
  if (L >= kBwdMaxL) return MSM_ERR_UNSUPPORTED;
  if ((int64_t)4 * msm::kBwdTile * D * (io == MSM_BF16 ? 2 : 4) >= ((int64_t)1 << 31))
    return MSM_ERR_UNSUPPORTED;

  const size_t es = io == MSM_BF16 ? 2 : 4;
  const size_t nxd = (size_t)(Bt * L * D), nbc = (size_t)(Bt * L * N);
  const BwdLayout lay = bwd_layout(Bt, L, D, N);
  if (workspace_bytes < lay.total || !workspace) return MSM_ERR_WORKSPACE;
  const size_t nst = (size_t)(Bt * D * N) * 4;
  const Range ins[] = {rng(x, nxd * es),
                       rng(delta, nxd * es),
                       rng(A, (size_t)(D * N) * 4),
                       rng(B, nbc * es),
                       rng(C, nbc * es),
                       rng(Dskip, Dskip ? (size_t)D * 4 : 0),
                       rng(dy, nxd * es),
                       rng(h0, h0 ? nst : 0),
                       rng(v0, v0 ? nst : 0),
                       rng(dlast_h, dlast_h ? nst : 0),
                       rng(dlast_v, dlast_v ? nst : 0),
                       rng(z, z ? nxd * es : 0),
                       rng(delta_bias, delta_bias ? (size_t)D * 4 : 0)};
  const Range outs[] = {rng(dx, nxd * es),           rng(ddelta, nxd * es),
                        rng(dA, (size_t)(D * N) * 4), rng(dB, nbc * es),
                        rng(dC, nbc * es),           rng(dDskip, dDskip ? (size_t)D * 4 : 0),
                        rng(dh0, dh0 ? nst : 0),     rng(dv0, dv0 ? nst : 0),
                        rng(dz, dz ? nxd * es : 0),
                        rng(ddelta_bias, ddelta_bias ? (size_t)D * 4 : 0),
                        rng(workspace, lay.total)};
  if (any_overlap(outs, 11, ins, 13)) return MSM_ERR_INVALID_ARG;

  msm::BwdArgs a{};
  a.x = x;
  a.delta = delta;
  a.A = A;
  a.B = B;
  a.C = C;
  a.Dskip = Dskip;
  a.dy = dy;
  a.h0 = h0;
  a.v0 = v0;
  a.dlast_h = dlast_h;
  a.dlast_v = dlast_v;
  a.dh0 = dh0;
  a.dv0 = dv0;
  a.dx = dx;
  a.ddelta = ddelta;
  a.dA = dA;
  a.dB = dB;
  a.dC = dC;
  a.dDskip = dDskip;
  a.z = z;
  a.delta_bias = delta_bias;
  a.delta_softplus = delta_softplus;
  a.dz = dz;
  a.ddelta_bias = ddelta_bias;
  char* ws = static_cast<char*>(workspace);
  a.ckpt = reinterpret_cast<float*>(ws + lay.off_ckpt);
  a.dbc_part = reinterpret_cast<float*>(ws + lay.off_dbc);
  a.dA_part = reinterpret_cast<float*>(ws + lay.off_dA);
  a.dD_part = reinterpret_cast<float*>(ws + lay.off_dD);
  a.dbias_part = reinterpret_cast<float*>(ws + lay.off_dbias);
  a.acc_q = reinterpret_cast<double*>(ws + lay.off_accq);
  a.acc_dz = reinterpret_cast<float*>(ws + lay.off_accz);
  a.Bt = Bt;
  a.L = L;
  a.D = D;
  a.N = N;
  // (the split passes of 64 states and the full-wavefront kernel take kBwdTile rows)
  a.NT = ceil_div(L, NP == 64 ? msm::kBwdTile : msm::bwd_tile_rows(ext, pl.states_per_wave, 0));
  a.ncb = (int32_t)ceil_div(D, bwd_chans(NP, pl.states_per_wave));
  a.NP = NP;
  a.beta = beta;
  a.alpha = alpha;
  hipError_t e = msm::launch_bwd(a, io == MSM_BF16, pl.states_per_wave, beta == 0.0f, ext,
                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSM_OK : MSM_ERR_LAUNCH;
}

msm_status msm_scan_bwd_state(const void* x, const void* delta, const float* A, const void* B,
                              const void* C, const float* Dskip, const void* dy, const float* h0,
                              const float* v0, const float* dlast_h, const float* dlast_v,
                              void* dx, void* ddelta, float* dA, void* dB, void* dC,
                              float* dDskip, float* dh0, float* dv0, int64_t Bt, int64_t L,
                              int64_t D, int64_t N, float beta, float alpha, msm_dtype io,
                              void* workspace, size_t workspace_bytes, void* stream,
                              const msm_plan* plan) {
  return msm_selective_scan_bwd(x, delta, A, B, C, Dskip, nullptr, nullptr, 0, 0, dy, h0, v0,
                                dlast_h, dlast_v, dx, ddelta, dA, dB, dC, dDskip, nullptr,
                                nullptr, dh0, dv0, Bt, L, D, N, beta, alpha, io, workspace,
                                workspace_bytes, stream, plan);
}

msm_status msm_scan_bwd_with_plan(const void* x, const void* delta, const float* A,
                                  const void* B, const void* C, const float* Dskip,
                                  const void* dy, void* dx, void* ddelta, float* dA, void* dB,
                                  void* dC, float* dDskip, int64_t Bt, int64_t L, int64_t D,
                                  int64_t N, float beta, float alpha, msm_dtype io,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  const msm_plan* plan) {
  return msm_scan_bwd_state(x, delta, A, B, C, Dskip, dy, nullptr, nullptr, nullptr, nullptr, dx,
                            ddelta, dA, dB, dC, dDskip, nullptr, nullptr, Bt, L, D, N, beta,
                            alpha, io, workspace, workspace_bytes, stream, plan);
}

msm_status msm_scan_bwd(const void* x, const void* delta, const float* A, const void* B,
                        const void* C, const float* Dskip, const void* dy, void* dx,
                        void* ddelta, float* dA, void* dB, void* dC, float* dDskip, int64_t Bt,
                        int64_t L, int64_t D, int64_t N, float beta, float alpha, msm_dtype io,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return msm_scan_bwd_with_plan(x, delta, A, B, C, Dskip, dy, dx, ddelta, dA, dB, dC, dDskip, Bt,
                                L, D, N, beta, alpha, io, workspace, workspace_bytes, stream,
                                nullptr);
}

msm_status msm_scan_step(const void* x, const void* delta, const float* A, const void* B,
                         const void* C, const float* Dskip, const void* z,
                         const float* delta_bias, int32_t delta_softplus,
                         int32_t zero_order_hold, float* h, float* v, void* y, int64_t Bt,
                         int64_t D, int64_t N, float beta, float alpha, msm_dtype io,
                         void* stream) {
  msm_status st = check_common(Bt, 1, D, N, beta, alpha, io);
  if (st != MSM_OK) return st;
  if (!x || !delta || !A || !B || !C || !h || !v || !y) return MSM_ERR_INVALID_ARG;
  if (delta_softplus != 0 && delta_softplus != 1) return MSM_ERR_INVALID_ARG;
  if (zero_order_hold != 0 && zero_order_hold != 1) return MSM_ERR_INVALID_ARG;
  const size_t es = io == MSM_BF16 ? 2 : 4;
  const size_t nxd = (size_t)(Bt * D), nbc = (size_t)(Bt * N), nst = (size_t)(Bt * D * N) * 4;
  const Range ins[] = {rng(x, nxd * es),          rng(delta, nxd * es),
                       rng(A, (size_t)(D * N) * 4), rng(B, nbc * es),
                       rng(C, nbc * es),          rng(Dskip, Dskip ? (size_t)D * 4 : 0),
                       rng(z, z ? nxd * es : 0),  rng(delta_bias, delta_bias ? (size_t)D * 4 : 0)};
  // h and v are read and written in place: they may not overlap an input, y or each other
  const Range outs[] = {rng(y, nxd * es), rng(h, nst), rng(v, nst)};
  if (any_overlap(outs, 3, ins, 8)) return MSM_ERR_INVALID_ARG;

  int G = 1;
  while (4 * G < N) G *= 2;
  msm::StepArgs a{};
  a.x = x;
  a.delta = delta;
  a.z = z;
  a.A = A;
  a.B = B;
  a.C = C;
  a.Dskip = Dskip;
  a.delta_bias = delta_bias;
  a.delta_softplus = delta_softplus;
  a.zoh = zero_order_hold;
  a.h = h;
  a.v = v;
  a.y = y;
  a.Bt = Bt;
  a.D = D;
  a.N = N;
  a.G = G;
  a.beta = beta;
  a.alpha = alpha;
  const bool vec = N % 4 == 0 && (((uintptr_t)h | (uintptr_t)v | (uintptr_t)A) & 15) == 0;
  hipError_t e = msm::launch_step(a, io == MSM_BF16, vec, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSM_OK : MSM_ERR_LAUNCH;
}


size_t msm_scan_complex_bwd_workspace_bytes(int64_t Bt, int64_t L, int64_t D, int64_t N,
                                            msm_dtype io) {
  if (check_complex(Bt, L, D, N, 0.f, 1.f, io) != MSM_OK) return 0;
  return cbwd_layout(Bt, L, D, N).total;
}

msm_status msm_scan_complex_fwd(const void* x, const void* delta, const float* A, const void* B,
                                const void* C, const float* Dskip, const float* h0,
                                const float* v0, void* y, float* last_h, float* last_v,
                                int64_t Bt, int64_t L, int64_t D, int64_t N, float beta,
                                float alpha, msm_dtype io, void* stream) {
  msm_status st = check_complex(Bt, L, D, N, beta, alpha, io);
  if (st != MSM_OK) return st;
  if (!x || !delta || !A || !B || !C || !y) return MSM_ERR_INVALID_ARG;
  const size_t es = io == MSM_BF16 ? 2 : 4;
  if (!aligned(B, 2 * es) || !aligned(C, 2 * es)) return MSM_ERR_INVALID_ARG;
  const size_t nxd = (size_t)(Bt * L * D), nbc = (size_t)(Bt * L * N);
  const size_t nst = (size_t)(Bt * D * N) * 8;
  const Range ins[] = {rng(x, nxd * es),          rng(delta, nxd * es),
                       rng(A, (size_t)(D * N) * 8), rng(B, nbc * 2 * es),
                       rng(C, nbc * 2 * es),      rng(Dskip, Dskip ? (size_t)D * 4 : 0),
                       rng(h0, h0 ? nst : 0),     rng(v0, v0 ? nst : 0)};
  const Range outs[] = {rng(y, nxd * es), rng(last_h, last_h ? nst : 0),
                        rng(last_v, last_v ? nst : 0)};
  if (any_overlap(outs, 3, ins, 8)) return MSM_ERR_INVALID_ARG;
  msm::CFwdArgs a{};
  a.x = x;
  a.delta = delta;
  a.A = A;
  a.B = B;
  a.C = C;
  a.Dskip = Dskip;
  a.h0 = h0;
  a.v0 = v0;
  a.y = y;
  a.last_h = last_h;
  a.last_v = last_v;
  a.hist = nullptr;
  a.Bt = Bt;
  a.L = L;
  a.D = D;
  a.N = N;
  a.ncb = (int32_t)ceil_div(D, msm::kBwdChans);
  a.beta = beta;
  a.alpha = alpha;
  hipError_t e = msm::launch_cfwd(a, io == MSM_BF16, false, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSM_OK : MSM_ERR_LAUNCH;
}

msm_status msm_scan_complex_bwd(const void* x, const void* delta, const float* A, const void* B,
                                const void* C, const float* Dskip, const float* h0,
                                const float* v0, const void* dy, const float* dlast_h,
                                const float* dlast_v, void* dx, void* ddelta, float* dA,
                                void* dB, void* dC, float* dDskip, float* dh0, float* dv0,
                                int64_t Bt, int64_t L, int64_t D, int64_t N, float beta,
                                float alpha, msm_dtype io, void* workspace,
                                size_t workspace_bytes, void* stream) {
  msm_status st = check_complex(Bt, L, D, N, beta, alpha, io);
  if (st != MSM_OK) return st;
  if (!x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dA || !dB || !dC)
    return MSM_ERR_INVALID_ARG;
  if ((Dskip == nullptr) != (dDskip == nullptr)) return MSM_ERR_INVALID_ARG;
  const CBwdLayout lay = cbwd_layout(Bt, L, D, N);
  if (workspace_bytes < lay.total || !workspace) return MSM_ERR_WORKSPACE;
  const size_t es = io == MSM_BF16 ? 2 : 4;
  if (!aligned(B, 2 * es) || !aligned(C, 2 * es) || !aligned(workspace, 16))
    return MSM_ERR_INVALID_ARG;
  const size_t nxd = (size_t)(Bt * L * D), nbc = (size_t)(Bt * L * N);
  const size_t nst = (size_t)(Bt * D * N) * 8;
  const Range ins[] = {rng(x, nxd * es),          rng(delta, nxd * es),
                       rng(A, (size_t)(D * N) * 8), rng(B, nbc * 2 * es),
                       rng(C, nbc * 2 * es),      rng(Dskip, Dskip ? (size_t)D * 4 : 0),
                       rng(h0, h0 ? nst : 0),     rng(v0, v0 ? nst : 0),
                       rng(dy, nxd * es),         rng(dlast_h, dlast_h ? nst : 0),
                       rng(dlast_v, dlast_v ? nst : 0)};
  const Range outs[] = {rng(dx, nxd * es),       rng(ddelta, nxd * es),
                        rng(dA, (size_t)(D * N) * 8), rng(dB, nbc * 2 * es),
                        rng(dC, nbc * 2 * es),   rng(dDskip, dDskip ? (size_t)D * 4 : 0),
                        rng(dh0, dh0 ? nst : 0), rng(dv0, dv0 ? nst : 0),
                        rng(workspace, lay.total)};
  if (any_overlap(outs, 9, ins, 11)) return MSM_ERR_INVALID_ARG;

  char* ws = static_cast<char*>(workspace);
  float* hist = reinterpret_cast<float*>(ws + lay.off_hist);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  msm::CFwdArgs f{};
  f.x = x;
  f.delta = delta;
  f.A = A;
  f.B = B;
  f.C = C;
  f.h0 = h0;
  f.v0 = v0;
  f.hist = hist;
  f.Bt = Bt;
  f.L = L;
  f.D = D;
  f.N = N;
  f.ncb = (int32_t)ceil_div(D, msm::kBwdChans);
  f.beta = beta;
  f.alpha = alpha;
  hipError_t e = msm::launch_cfwd(f, io == MSM_BF16, true, s);
  if (e != hipSuccess) return MSM_ERR_LAUNCH;

  msm::CBwdArgs a{};
  a.x = x;
  a.delta = delta;
  a.A = A;
  a.B = B;
  a.C = C;
  a.Dskip = Dskip;
  a.dy = dy;
  a.dlast_h = dlast_h;
  a.dlast_v = dlast_v;
  a.dh0 = dh0;
  a.dv0 = dv0;
  a.dx = dx;
  a.ddelta = ddelta;
  a.dA = dA;
  a.dB = dB;
  a.dC = dC;
  a.dDskip = dDskip;
  a.hist = hist;
  a.dbc_part = reinterpret_cast<float*>(ws + lay.off_dbc);
  a.dA_part = reinterpret_cast<float*>(ws + lay.off_dA);
  a.dD_part = reinterpret_cast<float*>(ws + lay.off_dD);
  a.acc = reinterpret_cast<double*>(ws + lay.off_acc);
  a.n0 = 0;
  a.Bt = Bt;
  a.L = L;
  a.D = D;
  a.N = N;
  a.ncb = f.ncb;
  a.NP = msm::complex_padded_states(N);
  a.beta = beta;
  a.alpha = alpha;
  e = msm::launch_cbwd(a, io == MSM_BF16, s);
  return e == hipSuccess ? MSM_OK : MSM_ERR_LAUNCH;
}

}  // extern "C"
