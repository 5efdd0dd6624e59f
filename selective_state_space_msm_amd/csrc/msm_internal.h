// Internal interface between the C-ABI layer (msm_api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace msm {

constexpr int kWave = 64;        // wavefront width on CDNA
constexpr int kTile = 16;        // time steps staged per LDS tile in the forward
constexpr int kMaxChunks = 64;   // upper bound on time chunks (sizes the workspace)
constexpr int kMaxN = 64;        // states supported per channel
constexpr int kBwdTile = 16;     // time steps recomputed per register tile in the backward
constexpr int kBwdChans = 32;    // channels per workgroup in the backward (half a wavefront)
// Rows per tile of the half-wavefront backward: 2 kBwdTile for the plain variant (EXT 0) at
// one state per lane in one launch, kBwdTile otherwise.  NT (and the checkpoint count) follow.
constexpr int bwd_tile_rows(int ext, int K, int split) {
  return (ext == 0 && K == 1 && split == 0) ? 2 * kBwdTile : kBwdTile;
}
// A chunk summary ignores rows whose share of the chunk's end state is below 2^-kWinLog2.
constexpr float kWinLog2 = 32.f;

struct FwdArgs {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;
  const float* h0;   // (Bt, D, N) initial state or null (zero)
  const float* v0;
  void* y;
  float* last_h;
  float* last_v;
  // fused extras (used by the EXT kernels only): delta_eff = softplus(delta + delta_bias[d])
  // (or delta + delta_bias[d]), y = y_raw * silu(z); null pointers mean no bias / no gate
  const void* z;
  const float* delta_bias;
  int32_t delta_softplus;
  // chunk summaries, [Bt][G][N][D] (sd: [Bt][G][D]); unused when G == 1
  float* s_bv;
  float* s_bh;
  float* s_q;
  float* s_sd;
  int64_t Bt, L, D, N;
  int64_t Tc;        // chunk length, a multiple of kTile
  int32_t G;         // number of chunks
  int32_t ncb;       // channel blocks of 64
  float beta, alpha;
  float beta_pow_tc;  // beta^Tc, the velocity decay across one full chunk
  int64_t win_rows;   // rows over which beta^rows < 2^-kWinLog2 (a summary window's minimum)
  int32_t cus;        // compute units of the device (picks the LDS layout of the y partials)
  // main pass in the half-wavefront layout (32-channel workgroups, 2 state groups per
  // wavefront) when the plan has one; ncb_hw = its channel blocks, 2 ceil(D / 64)
  int32_t half_wave;
  int32_t ncb_hw;
};

struct BwdArgs {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;
  const void* dy;
  const float* h0;       // (Bt, D, N) initial state or null (zero)
  const float* v0;
  const float* dlast_h;  // (Bt, D, N) adjoints of the final state or null (zero)
  const float* dlast_v;
  float* dh0;            // (Bt, D, N) adjoints of the initial state or null (not written)
  float* dv0;
  // fused extras (EXT kernels only): gate z and its gradient dz (Bt, L, D, I/O dtype), the
  // delta bias (D,) and its gradient; ddelta is then the gradient of the raw delta
  const void* z;
  const float* delta_bias;
  int32_t delta_softplus;
  void* dz;
  float* ddelta_bias;
  void* dx;
  void* ddelta;
  float* dA;
  void* dB;
  void* dC;
  float* dDskip;
  // workspace
  float* ckpt;       // [Bt][NT][2][N][D]  (v, h) before each tile of kBwdTile steps
  float* dbc_part;   // [Bt][ncb][L][2][NP] per channel-block (kBwdChans) partial sums
                     // of dB/alpha and dC
  // 64 padded states in two launches of the 32-state kernel: the launch's first state, which
  // launch (1, 2), and the first launch's sums for the second ([Bt][L][2][D] fp64 dx, ddelta;
  // [Bt][L][D] fp32 dz)
  int32_t n0;
  int32_t split_pass;
  double* acc_q;
  float* acc_dz;
  float* dA_part;    // [Bt][N][D]
  float* dD_part;    // [Bt][D]
  float* dbias_part; // [Bt][D] per batch row partial sums of the delta-bias gradient
  int64_t Bt, L, D, N;
  int64_t NT;        // tiles = ceil(L / kBwdTile)
  int32_t ncb;       // channel blocks: kBwdChans channels, or 64 when NP == 64
  int32_t NP;        // padded states
  float beta, alpha;
};

struct StepArgs {
  const void* x;          // (Bt, D) I/O dtype: the token's input, raw delta and gate
  const void* delta;
  const void* z;          // or null (no gate)
  const float* A;         // (D, N)
  const void* B;          // (Bt, N) I/O dtype
  const void* C;
  const float* Dskip;     // (D,) or null
  const float* delta_bias;  // (D,) or null
  int32_t delta_softplus;
  int32_t zoh;            // zero-order-hold write coefficient
  float* h;               // (Bt, D, N) fp32 states, updated in place
  float* v;
  void* y;                // (Bt, D) I/O dtype
  int64_t Bt, D, N;
  int32_t G;              // lanes per channel: ceil(N / 4) rounded up to a power of two
  float beta, alpha;
};

// Complex-valued scan: A (D, N), B, C (Bt, L, N), the states and their adjoints are
// interleaved (re, im) pairs; x, delta, y, dy, dx, ddelta are real.
struct CFwdArgs {
  const void* x;
  const void* delta;
  const float* A;       // (D, N) complex fp32
  const void* B;        // (Bt, L, N) complex, I/O dtype
  const void* C;
  const float* Dskip;
  const float* h0;      // (Bt, D, N) complex fp32 or null (zero)
  const float* v0;
  void* y;              // (Bt, L, D); unused by the recording pass
  float* last_h;        // (Bt, D, N) complex fp32 or null
  float* last_v;
  float* hist;          // recording pass: (Bt, L + 1, N, D) complex fp32, row r = h_{r-1}
  int64_t Bt, L, D, N;
  int32_t ncb;          // channel blocks of kBwdChans
  float beta, alpha;
};

struct CBwdArgs {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;
  const void* dy;
  const float* dlast_h;  // (Bt, D, N) complex fp32 or null (zero)
  const float* dlast_v;
  float* dh0;            // (Bt, D, N) complex fp32 or null (not written)
  float* dv0;
  void* dx;
  void* ddelta;
  float* dA;             // (D, N) complex fp32
  void* dB;              // (Bt, L, N) complex, I/O dtype
  void* dC;
  float* dDskip;
  const float* hist;     // written by the recording forward pass
  float* dbc_part;       // [Bt][ncb][L][NP][4]: per channel block (dB re, im, dC re, im)
  float* dA_part;        // [Bt][D][N][2]
  float* dD_part;        // [Bt][D]
  // 32 or 64 padded states run as launches of 16 states: the launch's first state and the
  // running fp64 sums of dx, ddelta ([Bt][L][2][D])
  int32_t n0;
  double* acc;
  int64_t Bt, L, D, N;
  int32_t ncb;
  int32_t NP;            // padded states
  float beta, alpha;
};

// Complex forward (record = false: y and the last states; record = true: the state history
// only, for the backward) and complex backward (its sweep and the partial-sum reduction).
hipError_t launch_cfwd(const CFwdArgs& a, int io_bf16, bool record, hipStream_t s);
hipError_t launch_cbwd(const CBwdArgs& a, int io_bf16, hipStream_t s);
// padded complex states of a plan: 4, 16, 32 or 64
inline int complex_padded_states(int64_t N) {
  return N <= 4 ? 4 : (N <= 16 ? 16 : (N <= 32 ? 32 : 64));
}

// One decode step; vec selects 16-byte state access (N % 4 == 0 and 16-byte aligned states
// and A).  Returns hipSuccess or the launch error.
hipError_t launch_step(const StepArgs& a, int io_bf16, bool vec, hipStream_t s);

// Both return hipSuccess or the first launch error.  `ext` selects the variant: 0 plain,
// 1 fused (bias, softplus, gate), 2 fused with the zero-order-hold write coefficient.
hipError_t launch_fwd(const FwdArgs& a, int io_bf16, int K, bool beta0, int ext, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, int io_bf16, int K, bool beta0, int ext, hipStream_t s);

// The recurrence kernels are compiled once per (I/O dtype, variant) pair, each build of
// msm_fwd.hip / msm_bwd.hip defining one of these (suffix: bf16 I/O, variant 0 / 1 / 2).
#define MSM_PART_NAME_(prefix, io, ext) prefix##io##_##ext
#define MSM_PART_NAME(prefix, io, ext) MSM_PART_NAME_(prefix, io, ext)
#define MSM_FWD_PART(io, ext) MSM_PART_NAME(launch_fwd_part_, io, ext)
#define MSM_BWD_PART(io, ext) MSM_PART_NAME(launch_bwd_part_, io, ext)
hipError_t launch_fwd_part_0_0(const FwdArgs& a, int K, bool beta0, hipStream_t s);
hipError_t launch_fwd_part_0_1(const FwdArgs& a, int K, bool beta0, hipStream_t s);
hipError_t launch_fwd_part_1_0(const FwdArgs& a, int K, bool beta0, hipStream_t s);
hipError_t launch_fwd_part_1_1(const FwdArgs& a, int K, bool beta0, hipStream_t s);
hipError_t launch_fwd_part_0_2(const FwdArgs& a, int K, bool beta0, hipStream_t s);
hipError_t launch_fwd_part_1_2(const FwdArgs& a, int K, bool beta0, hipStream_t s);
hipError_t launch_bwd_part_0_0(const BwdArgs& a, int K, bool beta0, hipStream_t s);
hipError_t launch_bwd_part_0_1(const BwdArgs& a, int K, bool beta0, hipStream_t s);
hipError_t launch_bwd_part_1_0(const BwdArgs& a, int K, bool beta0, hipStream_t s);
hipError_t launch_bwd_part_1_1(const BwdArgs& a, int K, bool beta0, hipStream_t s);
hipError_t launch_bwd_part_0_2(const BwdArgs& a, int K, bool beta0, hipStream_t s);
hipError_t launch_bwd_part_1_2(const BwdArgs& a, int K, bool beta0, hipStream_t s);
// The 64-state backward (channel blocks of 64, K = 4); launch_bwd calls it for NP == 64.
hipError_t launch_bwd_wide(const BwdArgs& a, int io_bf16, bool beta0, int ext, hipStream_t s);

// Size of the static device scratch behind msm_scan_fwd_noalloc (the chunk summaries of one
// call), and its device address on the current device (looked up on first use per device).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace msm
