// Backward of the momentum selective scan (gfx950): gradients of sum(dy * y).
//
// Adjoints (Momentum Mamba README, "Gradient Flow" and "Gradient Formulas", read with the
// velocity adjoint also collecting the hidden-state adjoint since v_t feeds h_t directly):
//   gh_t = C_t dy_t + a_{t+1} gh_{t+1},     gv_t = gh_t + beta gv_{t+1}
//   dx_t += alpha delta_t B_t gv_t          ddelta_t += alpha B_t x_t gv_t + A a_t h_{t-1} gh_t
//   dA   += delta_t a_t h_{t-1} gh_t        dB_t += alpha delta_t x_t gv_t  (sum over d)
//   dC_t += dy_t h_t  (sum over d)          dx += Dskip dy, dDskip = sum dy x
//
// Work decomposition.  A workgroup owns kBwdChans = 32 channels of one batch row; lane l of a
// wavefront serves channel l % 32 and the two 32-lane halves hold different states, so a
// wavefront keeps 2K states of 32 channels and a workgroup of S wavefronts covers all NP = 2SK
// (padded) states.  Half-width channel blocks double the number of workgroups, which is what
// fills the 256 CUs at the usual training shapes (Bt * D / 32 workgroups).
//   phase 1: forward over the whole sequence, writing the (v, h) state before every tile of
//            TB steps (32 for the plain variant at one state per lane, else 16) to a
//            checkpoint buffer (the recompute strategy of the README's backward notes:
//            reconstruct the forward instead of storing it);
//   phase 2: tiles in reverse order; each tile is recomputed from its checkpoint into
//            registers (h_t and a_t for every step), then swept backwards.
// x, delta, dy and B, C are staged once per workgroup into LDS, one tile ahead (the loads for
// the next tile are issued before the current tile's arithmetic and written to the other LDS
// buffer after it).  The adjoint state and the sums behind dx / ddelta / dA are fp64: ddelta
// is a difference of two large sums, and fp32 adjoints lose too many bits over long sequences.
// Reductions, all in a fixed order so results do not depend on scheduling:
//   over n for dx / ddelta: in-lane over K, across the two halves with v_permlane32_swap,
//     across the S wavefronts through LDS;
//   over d for dB / dC: across the 32 lanes of a half with a reduce-scatter (v_permlane16_swap
//     then DPP), then across channel blocks in a small finalize kernel.
// The fused variant (EXT) differentiates the selective-scan function's extras of the Momentum
// Mamba README ("Low-Level Functions": z, delta_bias, delta_softplus) inside the same sweep:
// delta_eff is re-formed where delta is staged; dy is gated (dy silu(z)) there too, and
// dy silu'(z) and softplus' = logistic(delta + bias) are kept beside it in LDS; the output
// before the gate, needed for dz, is re-formed from the recomputed states (C . h + Dskip x,
// reduced across the state groups like dx); dz and the raw-delta gradient are finished with
// dx / ddelta, and the bias gradient is summed per channel.  Its zero-order-hold form (EXT = 2)
// also carries the write coefficient g = delta phi(delta A) and its derivatives (dg/ddelta =
// e^(delta A), dg/dA = delta^2 psi(delta A)) through dx, ddelta, dA and dB.
// This kernel serves 4, 16 and 32 padded states, and 64 padded states as two launches of its
// 32-state plan (SPLIT below); the full-wavefront backward in msm_bwd_wide.hip takes 64 padded
// states only when those halves would exceed 32-bit offsets.
#include <type_traits>

#include "msm_device.hpp"
#include "msm_internal.h"
#include "msm_lanes.hpp"

namespace msm {
namespace {

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// SPLIT: 0 = all states of the channel in one launch; 1 / 2 = the first / second half of 64
// padded states (states n0 .. n0 + NPB - 1 of the arrays), run as two launches of the 32-state
// plan.  Every gradient is a sum of per-state terms, so the halves' partial sums add up: the
// first launch leaves its dx / ddelta (fp64) and dz (fp32) sums in the workspace and writes no
// bias gradient, the second adds them to its own before storing; the skip term belongs to the
// first launch (the second runs without Dskip).
template <typename IO, int K, int S, bool BETA0, bool HAS_DSKIP, int EXT, int SPLIT>
__global__ __launch_bounds__(S* kWave) void bwd_kernel(const BwdArgs p) {
  using T = io<IO>;
  using raw = typename T::raw;
  constexpr int CB = kBwdChans;          // channels per workgroup
  constexpr int P = kWave / CB;          // state groups per wavefront (2)
  // rows per tile: 32 for the plain variant at one state per lane (its registers and LDS have
  // room: a tile's states, decays and partials), 16 otherwise; the host sizes NT to match.
  // Measured at Bt=4 L=2048 D=2048 N=16 fp32: 0.366 ms against 0.370 ms with 16-row tiles,
  // and half the checkpoint traffic.
  constexpr int TB = bwd_tile_rows(EXT, K, SPLIT);
  // the dx / ddelta partials of 32-row tiles are single-buffered (64 KB at 8 wavefronts), with
  // a barrier between the finalize that reads them and the sweep that rewrites them
  constexpr int SPB = TB > kBwdTile ? 1 : 2;
  constexpr int NTHR = S * kWave;
  constexpr int NPB = S * P * K;         // padded states of the workgroup
  constexpr int GS = S * P;              // state groups of the workgroup
  constexpr int M = 32;                  // values per lane in one dB/dC reduce-scatter
  constexpr int RB = M / (2 * K);        // rows per reduce-scatter
  constexpr int NRB = TB / RB;
  static_assert(P == 2, "the lane pairing below assumes two 32-lane halves");
  constexpr bool ZOH = EXT == 2;  // zero-order-hold write coefficient g = delta phi(delta A)
  // DEF: the sweep keeps per-state sums without the factors every state shares (delta for dx, x
  // for ddelta's write term); the finalize applies them once per (row, channel).  The
  // zero-order hold's sums already carry g and dg/ddelta per state, so it keeps the finished
  // per-lane products.
  constexpr bool DEF = !ZOH;
  static_assert(RB >= 1 && TB % RB == 0, "tile must split into reduce blocks");

  // (delta, delta x), dy and x of each staged element, in three arrays: the recompute reads 8
  // bytes per lane, and the sweep, which reuses those, reads dy alone from a contiguous array
  // (dy read as one half of an 8-byte element touched every other bank, and those reads
  // conflicted: 0.041 conflict cycles per state update against 0.005 with the old 16-byte
  // element).  Odd rows have their channel halves swapped (position ch ^ 16), so the
  // finalize's rows 2g and 2g + 1 read different banks
  __shared__ float2 xs[2][TB][CB];
  __shared__ float gys[2][TB][CB];
  __shared__ float xvs[2][TB][CB];
  __shared__ float bs[2][TB][GS][K];        // alpha B
  __shared__ double cs64[2][TB][GS][K];     // C, widened for the adjoint recurrence
  // fused variant: (dy silu'(z), logistic(delta + bias)) per staged element, the per-wavefront
  // partials of the output before the gate, and the bias-gradient partials
  __shared__ float2 xe[EXT ? 2 : 1][EXT ? TB : 1][CB];
  __shared__ float ypt[EXT ? 2 : 1][EXT ? S : 1][EXT ? TB : 1][CB];
  __shared__ double bred[EXT ? S : 1][EXT ? 2 : 1][CB];
  // Phase 1 stages R1 rows at a time: (delta, delta x) per channel and alpha B per state group,
  // each with its rows contiguous (padded to keep 16-byte reads aligned and spread over the
  // banks).  The sweep's per-wavefront dx (lanes < 32) | ddelta partials reuse that LDS: phase 1
  // ends with a barrier.
  constexpr int TP = (S >= 4 ? 4 * kBwdTile / TB : 1);  // checkpoint tiles per phase-1 step
  constexpr int R1 = TP * TB;
  struct Ph1 {
    float2 xd1[2][CB][R1 + 2];
    float b1[2][GS][R1 * K + 4];
  };
  struct Ph2 {
    float spart[SPB][S][TB][kWave];
  };
  union Ph12 {
    Ph1 f;
    Ph2 r;
  };
  __shared__ __attribute__((aligned(16))) Ph12 ph;
  auto& spart = ph.r.spart;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int g = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int ch = lane & (CB - 1);
  const int gs = g * P + lane / CB;  // state group of this lane
  // position of channel c of staged row t in xs, gys, xvs and xe (odd rows: halves swapped)
  auto swz = [](int t, int c) { return c ^ ((t & 1) * (CB / 2)); };
  const uint32_t bq = blockIdx.x / (uint32_t)p.ncb;
  const int cb = (int)(blockIdx.x - bq * (uint32_t)p.ncb);
  const int64_t b = bq;
  const int64_t L = p.L, D = p.D, N = p.N, NT = p.NT;
  const int d = cb * CB + ch;
  const bool dvalid = d < D;
  const int dl = dvalid ? d : (int)D - 1;
  const float beta = p.beta;
  const double beta64 = p.beta;
  const int n0 = SPLIT ? p.n0 : 0;      // first state of this launch
  const int NPD = SPLIT ? p.NP : NPB;   // states per row of the dB / dC partials

  float A2[K], Af[K], v[K], h[K];
  float invA[EXT == 2 ? K : 1];  // zero-order hold: 1 / A (0 for A = 0 and padded states)
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t n = n0 + (int64_t)gs * K + j;
    const float an = n < N ? p.A[dl * N + n] : 0.f;
    A2[j] = an * kLog2e;
    Af[j] = an;
    if (EXT == 2) invA[EXT == 2 ? j : 0] = an != 0.f ? 1.f / an : 0.f;
    // the forward starts at the given initial state
    const int64_t si = (b * D + dl) * N + n;
    v[j] = (p.v0 && dvalid && n < N) ? p.v0[si] : 0.f;
    h[j] = (p.h0 && dvalid && n < N) ? p.h0[si] : 0.f;
  }
  // fused extras: every x / delta element a thread stages belongs to its lane's channel
  const float dbias = (EXT && p.delta_bias) ? p.delta_bias[dl] : 0.f;
  const bool softplus = EXT && p.delta_softplus != 0;
  const bool has_z = EXT && p.z != nullptr;
  auto delta_eff = [&](float dv) {
    if (!EXT) return dv;
    const float u = dv + dbias;
    return softplus ? softplus_f(u) : u;
  };

  // ---- staging addresses (per-tile buffer resources, constant per-thread offsets) ----
  const int64_t row_bytes = D * T::es, bc_row_bytes = N * T::es;
  const int64_t tot_d = L * row_bytes, tot_n = L * bc_row_bytes;
  const char* x0 = static_cast<const char*>(p.x) + b * tot_d;
  const char* dl0 = static_cast<const char*>(p.delta) + b * tot_d;
  const char* dy0 = static_cast<const char*>(p.dy) + b * tot_d;
  const char* B0 = static_cast<const char*>(p.B) + b * tot_n;
  const char* C0 = static_cast<const char*>(p.C) + b * tot_n;
  const char* z0 = has_z ? static_cast<const char*>(p.z) + b * tot_d : x0;
  // per-tile resources (tile_rsrc) span one tile's rows: 32-bit row indices and extents (the
  // host keeps L below 2^30)
  const int32_t L32 = (int32_t)L;
  // (the clamp compiles to a vector med3: read back as a scalar, or every resource built from it
  // would leave the scalar registers and each buffer access would loop over its lanes' values)
  auto rows_in = [&](int64_t ts, int rmax) {
    return __builtin_amdgcn_readfirstlane(min(max(L32 - (int32_t)ts, 0), rmax));
  };
  auto rows_at = [&](int64_t ts) { return rows_in(ts, TB); };
  const uint32_t rb_d = (uint32_t)row_bytes, rb_n = (uint32_t)bc_row_bytes;

  // x, delta, dy of channels past D are staged as zeros (their offset is past every extent),
  // so those lanes carry zero gradients without further masking
  constexpr int XE = TB * CB;  // elements of one array in one tile
  constexpr int NX = (XE + NTHR - 1) / NTHR;
  uint32_t x_voff[NX];
#pragma unroll
  for (int r = 0; r < NX; ++r) {
    const int i = tid + r * NTHR;
    const int ic = i < XE ? i : XE - 1;
    const int dch = cb * CB + ic % CB;
    x_voff[r] = dch < D ? (uint32_t)((ic / CB) * row_bytes + dch * T::es) : 0x80000000u;
  }
  raw xr[NX], dr[NX], gr[NX], zr[EXT ? NX : 1];
  auto x_load = [&](int64_t ts, bool with_dy) {
    const int32_t t32 = (int32_t)ts, nr = rows_at(ts);
    const auto rx = tile_rsrc(x0, t32, nr, rb_d);
    const auto rd = tile_rsrc(dl0, t32, nr, rb_d);
#pragma unroll
    for (int r = 0; r < NX; ++r) {
      xr[r] = T::bload(rx, x_voff[r], 0u);
      dr[r] = T::bload(rd, x_voff[r], 0u);
    }
    if (with_dy) {
      const auto rg = tile_rsrc(dy0, t32, nr, rb_d);
#pragma unroll
      for (int r = 0; r < NX; ++r) gr[r] = T::bload(rg, x_voff[r], 0u);
    }
    if (EXT) {
      // without a gate the loads read zeros through an empty resource
      const auto rz = tile_rsrc(z0, t32, has_z ? nr : 0, rb_d);
#pragma unroll
      for (int r = 0; r < NX; ++r) zr[r] = T::bload(rz, x_voff[r], 0u);
    }
  };
  auto x_store = [&](int buf, bool with_dy) {
#pragma unroll
    for (int r = 0; r < NX; ++r) {
      const int i = tid + r * NTHR;
      if (NX * NTHR == XE || i < XE) {
        const float xv = T::widen(xr[r]), draw = T::widen(dr[r]);
        const float dv = delta_eff(draw);
        const int xc = swz(i / CB, i % CB);
        float gy = with_dy ? T::widen(gr[r]) : 0.f;
        if (EXT) {
          const float dsp = softplus ? logistic_f(draw + dbias).s : 1.f;
          float gz = 0.f;
          if (has_z) {
            const float zv = T::widen(zr[r]);
            gz = gy * silu_grad_f(zv);
            gy *= silu_f(zv);
          }
          xe[EXT ? buf : 0][EXT ? i / CB : 0][xc] = make_float2(gz, dsp);
        }
        xs[buf][i / CB][xc] = make_float2(dv, dv * xv);
        gys[buf][i / CB][xc] = gy;
        xvs[buf][i / CB][xc] = xv;
      }
    }
  };

  constexpr int BCE = TB * NPB;  // (row, state) pairs of one tile
  constexpr int NPE = (BCE + NTHR - 1) / NTHR;
  uint32_t bc_voff[NPE];
#pragma unroll
  for (int r = 0; r < NPE; ++r) {
    const int i = tid + r * NTHR;
    const int ic = i < BCE ? i : BCE - 1;
    const int n = n0 + ic % NPB;
    bc_voff[r] = n < N ? (uint32_t)(((ic / NPB) * N + n) * T::es) : 0x80000000u;
  }
  raw bre[NPE], cre[NPE];
  auto bc_load = [&](int64_t ts, bool with_c) {
    const int32_t t32 = (int32_t)ts, nr = rows_at(ts);
    const auto rb = tile_rsrc(B0, t32, nr, rb_n);
#pragma unroll
    for (int r = 0; r < NPE; ++r) bre[r] = T::bload(rb, bc_voff[r], 0u);
    if (with_c) {
      const auto rc = tile_rsrc(C0, t32, nr, rb_n);
#pragma unroll
      for (int r = 0; r < NPE; ++r) cre[r] = T::bload(rc, bc_voff[r], 0u);
    }
  };
  auto bc_store = [&](int buf, bool with_c) {
#pragma unroll
    for (int r = 0; r < NPE; ++r) {
      const int i = tid + r * NTHR;
      if (NPE * NTHR == BCE || i < BCE) {
        const int tt = i / NPB, n = i % NPB;
        bs[buf][tt][n / K][n % K] = T::widen(bre[r]) * p.alpha;
        if (with_c) cs64[buf][tt][n / K][n % K] = T::widen(cre[r]);
      }
    }
  };
  // checkpoints, [Bt][NT][2][N][D] fp32: one buffer resource per (b, tile) and constant
  // per-lane offsets; lanes without a state (channel past D, padded n) get an offset past
  // the extent, so their stores are dropped and their loads read zero
  const int64_t ck_tile_bytes = 2 * N * D * 4;
  uint32_t ck_voff[2][K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t n = n0 + (int64_t)gs * K + j;
#pragma unroll
    for (int w = 0; w < 2; ++w)
      ck_voff[w][j] = (dvalid && n < N) ? (uint32_t)(((w * N + n) * D + d) * 4) : 0x80000000u;
  }
  const char* ck_b = reinterpret_cast<const char*>(p.ckpt) + b * NT * ck_tile_bytes;
  const uint32_t ck_tb = (uint32_t)ck_tile_bytes;
  auto ck_rsrc = [&](int64_t tile) {
    return make_rsrc_u32(ck_b + (uint64_t)(uint32_t)tile * ck_tb, ck_tb);
  };

  // one forward step of the K states (recurrence only); c = delta * x, or x with the
  // zero-order hold, whose write is x B g.  That variant also hands out g = delta phi(delta A)
  // and dg/dA of the step for the reverse sweep (g_out / gA_out).
  auto fstep = [&](float dv, float c, const float* bb, float* a_out, float* h_out,
                   float* g_out = nullptr, float* gA_out = nullptr) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float arg = dv * A2[j];
      const float a = exp2_fast(arg);
      float w = c * bb[j];
      if (ZOH) {
        const float gz = zoh_g_bwd(arg, a, dv, invA[ZOH ? j : 0]);
        w *= gz;
        if (g_out) {
          g_out[j] = gz;
          gA_out[j] = zoh_gA_bwd(arg, a, dv, invA[ZOH ? j : 0], gz);
        }
      }
      v[j] = BETA0 ? w : fmaf(beta, v[j], w);
      h[j] = fmaf(a, h[j], v[j]);
      if (a_out) a_out[j] = a;
      if (h_out) h_out[j] = h[j];
    }
  };

  // ---------------- phase 1: forward over the whole sequence, checkpoint every tile ----
  // Steps of R1 rows (TP checkpoint tiles): one barrier and one set of resources per step.
  // The loads of step k + 2 are issued at the start of step k into one of two register sets
  // (the one step k's data was staged from) and staged into LDS at the end of step k + 1.  The
  // first step is staged before the loop, and every step of the loop computes: steps past the
  // end read zeros, advance a state nothing reads afterwards and drop their checkpoint stores
  // (no memory operation depends on a branch, so the compiler counts the loads in flight
  // exactly).
  {
    constexpr int XE1 = R1 * CB, NX1 = (XE1 + NTHR - 1) / NTHR;
    constexpr int BE1 = R1 * NPB, NB1 = (BE1 + NTHR - 1) / NTHR;
    uint32_t x1_voff[NX1], b1_voff[NB1];
#pragma unroll
    for (int r = 0; r < NX1; ++r) {
      const int i = tid + r * NTHR;
      const int ic = i < XE1 ? i : XE1 - 1;
      const int dch = cb * CB + ic % CB;
      x1_voff[r] = dch < D ? (uint32_t)((ic / CB) * row_bytes + dch * T::es) : 0x80000000u;
    }
#pragma unroll
    for (int r = 0; r < NB1; ++r) {
      const int i = tid + r * NTHR;
      const int ic = i < BE1 ? i : BE1 - 1;
      const int n = n0 + ic % NPB;
      b1_voff[r] = n < N ? (uint32_t)(((ic / NPB) * N + n) * T::es) : 0x80000000u;
    }
    struct Set {
      raw x[NX1], d[NX1], b[NB1];
    };
    Set s0{}, s1{};
    auto load1 = [&](Set& st, int64_t k) {
      const int64_t ts = k * R1;
      const int32_t t32 = (int32_t)ts, nr = rows_in(ts, R1);
      const auto rx = tile_rsrc(x0, t32, nr, rb_d);
      const auto rd = tile_rsrc(dl0, t32, nr, rb_d);
      const auto rb = tile_rsrc(B0, t32, nr, rb_n);
#pragma unroll
      for (int r = 0; r < NX1; ++r) {
        st.x[r] = T::bload(rx, x1_voff[r], 0u);
        st.d[r] = T::bload(rd, x1_voff[r], 0u);
      }
#pragma unroll
      for (int r = 0; r < NB1; ++r) st.b[r] = T::bload(rb, b1_voff[r], 0u);
    };
    // The forward here reads only (delta, delta x) and alpha B, so it stages them in their own
    // layout: a channel's steps contiguous ((delta, delta x) of two steps per 16-byte read) and
    // a state group's steps contiguous (alpha B of 4 / K steps per 16-byte read).  That is 12
    // bytes per lane and step against 20 through the sweep's layout, which kept this loop
    // waiting on LDS bandwidth.
    auto store1 = [&](const Set& st, int buf) {
#pragma unroll
      for (int r = 0; r < NX1; ++r) {
        const int i = tid + r * NTHR;
        if (NX1 * NTHR == XE1 || i < XE1) {
          const float xv = T::widen(st.x[r]), dv = delta_eff(T::widen(st.d[r]));
          ph.f.xd1[buf][i % CB][i / CB] = make_float2(dv, ZOH ? xv : dv * xv);
        }
      }
#pragma unroll
      for (int r = 0; r < NB1; ++r) {
        const int i = tid + r * NTHR;
        if (NB1 * NTHR == BE1 || i < BE1) {
          const int n = i % NPB;
          ph.f.b1[buf][n / K][(i / NPB) * K + n % K] = T::widen(st.b[r]) * p.alpha;
        }
      }
    };
    // step k: refill `ld` with step k + 2, checkpoint and compute the TP tiles of step k, stage
    // step k + 1 from `st` into the other LDS buffer
    auto step1 = [&](int64_t k, Set& ld, const Set& st) {
      load1(ld, k + 2);
      const int buf = (int)(k & 1);
#pragma unroll
      for (int q = 0; q < TP; ++q) {
        const int64_t tile = k * TP + q;
        {
          // tiles past the last one store through an empty resource (dropped)
          const auto rc = tile < NT ? ck_rsrc(tile) : make_rsrc(p.ckpt, 0);
#pragma unroll
          for (int j = 0; j < K; ++j) {
            io<float>::bstore(rc, ck_voff[0][j], 0u, v[j]);
            io<float>::bstore(rc, ck_voff[1][j], 0u, h[j]);
          }
        }
        float4 dd[TB / 2], bq[TB * K / 4];
#pragma unroll
        for (int i = 0; i < TB / 2; ++i)
          dd[i] = *reinterpret_cast<const float4*>(&ph.f.xd1[buf][ch][q * TB + 2 * i]);
#pragma unroll
        for (int i = 0; i < TB * K / 4; ++i)
          bq[i] = *reinterpret_cast<const float4*>(&ph.f.b1[buf][gs][q * TB * K + 4 * i]);
        const float* bf = reinterpret_cast<const float*>(bq);
#pragma unroll
        for (int tt = 0; tt < TB; ++tt) {
          const float4 r = dd[tt / 2];
          fstep((tt & 1) ? r.z : r.x, (tt & 1) ? r.w : r.y, bf + tt * K, nullptr, nullptr);
        }
      }
      store1(st, (int)((k + 1) & 1));
      __syncthreads();
    };
    const int64_t NS = (NT + TP - 1) / TP;  // phase-1 steps
    load1(s0, 0);
    load1(s1, 1);
    store1(s0, 0);
    __syncthreads();
    // pairs of steps so the two register sets alternate without copies; one loop exit
    for (int64_t k = 0; k < NS; k += 2) {
      step1(k, s0, s1);
      step1(k + 1, s1, s0);
    }
  }

  // ---------------- phase 2: reverse sweep ----------------
  // The adjoint recurrence (gh, gv) runs in fp64: fp32 adjoints lose too many bits over long
  // sequences for ddelta, a difference of two large sums.  Products that leave the
  // recurrence are rounded to fp32; dA is summed in fp32 within a tile and in fp64 across.
  double ghn[K], gvp[K], dA64[K];  // ghn = a_{t+1} gh_{t+1}, gvp = gv_{t+1}
#pragma unroll
  for (int j = 0; j < K; ++j) {
    ghn[j] = 0.0;
    gvp[j] = 0.0;
    dA64[j] = 0.0;
  }
  double dD64 = 0.0;
  double dbias64 = 0.0;  // fused variant: this lane's rows of the bias gradient (lanes >= 32)
  // (the zero-order-hold variant always runs with the skip term compiled in, a zero weight
  // when no Dskip is given; see launch_ks)
  // (added in the finalize, by every lane, or in the sweep by state group 0)
  const float dsk = (HAS_DSKIP && (DEF || gs == 0) && p.Dskip) ? p.Dskip[dl] : 0.f;
  const float* dbc = p.dbc_part + (b * p.ncb + cb) * L * 2 * NPD;
  char* dx0 = static_cast<char*>(p.dx) + b * tot_d;
  char* ddl0 = static_cast<char*>(p.ddelta) + b * tot_d;
  const uint32_t lane_off = (uint32_t)dl * T::es;

  // dx / ddelta of the rows of `tile`, whose partials sit in spart[pb]: each wavefront takes
  // every S-th row and adds the S partials of its lane in a fixed order (fp64), rounding once.
  // Lanes 0-31 hold dx and lanes 32-63 ddelta; both stores are issued by every lane, and the
  // lanes that must not write (other half, channels past D) carry an offset past every
  // extent, which the buffer unit drops.  (A per-lane choice of buffer would make the
  // compiler loop over the distinct descriptors.)
  const uint32_t vo_dx = (dvalid && lane < CB) ? lane_off : 0x80000000u;
  const uint32_t vo_dd = (dvalid && lane >= CB) ? lane_off : 0x80000000u;
  // fused variant: dz of the row comes from lanes 0-31 as well
  char* dz0 = (EXT && p.dz) ? static_cast<char*>(p.dz) + b * tot_d : dx0;
  const uint32_t vo_dz = (dvalid && lane < CB) ? lane_off : 0x80000000u;
  // split passes: per-lane offsets into the first half's sums
  const int64_t aq_row_bytes = 2 * D * 8, aq_tot = L * aq_row_bytes;
  char* aq0 = SPLIT ? reinterpret_cast<char*>(p.acc_q) + b * aq_tot : dx0;
  char* az0 = SPLIT ? reinterpret_cast<char*>(p.acc_dz) + b * L * D * 4 : dx0;
  const uint32_t vo_aq = dvalid ? (uint32_t)(((lane >= CB ? 1 : 0) * D + dl) * 8) : 0x80000000u;
  const uint32_t vo_dz32 = (dvalid && lane < CB) ? (uint32_t)dl * 4u : 0x80000000u;
  // DEF finalize: every lane stores both outputs of its element (dx, ddelta, dz; and in the
  // split passes its fp64 sums at [row][0][d] and [row][1][d], and dz at [row][d])
  const uint32_t vo_c = dvalid ? lane_off : 0x80000000u;
  const uint32_t vo_q = dvalid ? (uint32_t)dl * 8u : 0x80000000u;
  const uint32_t q_dd = (uint32_t)(D * 8);
  const uint32_t vo_z = dvalid ? (uint32_t)dl * 4u : 0x80000000u;
  // xb: the LDS staging buffer that still holds the tile's inputs
  auto finalize = [&](int64_t tile, int pb, bool valid, int xb) __attribute__((always_inline)) {
    const int64_t ts = tile * TB;
    // an invalid tile gets empty resources: every store below is then dropped
    const int32_t t32 = valid ? (int32_t)ts : 0, nr = valid ? rows_at(ts) : 0;
    const auto rdx = tile_rsrc(dx0, t32, nr, rb_d);
    const auto rdd = tile_rsrc(ddl0, t32, nr, rb_d);
    const auto rdz = tile_rsrc(dz0, t32, has_z ? nr : 0, rb_d);
    // split passes: the first half's sums, [L][2][D] fp64 (dx, ddelta) and [L][D] fp32 (dz)
    const auto raq = tile_rsrc(aq0, t32, SPLIT ? nr : 0, (uint32_t)aq_row_bytes);
    const auto raz = tile_rsrc(az0, t32, (SPLIT && has_z) ? nr : 0, (uint32_t)(D * 4));
    if constexpr (DEF) {
      // Lane l finishes channel l % 32 of row tt = r 2S + 2g + l / 32: from the S wavefronts'
      // sums S1 = sum(B gv) and S2 = sum(A a h gh) (written by lanes l % 32 and l % 32 + 32,
      // at positions l and l ^ 32 of the row, as odd rows are stored with the halves swapped)
      // it forms dx = delta S1 + Dskip dy and ddelta = x S1 + S2 in fp64, and stores both.
      // Every partial is read before the first sum, so the reads share one LDS round trip.
      constexpr int FR2 = TB / (2 * S);
      const int hf = lane / CB;
      float sp[FR2][2][S];
      float yp[EXT ? FR2 : 1][EXT ? S : 1];
#pragma unroll
      for (int r = 0; r < FR2; ++r) {
        const int tt = r * 2 * S + 2 * g + hf;
#pragma unroll
        for (int w = 0; w < S; ++w) {
          sp[r][0][w] = spart[SPB == 2 ? pb : 0][w][tt][lane];
          sp[r][1][w] = spart[SPB == 2 ? pb : 0][w][tt][lane ^ CB];
          if (EXT) yp[EXT ? r : 0][EXT ? w : 0] = ypt[EXT ? pb : 0][EXT ? w : 0][EXT ? tt : 0][ch];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < FR2; ++r) {
        const int tt = r * 2 * S + 2 * g + hf;
        double s1 = (double)sp[r][0][0], s2 = (double)sp[r][1][0];
#pragma unroll
        for (int w = 1; w < S; ++w) {
          s1 += (double)sp[r][0][w];
          s2 += (double)sp[r][1][w];
        }
        const int xc = swz(tt, ch);
        const float dv = xs[xb][tt][xc].x;
        const float2 gx = make_float2(gys[xb][tt][xc], xvs[xb][tt][xc]);  // dy, x
        double qdx = (double)dv * s1;
        double qdd = fma((double)gx.y, s1, s2);
        if (HAS_DSKIP) qdx = fma((double)dsk, (double)gx.x, qdx);
        float zv = 0.f;
        if (EXT) {
          // the raw delta's gradient (through softplus) and dz from the output before the gate
          const float2 e = xe[EXT ? xb : 0][EXT ? tt : 0][xc];
          qdd *= (double)e.y;
          float yr = yp[EXT ? r : 0][0];
#pragma unroll
          for (int w = 1; w < S; ++w) yr += yp[EXT ? r : 0][EXT ? w : 0];
          if (HAS_DSKIP) yr = fmaf(dsk, gx.y, yr);
          zv = e.x * yr;
        }
        // rows past the end of the sequence are past the extent: dropped
        const uint32_t ro = vo_c + (uint32_t)(tt * row_bytes);
        if constexpr (SPLIT != 0) {
          // split passes: the first stores its fp64 sums, the second adds them
          const uint32_t aqo = vo_q + (uint32_t)(tt * aq_row_bytes);
          const uint32_t azo = vo_z + (uint32_t)(tt * D * 4);
          if constexpr (SPLIT == 1) {
            const uint64_t ux = (uint64_t)__double_as_longlong(qdx);
            const uint64_t ud = (uint64_t)__double_as_longlong(qdd);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{(uint32_t)ux, (uint32_t)(ux >> 32)},
                                                  raq, aqo, 0u, 0);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{(uint32_t)ud, (uint32_t)(ud >> 32)},
                                                  raq, aqo + q_dd, 0u, 0);
            if (EXT) io<float>::bstore(raz, azo, 0u, zv);
            continue;
          } else {
            const u32x2_t wx = __builtin_amdgcn_raw_buffer_load_b64(raq, aqo, 0u, 0);
            const u32x2_t wd = __builtin_amdgcn_raw_buffer_load_b64(raq, aqo + q_dd, 0u, 0);
            qdx += __longlong_as_double((long long)(((uint64_t)wx.y << 32) | wx.x));
            qdd += __longlong_as_double((long long)(((uint64_t)wd.y << 32) | wd.x));
            if (EXT) zv += io<float>::bload(raz, azo, 0u);
          }
        }
        T::bstore(rdx, ro, 0u, (float)qdx);
        T::bstore(rdd, ro, 0u, (float)qdd);
        if (EXT) {
          if (valid) dbias64 += qdd;
          T::bstore(rdz, ro, 0u, zv);
        }
      }
    } else {
    // zero-order hold: lanes 0-31 finish dx and lanes 32-63 ddelta of every S-th row.  Every
    // partial of the wavefront's rows is read before the first sum, so the reads share one LDS
    // round trip (summed as they arrive, the compiler waits on each in turn)
    constexpr int FR = (TB + S - 1) / S;  // rows finished by this wavefront
    float sp[FR][S];
#pragma unroll
    for (int r = 0; r < FR; ++r) {
      const int tt = r * S + g < TB ? r * S + g : TB - 1;
#pragma unroll
      for (int w = 0; w < S; ++w) sp[r][w] = spart[SPB == 2 ? pb : 0][w][tt][lane];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tr0 = 0; tr0 < TB; tr0 += S) {
      const int tt = tr0 + g;
      if (tr0 + S <= TB || tt < TB) {
        double q = (double)sp[tr0 / S][0];
#pragma unroll
        for (int w = 1; w < S; ++w) q += (double)sp[tr0 / S][w];
        // rows past the end of the sequence are past the extent: dropped
        const uint32_t ro = (uint32_t)(tt * row_bytes);
        if constexpr (SPLIT == 0) {
          T::bstore(rdx, vo_dx + ro, 0u, (float)q);
          if (EXT) {
            // lanes 32-63: the gradient of the raw delta (through softplus); lanes 0-31: dz from
            // the output before the gate, summed over the S wavefronts in a fixed order
            const float2 e = xe[EXT ? xb : 0][EXT ? tt : 0][swz(tt, ch)];
            const double qd = q * (double)e.y;
            if (valid) dbias64 += qd;
            T::bstore(rdd, vo_dd + ro, 0u, (float)qd);
            float yr = ypt[EXT ? pb : 0][0][EXT ? tt : 0][ch];
#pragma unroll
            for (int w = 1; w < S; ++w) yr += ypt[EXT ? pb : 0][EXT ? w : 0][EXT ? tt : 0][ch];
            T::bstore(rdz, vo_dz + ro, 0u, e.x * yr);
          } else {
            T::bstore(rdd, vo_dd + ro, 0u, (float)q);
          }
        } else {
          // split passes: lanes 0-31 carry dx, lanes 32-63 ddelta (the raw delta's, through
          // softplus, when fused); the first pass stores its sums, the second adds them
          const uint32_t aqo = vo_aq + (uint32_t)(tt * aq_row_bytes);
          const uint32_t azo = vo_dz32 + (uint32_t)(tt * D * 4);
          double val = q;
          float2 e = make_float2(0.f, 0.f);
          if (EXT) {
            e = xe[EXT ? xb : 0][EXT ? tt : 0][swz(tt, ch)];
            if (lane >= CB) val = q * (double)e.y;
          }
          if (SPLIT == 2) {
            const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(raq, aqo, 0u, 0);
            val += __longlong_as_double((long long)(((uint64_t)w.y << 32) | w.x));
          }
          if (SPLIT == 1) {
            const uint64_t u = (uint64_t)__double_as_longlong(val);
            const u32x2_t w = {(uint32_t)u, (uint32_t)(u >> 32)};
            __builtin_amdgcn_raw_buffer_store_b64(w, raq, aqo, 0u, 0);
          } else {
            T::bstore(rdx, vo_dx + ro, 0u, (float)val);
            T::bstore(rdd, vo_dd + ro, 0u, (float)val);
            if (EXT && valid && lane >= CB) dbias64 += val;
          }
          if (EXT) {
            float yr = ypt[EXT ? pb : 0][0][EXT ? tt : 0][ch];
#pragma unroll
            for (int w = 1; w < S; ++w) yr += ypt[EXT ? pb : 0][EXT ? w : 0][EXT ? tt : 0][ch];
            float zv = e.x * yr;
            if (SPLIT == 2) zv += io<float>::bload(raz, azo, 0u);
            if (SPLIT == 1)
              io<float>::bstore(raz, azo, 0u, zv);
            else
              T::bstore(rdz, vo_dz + ro, 0u, zv);
          }
        }
      }
    }
    }
  };

  // dB / dC partials of this workgroup, [L][2][NPB] fp32 at dbc: a resource per tile and a
  // constant offset per lane and reduce block (lane l of a half holds value l & 31)
  const int64_t dbc_row_bytes = 2 * NPD * 4;
  uint32_t dbc_voff[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int m = lane & 31;
    const int tt = rb * RB + m / (2 * K);
    const int n = gs * K + m % K;
    dbc_voff[rb] = (uint32_t)((tt * 2 * NPD + ((m / K) & 1) * NPD + n0 + n) * 4);
  }

  auto load_ckpt = [&](float(&ov)[K], float(&oh)[K], int64_t tile) {
    const auto rc = ck_rsrc(tile);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      ov[j] = io<float>::bload(rc, ck_voff[0][j], 0u);
      oh[j] = io<float>::bload(rc, ck_voff[1][j], 0u);
    }
  };

  // one step of the reverse sweep: prefetch tile - 1 (its checkpoint into `nv_`/`nh_`, its
  // inputs into registers), recompute and sweep `tile` (if it exists) from LDS, finish the
  // dx / ddelta of tile + 1, stage tile - 1 into the other LDS buffer.  Loads, stores and the
  // barrier are unconditional, so every step has the same memory pattern.
  // rows of the last tile: the terminal adjoints enter at its row nlast - 1 (the rows after
  // it are past the end of the sequence and keep the adjoint state at zero)
  const int nlast = (int)(L - (NT - 1) * TB);
  // `first` (std::true_type for the step of tile NT-1 only) compiles the terminal-adjoint
  // injection into that step alone
  auto step2 = [&](auto first, int64_t tile, const float(&cv)[K], const float(&chh)[K],
                   float(&nv_)[K], float(&nh_)[K]) {
    constexpr bool FIRST = decltype(first)::value;
    const bool live = tile >= 0;
    // adjoints of the final state, loaded in the first step only
    double dlh[K], dlv[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t n = n0 + (int64_t)gs * K + j;
      const int64_t si = (b * D + dl) * N + n;
      dlh[j] = (FIRST && p.dlast_h && dvalid && n < N) ? (double)p.dlast_h[si] : 0.0;
      dlv[j] = (FIRST && p.dlast_v && dvalid && n < N) ? (double)p.dlast_v[si] : 0.0;
    }
    const int buf = (int)((NT - 1 - tile) & 1);
    const int pb = (int)(tile & 1);
    const int64_t tp = tile > 0 ? tile - 1 : 0;  // prefetch (tile 0 again at the end)
    load_ckpt(nv_, nh_, tp);
    bc_load(tp * TB, true);
    x_load(tp * TB, true);
    // tile + 1's partials were completed before the last barrier
    finalize(tile + 1, pb ^ 1, tile + 1 < NT && tile + 1 >= 0, buf ^ 1);
    // single-buffered partials: every wavefront has read them before the sweep rewrites them
    // (this also orders the finalize's reads of the staging buffer before its refill below)
    if constexpr (SPB == 1) __syncthreads();

    // The sweep runs in every step (a step past tile 0 sweeps stale LDS data): its stores are
    // dropped through an empty resource and its sums are not kept.  No memory operation
    // depends on a branch, so the compiler can count the loads still in flight exactly.
    const int64_t ts = tile * TB;
    const auto rdbc = tile_rsrc(dbc, live ? (int32_t)ts : 0, live ? rows_at(ts) : 0,
                                (uint32_t)dbc_row_bytes);
    // recompute the tile from its checkpoint: hs[tt] = h_{ts+tt-1}, av[tt] = a_{ts+tt} (and for
    // the zero-order hold g and dg/dA of each step in phs, pss)
    float hs[TB + 1][K], av[TB][K];
    float phs[ZOH ? TB : 1][K], pss[ZOH ? TB : 1][K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      v[j] = cv[j];
      h[j] = chh[j];
      hs[0][j] = h[j];
    }
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) {
      const int xc = swz(tt, ch);
      const float2 r = xs[buf][tt][xc];
      fstep(r.x, ZOH ? xvs[buf][tt][xc] : r.y, &bs[buf][tt][gs][0], av[tt], hs[tt + 1],
            ZOH ? phs[ZOH ? tt : 0] : nullptr, ZOH ? pss[ZOH ? tt : 0] : nullptr);
    }

    float dAt[K];
#pragma unroll
    for (int j = 0; j < K; ++j) dAt[j] = 0.f;
    float dDt = 0.f;
#pragma unroll
    for (int rb = NRB - 1; rb >= 0; --rb) {
      float vals[M];
#pragma unroll
      for (int tb = RB - 1; tb >= 0; --tb) {
        const int tt = rb * RB + tb;
        const int xc = swz(tt, ch);
        const float2 r0 = xs[buf][tt][xc];
        const float dv = r0.x, c = r0.y, gy = gys[buf][tt][xc], xv = xvs[buf][tt][xc];
        const double gy64 = gy;
        float p1 = 0.f, p2 = 0.f, yq = 0.f, p1d = 0.f;
#pragma unroll
        for (int j = 0; j < K; ++j) {
          if (EXT) yq = fmaf((float)cs64[buf][tt][gs][j], hs[tt + 1][j], yq);
          if (FIRST && tt == nlast - 1) ghn[j] = dlh[j];
          const double gh = fma(cs64[buf][tt][gs][j], gy64, ghn[j]);
          double gv = BETA0 ? gh : fma(beta64, gvp[j], gh);
          if (FIRST && tt == nlast - 1) gv += dlv[j];
          ghn[j] = (double)av[tt][j] * gh;
          if (!BETA0) gvp[j] = gv;
          const float gvf = (float)gv;
          const float gg = (float)ghn[j] * hs[tt][j];  // a_t h_{t-1} gh_t
          p2 = j == 0 ? Af[j] * gg : fmaf(Af[j], gg, p2);
          dAt[j] = fmaf(dv, gg, dAt[j]);
          if (!ZOH) {
            p1 = j == 0 ? bs[buf][tt][gs][j] * gvf : fmaf(bs[buf][tt][gs][j], gvf, p1);
            vals[(tb * 2 + 0) * K + j] = c * gvf;             // dB / alpha
          } else {
            // write x B g: dx and dB take g, ddelta's write part dg/ddelta = a, and dA gains
            // alpha B x gv dg/dA (phs: g, pss: dg/dA of the step)
            const float a = av[tt][j];
            const float gz = phs[ZOH ? tt : 0][j];
            const float bg = bs[buf][tt][gs][j] * gvf;  // alpha B gv
            p1 = j == 0 ? bg * gz : fmaf(bg, gz, p1);
            p1d = j == 0 ? bg * a : fmaf(bg, a, p1d);
            dAt[j] = fmaf(bg * xv, pss[ZOH ? tt : 0][j], dAt[j]);
            vals[(tb * 2 + 0) * K + j] = xv * gz * gvf;       // dB / alpha
          }
          vals[(tb * 2 + 1) * K + j] = gy * hs[tt + 1][j];  // dC
        }
        float qx = p1, qd = p2;  // DEF: sums over the lane's states, finished in the finalize
        if (HAS_DSKIP) dDt = fmaf(gy, xv, dDt);
        if constexpr (!DEF) {
          // zero-order hold: g already carries delta; the skip term on state group 0
          if (HAS_DSKIP) qx = fmaf(dsk, gy, qx);
          qd = fmaf(xv, p1d, p2);
        }
        // (DEF: odd rows with the halves swapped, so the finalize's two rows per wavefront
        // fall in different LDS banks)
        spart[SPB == 2 ? pb : 0][g][tt][DEF ? (lane ^ ((tt & 1) * CB)) : lane] = swap_add32(qx, qd);
        if (EXT) {
          // the output before the gate: this lane's states (+ the skip term on group 0 with
          // the zero-order hold; the finalize adds it otherwise), then both halves
          if (!DEF && HAS_DSKIP) yq = fmaf(dsk, xv, yq);
          const float ys = swap_add32(yq, yq);
          if (lane < CB) ypt[EXT ? pb : 0][EXT ? g : 0][EXT ? tt : 0][lane] = ys;
        }
        // the zero-order hold's extra per-row values would otherwise be interleaved across rows
        // by the scheduler and overflow the registers
        if (ZOH) __builtin_amdgcn_sched_barrier(0);
      }
      reduce_scatter32(vals, lane);
      // rows past the end of the sequence are past the extent: dropped
      io<float>::bstore(rdbc, dbc_voff[rb], 0u, vals[0]);
    }
    if (live) {
#pragma unroll
      for (int j = 0; j < K; ++j) dA64[j] += (double)dAt[j];
      if (HAS_DSKIP) dD64 += (double)dDt;
    }
    // after step 0 the adjoint carries are the adjoints of the initial state:
    // dh0 = a_0 gh_0, dv0 = beta gv_0 (stores under this branch happen once per workgroup)
    if (tile == 0 && dvalid) {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int64_t n = n0 + (int64_t)gs * K + j;
        const int64_t si = (b * D + d) * N + n;
        if (n < N && p.dh0) p.dh0[si] = (float)ghn[j];
        if (n < N && p.dv0) p.dv0[si] = BETA0 ? 0.f : (float)(beta64 * gvp[j]);
      }
    }
    // the finalize above read xs, gys, xvs (and in the fused variants xe) [buf ^ 1], which the
    // staging below refills: every wavefront must be past those reads first
    if constexpr (SPB == 2) __syncthreads();
    bc_store(buf ^ 1, true);
    x_store(buf ^ 1, true);
    __syncthreads();
  };

  float ckv0[K], ckh0[K], ckv1[K], ckh1[K];
  load_ckpt(ckv0, ckh0, NT - 1);
  bc_load((NT - 1) * TB, true);
  x_load((NT - 1) * TB, true);
  bc_store(0, true);
  x_store(0, true);
  __syncthreads();
  // tile NT-1, then tiles NT-2 .. 0 and tile -1 (finishes tile 0) in pairs so the checkpoint
  // registers alternate instead of being copied; a possible extra step (tile -2) only loads
  step2(std::true_type{}, NT - 1, ckv0, ckh0, ckv1, ckh1);
  for (int64_t t = NT - 2; t >= -1; t -= 2) {
    step2(std::false_type{}, t, ckv1, ckh1, ckv0, ckh0);
    step2(std::false_type{}, t - 1, ckv0, ckh0, ckv1, ckh1);
  }

  if (dvalid) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t n = n0 + (int64_t)gs * K + j;
      if (n < N) p.dA_part[(b * N + n) * D + d] = (float)dA64[j];
    }
    if (HAS_DSKIP && gs == 0 && p.Dskip) p.dD_part[b * D + d] = (float)dD64;
  }
  if (EXT && SPLIT != 1 && p.delta_bias) {
    // the bias gradient of the channel: lanes 32-63 of every wavefront hold their rows' sum
    // (DEF: both halves hold rows of the channel; otherwise lanes 32-63 hold them all)
    if (DEF)
      bred[EXT ? g : 0][EXT ? lane / CB : 0][ch] = dbias64;
    else if (lane >= CB)
      bred[EXT ? g : 0][0][ch] = dbias64;
    __syncthreads();
    if (g == 0 && lane < CB && dvalid) {
      double t = bred[0][0][ch];
      if (DEF) t += bred[0][EXT ? 1 : 0][ch];
#pragma unroll
      for (int w = 1; w < S; ++w) {
        t += bred[EXT ? w : 0][0][ch];
        if (DEF) t += bred[EXT ? w : 0][EXT ? 1 : 0][ch];
      }
      p.dbias_part[b * D + d] = (float)t;
    }
  }
}

template <typename IO, int K, int S, bool BETA0, int EXT, int SPLIT = 0>
hipError_t launch_ks(const BwdArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.ncb * a.Bt)), block(S * kWave);
  // The zero-order-hold variant takes the skip-term build even without Dskip (weight zero, its
  // partials left unread): the compiler schedules that build with far fewer spills (measured
  // at Bt=4, L=2048, D=2048, N=16, fp32: 1.16 ms against 2.24 ms without the skip term).
  if constexpr (EXT == 2) {
    hipLaunchKernelGGL((bwd_kernel<IO, K, S, BETA0, true, EXT, SPLIT>), grid, block, 0, s, a);
  } else {
    if (a.Dskip)
      hipLaunchKernelGGL((bwd_kernel<IO, K, S, BETA0, true, EXT, SPLIT>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((bwd_kernel<IO, K, S, BETA0, false, EXT, SPLIT>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <typename IO, bool BETA0, int EXT>
hipError_t launch_io(const BwdArgs& a, int K, hipStream_t s) {
  switch (a.NP * 100 + K) {
    // S = NP / (2K) wavefronts per workgroup
    case 401: return launch_ks<IO, 1, 2, BETA0, EXT>(a, s);
    case 402: return launch_ks<IO, 2, 1, BETA0, EXT>(a, s);
    case 1601: return launch_ks<IO, 1, 8, BETA0, EXT>(a, s);
    case 1602: return launch_ks<IO, 2, 4, BETA0, EXT>(a, s);
    case 1604: return launch_ks<IO, 4, 2, BETA0, EXT>(a, s);
    case 3202: return launch_ks<IO, 2, 8, BETA0, EXT>(a, s);
    // 64 padded states as two halves of the 32-state plan (a.split_pass 1, then 2)
    case 6402:
      return a.split_pass == 1 ? launch_ks<IO, 2, 8, BETA0, EXT, 1>(a, s)
                               : launch_ks<IO, 2, 8, BETA0, EXT, 2>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// This file is compiled once per (I/O dtype, variant) pair; MSM_IO_BF16 and MSM_EXT select
// which launcher a build of it defines.
#if !defined(MSM_IO_BF16) || !defined(MSM_EXT)
#error "compile with -DMSM_IO_BF16=0|1 -DMSM_EXT=0|1|2"
#endif
#if MSM_IO_BF16
using PartIO = bf16_storage;
#else
using PartIO = float;
#endif

hipError_t MSM_BWD_PART(MSM_IO_BF16, MSM_EXT)(const BwdArgs& a, int K, bool beta0, hipStream_t s) {
  return beta0 ? launch_io<PartIO, true, MSM_EXT>(a, K, s)
               : launch_io<PartIO, false, MSM_EXT>(a, K, s);
}

}  // namespace msm
