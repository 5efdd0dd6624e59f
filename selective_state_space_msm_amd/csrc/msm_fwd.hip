// Forward selective scan with momentum (gfx950).
//
// Recurrence (Momentum Mamba README, "Momentum Mamba Recurrence"), per (b, d, n):
//   v_t = beta v_{t-1} + alpha delta_t B_t x_t,  h_t = exp(delta_t A) h_{t-1} + v_t,
//   y_t = sum_n C_t h_t (+ Dskip x_t).
// Each step is the affine map (v, h) -> ([[beta, 0], [beta, a_t]] (v, h) + (w_t, w_t)); maps
// compose associatively, which is what lets the sequence be cut into chunks (the chunked
// scan with a running prefix of the README's kernel notes; the inter-chunk scan over chunk
// states of the Mamba-2 page's four-step algorithm).
//
// Work decomposition (one 64-lane wavefront = 64 consecutive channels x K states):
//   * lane = channel d, so every x/delta/y access of a wavefront is one contiguous row;
//   * the K states of a channel live in registers; a workgroup holds S = NP/K wavefronts that
//     own disjoint state groups of the same 64 channels (NP = padded state count);
//   * B_t and C_t are the same for all channels, so each workgroup stages a tile of kTile steps
//     of them in LDS (fp32, B pre-multiplied by alpha) and every lane reads them as broadcasts;
//   * the per-wavefront partial sums of y_t = C_t . h_t are added across the S wavefronts in
//     LDS in a fixed order (deterministic), one barrier per tile when double-buffered;
//   * unchunked plans use a half-wavefront layout instead (HW below): 32 channels per
//     workgroup, the two lane halves on different state groups, 32-row tiles;
//   * time runs sequentially inside a lane.  When the channel count alone cannot fill the
//     GPU the sequence is cut into G chunks: a summary pass maps every chunk but the last to
//     its affine map from a zero start (bv, bh, q and the sum of delta), and the main pass
//     composes the maps of the preceding chunks in its prologue to get its exact start state.
//
// The fused variant (EXT) adds the selective-scan function's extras of the Momentum Mamba
// README ("Low-Level Functions": z, delta_bias, delta_softplus) at no extra pass over memory:
// delta_eff = softplus(delta + bias[d]) (or delta + bias[d]) is formed where delta is staged,
// once per workgroup, and the output is multiplied by silu(z) where it is stored; z is loaded
// with x and delta and stays in registers until its tile's y is stored.
// The zero-order-hold variant (EXT = 2) also replaces the write coefficient delta by
// (e^(delta A) - 1) / A = delta phi(delta A) (the exact discretisation of the glossary and
// complextorch pages), at a few more instructions per state update.
//
// The y reduction never needs MFMA: the scan is a per-element recurrence bound by VALU issue
// (one v_exp_f32 plus five fp32 multiply/FMA per state update), not a dense contraction.
#include "msm_device.hpp"
#include "msm_internal.h"

namespace msm {
namespace {

// Occupancy hint: the launch plans put one or two wavefronts on a SIMD, so the scheduler may
// spend registers on hiding LDS and transcendental latency instead of on more wavefronts.
// HW (half-wavefront layout, main pass only): a workgroup owns 32 channels; lane l serves
// channel l % 32 and the two 32-lane halves of a wavefront hold different state groups, so a
// workgroup of S wavefronts covers 2 S K states with half the wavefronts of the full layout.
// The grid then has twice the workgroups, two of them share a CU, and each keeps its own
// barrier schedule: while one workgroup stages its next tile and finishes y, the other one's
// wavefronts on the same SIMDs are still computing.
template <typename IO, int K, int S, bool BETA0, bool SUMMARY, bool HAS_DSKIP, int EXT, int YBP,
          bool HW>
__global__ __launch_bounds__(S* kWave) __attribute__((amdgpu_waves_per_eu(1, K >= 8 ? 1 : 2)))
void fwd_kernel(const FwdArgs p) {
  static_assert(!(HW && SUMMARY), "the summaries keep the full-wavefront layout");
  using T = io<IO>;
  using raw = typename T::raw;
  // rows per LDS tile: 32 in the half-wavefront layout, whose workgroups have LDS to spare
  // (Bt=4 L=4096 D=4096 bf16: 0.319 ms against 0.336 ms with 16-row tiles, both with
  // 4-row read batches)
  constexpr int TT = HW ? 2 * kTile : kTile;
  constexpr int BCW = 2 * K;                    // floats per (tile row, state group): B then C
  constexpr int NTHR = S * kWave;
  constexpr int CW = HW ? kWave / 2 : kWave;    // channels per workgroup
  constexpr int PG = kWave / CW;                // state groups per wavefront
  constexpr int GS = S * PG;                    // state groups per workgroup
  constexpr int RPF = NTHR / CW;                // rows one finalize round covers
  static_assert(TT % RPF == 0, "the finalize rounds must tile the LDS tile");
  constexpr bool YPART = !SUMMARY && GS > 1;
  // y partials are double-buffered (one barrier per tile) when one workgroup per CU is all
  // the grid provides (YBP = 2).  With more workgroups than CUs (YBP = 1), and always with 16
  // wavefronts, they are single-buffered and take a second barrier: the smaller LDS lets two
  // workgroups share a CU (measured at Bt=1, L=65536, D=2048, N=16 in 16 chunks: 1.13 ms
  // single-buffered, 1.27 ms double-buffered; at Bt=4, L=4096, D=4096: 0.366 ms double,
  // 0.388 ms single)
  // (the half-wavefront layout single-buffers its 32-row tiles: 56 KB of LDS per workgroup,
  // so two share a CU)
  constexpr int YB = HW ? 1 : ((S >= 16 || YBP == 1) ? 1 : 2);

  __shared__ float bcs[2][TT][GS][BCW];
  __shared__ float ypart[YPART ? YB : 1][YPART ? GS : 1][TT][CW];
  // (delta, delta * x) of the tile, widened once per workgroup: the S wavefronts share them
  __shared__ float2 xdl[2][TT][CW];
  __shared__ float xxl[HAS_DSKIP ? 2 : 1][HAS_DSKIP ? TT : 1][CW];  // x, for the skip term

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int g = tid / kWave;
  const int ch = lane & (CW - 1);          // channel within the workgroup's block
  const int gs = g * PG + lane / CW;       // state group of this lane
  // Half-wavefront layout: workgroups dispatch to the eight XCDs in turn, so within each
  // group of 16 the two halves of a 64-channel block are given indices 8 apart (one XCD, one
  // L2 for their shared cache lines).
  const uint32_t ncbk = HW ? (uint32_t)p.ncb_hw : (uint32_t)p.ncb;
  uint32_t bid = blockIdx.x;
  if (HW && bid < (gridDim.x & ~15u)) bid = (bid & ~15u) | ((bid & 7u) << 1) | ((bid >> 3) & 1u);
  const uint32_t blk = bid / ncbk;
  const int cb = (int)(bid - blk * ncbk);
  const int64_t b = blk % (uint32_t)p.Bt;
  const int k = (int)(blk / (uint32_t)p.Bt);
  const int64_t L = p.L, D = p.D, N = p.N;
  int64_t t0 = (int64_t)k * p.Tc;
  const int64_t t1 = (t0 + p.Tc < L) ? t0 + p.Tc : L;
  const int d = cb * CW + ch;
  const bool dvalid = d < D;
  const int dl = dvalid ? d : (int)D - 1;
  const float beta = p.beta;

  float A2[K], v[K], h[K], q[K];
  float invA[EXT == 2 ? K : 1];  // zero-order hold: 1 / A (0 for A = 0 and padded states)
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t n = (int64_t)gs * K + j;
    const float an = n < N ? p.A[dl * N + n] : 0.f;
    A2[j] = an * kLog2e;
    if (EXT == 2) invA[EXT == 2 ? j : 0] = an != 0.f ? 1.f / an : 0.f;
    // the scan starts at the given state; chunk summaries are maps from a zero start
    const int64_t si = (b * D + dl) * N + n;
    v[j] = (!SUMMARY && p.v0 && n < N) ? p.v0[si] : 0.f;
    h[j] = (!SUMMARY && p.h0 && n < N) ? p.h0[si] : 0.f;
    q[j] = 0.f;
  }
  float sd = 0.f, bpow = 1.f;
  const float dsk = (HAS_DSKIP && gs == 0) ? p.Dskip[dl] : 0.f;
  // fused extras: every x / delta element a thread stages belongs to its lane's channel
  constexpr bool ZG = EXT && !SUMMARY;  // the gate is loaded (the summaries produce no y)
  constexpr bool ZOH = EXT == 2;        // zero-order-hold write coefficient
  const float dbias = (EXT && p.delta_bias) ? p.delta_bias[dl] : 0.f;
  const bool softplus = EXT && p.delta_softplus != 0;
  const bool has_z = ZG && p.z != nullptr;

  if (!SUMMARY && k > 0) {
    // Exact start state of this chunk: apply the maps of chunks 0..k-1 in order to the
    // initial state.
    for (int kk = 0; kk < k; ++kk) {
      const int64_t base = b * p.G + kk;
      const float sdv = p.s_sd[base * D + dl];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int64_t n = (int64_t)gs * K + j;
        if (n < N) {
          const int64_t idx = (base * N + n) * D + dl;
          const float r = exp2_fast(A2[j] * sdv);     // product of a_t over the chunk
          float hn = fmaf(r, h[j], p.s_bh[idx]);
          if (!BETA0) {
            hn = fmaf(p.s_q[idx], v[j], hn);
            v[j] = fmaf(p.beta_pow_tc, v[j], p.s_bv[idx]);
          }
          h[j] = hn;
        }
      }
    }
  }

  // ---- summaries: the window of the chunk that decides its end state ----
  // A chunk's end state is its map applied to the start state plus the part written inside
  // it.  The start state's share shrinks by prod a_t = 2^(A2 sum delta) for h and beta^rows for
  // v, so once both fall below 2^-kWinLog2 over the chunk's last rows, those rows alone give the
  // end state: everything written before them, and the start state, reach the end scaled by
  // less than 2^-kWinLog2 (relative to their size there).  The window is found by summing
  // delta backwards from the chunk end, a tile at a time, until every channel of the workgroup
  // meets the bound for its slowest state (and at least win_rows rows for beta).  A truncated
  // summary then maps any start state to zero: q = 0 and sum delta = +inf (r = 0).
  // Each wavefront also finds the window of its own K states (their slowest decay): before it
  // the wavefront only adds up delta (the chunk's decay sum), so fast-decaying states cost less
  // than the workgroup's slowest one.  A wavefront whose window starts after the chunk start
  // reports its states' maps as truncated (q = 0); their decay over the whole chunk is below
  // 2^-kWinLog2 as well.
  bool trunc = false;
  const int64_t tc0 = t0;  // the chunk's first row
  int64_t wg0 = t0;        // this wavefront's window start
  if (SUMMARY && p.win_rows < t1 - t0) {
    float amin = INFINITY;  // slowest decay of this lane's channel, |A| log2 e
    for (int64_t n = 0; n < N; ++n) amin = fminf(amin, -p.A[dl * N + n] * kLog2e);
    float amin_w = INFINITY;  // the same over this wavefront's states
#pragma unroll
    for (int j = 0; j < K; ++j)
      if ((int64_t)gs * K + j < N) amin_w = fminf(amin_w, -A2[j]);
    bool wdone = false;
    // channels past D only repeat channel D - 1
    const uint32_t rb = (uint32_t)(D * T::es);
    const auto rdw = make_rsrc(static_cast<const char*>(p.delta) + (b * L + t0) * D * T::es,
                               (t1 - t0) * D * T::es);
    float acc = 0.f;
    // a state that does not decay (A >= 0) needs the whole chunk: no search
    int64_t w0 = __syncthreads_and(amin > 0.f) ? t1 : t0;
    while (w0 > t0) {
      // rows 2g, 2g + 1 of the tile ending at w0, channel dl, summed over the S wavefronts
      const int64_t tb = w0 - kTile;
      float part = 0.f;
      for (int r = 2 * g; r < kTile; r += 2 * S) {
        const uint32_t o0 = (uint32_t)((tb - t0 + r) * rb + (int64_t)dl * T::es);
        float d0 = T::widen(T::bload(rdw, o0, 0u)), d1 = T::widen(T::bload(rdw, o0 + rb, 0u));
        if (EXT) {
          const float u0 = d0 + dbias, u1 = d1 + dbias;
          d0 = softplus ? softplus_f(u0) : u0;
          d1 = softplus ? softplus_f(u1) : u1;
        }
        part += d0 + d1;
      }
      xdl[0][g][ch].x = part;
      __syncthreads();
      for (int gg = 0; gg < S; ++gg) acc += xdl[0][gg][ch].x;
      w0 = tb;
      if (!wdone && __all(amin_w * acc >= kWinLog2 && t1 - w0 >= p.win_rows)) {
        wdone = true;
        wg0 = w0;
      }
      const bool mine = amin * acc >= kWinLog2 && t1 - w0 >= p.win_rows;
      __syncthreads();  // every wavefront has read the partial sums before they are rewritten
      if (__syncthreads_and(mine)) {
        trunc = w0 > t0;
        t0 = w0;
        break;
      }
    }
    // (when the workgroup's bound holds, every wavefront's does: amin <= amin_w)
    if (!wdone) wg0 = t0;
  }

  // ---- addressing ----
  // Every global access goes through a buffer resource whose base is this chunk's first row
  // and whose extent ends at its last row; a tile adds its row offset to constant per-lane
  // offsets (one vector add per offset register), clamped so that a tile past the chunk end
  // starts at the extent.  Rows past the chunk end therefore read as zero and touch no memory.
  // That is what makes the prefetch unconditional (an uneven number of loads on different
  // paths would make the in-order vmcnt waits of the current tile drain the prefetch of the
  // next one).  Offsets are 32-bit: the host keeps every chunk below 2^31 bytes per array and
  // rows below 2^26 bytes, so a clamped tile's offsets stay below 2^32.
  const uint32_t lane_off = (uint32_t)dl * T::es;
  const uint32_t row_bytes = (uint32_t)(D * T::es);
  const uint32_t bc_row_bytes = (uint32_t)(N * T::es);
  const uint32_t chunk_rows = (uint32_t)(t1 - t0);
  const uint32_t ext_d = chunk_rows * row_bytes, ext_n = chunk_rows * bc_row_bytes;
  const char* x0 = static_cast<const char*>(p.x) + (b * L + t0) * D * T::es;
  const char* dl0 = static_cast<const char*>(p.delta) + (b * L + t0) * D * T::es;
  char* y0 = static_cast<char*>(p.y) + (b * L + t0) * D * T::es;
  const char* B0 = static_cast<const char*>(p.B) + (b * L + t0) * N * T::es;
  const char* C0 = static_cast<const char*>(p.C) + (b * L + t0) * N * T::es;
  // without a gate its loads go through an empty resource (they read zeros, touch no memory)
  const char* z0 = has_z ? static_cast<const char*>(p.z) + (b * L + t0) * D * T::es : x0;
  const uint32_t ext_z = has_z ? ext_d : 0u;
  const auto rsx = make_rsrc_u32(x0, ext_d), rsdl = make_rsrc_u32(dl0, ext_d);
  const auto rsy = make_rsrc_u32(y0, ext_d), rsz = make_rsrc_u32(z0, ext_z);
  const auto rsb = make_rsrc_u32(B0, ext_n), rsc = make_rsrc_u32(C0, ext_n);
  // first row of the tile starting at ts, relative to the chunk, clamped to the chunk end
  auto trow = [&](int64_t ts) -> uint32_t {
    const int64_t r = ts - t0;
    return __builtin_amdgcn_readfirstlane((uint32_t)(r < (int64_t)chunk_rows ? r : chunk_rows));
  };
  // y offsets: channels past D store at an offset past every extent (dropped)
  constexpr uint32_t kDrop = 0xFFFFFF00u;

  // ---- B/C staging: global (I/O dtype) -> registers -> LDS (fp32) ----
  // Element (tt, n) of a tile; both B and C are loaded for it.
  constexpr int BCE = TT * GS * K;                      // (tt, n) elements per tile
  constexpr int NPE = (BCE + NTHR - 1) / NTHR;
  uint32_t bc_voff[NPE];
  bool bc_nok[NPE];
#pragma unroll
  for (int r = 0; r < NPE; ++r) {
    const int i = tid + r * NTHR;
    const int ic = i < BCE ? i : BCE - 1;
    const int n = ic % (GS * K);
    bc_nok[r] = n < N;
    bc_voff[r] = (uint32_t)(((ic / (GS * K)) * N + (n < N ? n : 0)) * T::es);
  }
  // The inputs of one tile as this thread stages them (a few elements of B, C, x and delta).
  // Loads run two tiles ahead of the arithmetic through a ring of three such sets.
  constexpr int XE = TT * CW;
  constexpr int NX = (XE + NTHR - 1) / NTHR;
  // z[r] is the gate of row r * RPF + tid / CW, channel tid % CW of the tile: the same
  // (row, channel) this thread stores y for, so the gate never goes through LDS
  struct Set {
    raw b[NPE], c[NPE], x[NX], d[NX], z[ZG ? NX : 1];
  };
  auto stage_load = [&](Set& st, int64_t ts) {
    const uint32_t ob = trow(ts) * bc_row_bytes;
#pragma unroll
    for (int r = 0; r < NPE; ++r) {
      st.b[r] = T::bload(rsb, bc_voff[r] + ob, 0u);
      st.c[r] = T::bload(rsc, bc_voff[r] + ob, 0u);
    }
  };
  auto stage_store = [&](const Set& st, int buf) {
#pragma unroll
    for (int r = 0; r < NPE; ++r) {
      const int i = tid + r * NTHR;
      if (i < BCE) {
        const int tt = i / (GS * K);
        const int n = i % (GS * K);
        float* dst = &bcs[buf][tt][n / K][0];
        dst[n % K] = bc_nok[r] ? T::widen(st.b[r]) * p.alpha : 0.f;
        dst[K + n % K] = bc_nok[r] ? T::widen(st.c[r]) : 0.f;
      }
    }
  };
  // x / delta staging: element (row, channel) i of a tile goes through thread i mod NTHR; the
  // values are widened and delta * x formed once here, then every wavefront reads them from
  // LDS.  Channels past D read channel D - 1 (their lanes' results are never stored).
  uint32_t x_voff[NX];
#pragma unroll
  for (int r = 0; r < NX; ++r) {
    const int i = tid + r * NTHR;
    const int ic = i < XE ? i : XE - 1;
    const int dch = cb * CW + ic % CW;
    x_voff[r] = (uint32_t)((ic / CW) * row_bytes + (dch < D ? dch : (int)D - 1) * T::es);
  }
  auto load_xd = [&](Set& st, int64_t ts) {
    const uint32_t od = trow(ts) * row_bytes;
#pragma unroll
    for (int r = 0; r < NX; ++r) {
      st.x[r] = T::bload(rsx, x_voff[r] + od, 0u);
      st.d[r] = T::bload(rsdl, x_voff[r] + od, 0u);
    }
    if (ZG) {
#pragma unroll
      for (int r = 0; r < NX; ++r) st.z[r] = T::bload(rsz, x_voff[r] + od, 0u);
    }
  };
  auto store_xd = [&](const Set& st, int buf) {
#pragma unroll
    for (int r = 0; r < NX; ++r) {
      const int i = tid + r * NTHR;
      if (NX * NTHR == XE || i < XE) {
        const float xv = T::widen(st.x[r]), dv = T::widen(st.d[r]);
        if (EXT) {
          const float u = dv + dbias;
          const float de = softplus ? softplus_f(u) : u;
          xdl[buf][i / CW][i % CW] = make_float2(de, ZOH ? xv : de * xv);
        } else {
          xdl[buf][i / CW][i % CW] = make_float2(dv, T::mul_raw(st.d[r], st.x[r]));
        }
        if (HAS_DSKIP) xxl[HAS_DSKIP ? buf : 0][HAS_DSKIP ? i / CW : 0][i % CW] = xv;
      }
    }
  };
  auto load_set = [&](Set& st, int64_t ts) {
    stage_load(st, ts);
    load_xd(st, ts);
  };
  auto store_set = [&](const Set& st, int buf) {
    stage_store(st, buf);
    store_xd(st, buf);
  };

  // One time step for the K states of this lane.  bc holds [B(K) | C(K)] of that step.
  auto step = [&](float xv, float dv, float c, const float* bc) -> float {
    float ysum = HAS_DSKIP ? dsk * xv : 0.f;
    if (SUMMARY) bpow *= beta;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float arg = dv * A2[j];
      const float a = exp2_fast(arg);
      // the write: c B with c = delta x, or with the zero-order hold x B g (c = x staged) for
      // g = delta phi(delta A)
      float w = c * bc[j];
      if (ZOH) w *= zoh_g_fwd(arg, a, dv, invA[ZOH ? j : 0]);
      if (BETA0)
        v[j] = w;
      else
        v[j] = fmaf(beta, v[j], w);
      h[j] = fmaf(a, h[j], v[j]);
      if (SUMMARY) {
        if (!BETA0) q[j] = fmaf(a, q[j], bpow);
      } else {
        ysum = fmaf(bc[K + j], h[j], ysum);
      }
    }
    if (SUMMARY) sd += dv;
    return ysum;
  };
  // y stores are never under a branch (a store the compiler cannot count makes its waits for
  // the prefetched inputs drain more than they need): channels past D carry an offset past
  // every extent, and rows past the chunk end lie past the resource's extent, so the buffer
  // unit drops both.
  auto yoff = [&](uint32_t tr, int tt) -> uint32_t {
    return dvalid ? (tr + (uint32_t)tt) * row_bytes + lane_off : kDrop;
  };
  // the finalize's rows of this thread (tid / CW + r RPF): their offsets within a tile are
  // constants, so a tile adds its scalar row offset (one add and one select per store)
  constexpr int FR = TT / RPF;
  uint32_t fin_off[YPART ? FR : 1];
#pragma unroll
  for (int r = 0; r < (YPART ? FR : 1); ++r)
    fin_off[r] = (uint32_t)(r * RPF + tid / CW) * row_bytes + lane_off;
  auto gate = [&](float y, raw zr) { return (ZG && has_z) ? y * silu_f(T::widen(zr)) : y; };
  // tr: first row of the tile being computed; cur: its inputs (only used when GS == 1)
  auto emit = [&](int buf, int tt, uint32_t tr, float ysum, const Set& cur) {
    if (SUMMARY) return;
    if (GS == 1) {
      T::bstore(rsy, yoff(tr, tt), 0u, gate(ysum, cur.z[ZG ? tt : 0]));
    } else {
      ypart[YPART && YB == 2 ? buf : 0][YPART ? gs : 0][tt][ch] = ysum;
    }
  };
  // Full tile.  The B/C broadcasts of the next batch of RB steps are read from LDS into
  // registers before the current batch is computed; the scheduling barrier keeps the compiler
  // from sinking those reads next to their uses, where their latency would be exposed.
  // Batches of 2 steps: measured at N=16, 2 states per wavefront, Bt=4 L=4096 D=4096 bf16
  // (half-wavefront layout, 32-row tiles): 0.301 ms, against 0.305 ms with 1 step, 0.319 ms
  // with 4 and 0.357 ms with 8; Bt=1 L=65536 D=2048 in 16 chunks (full layout): 0.719 ms
  // against 0.772 ms with 4.
  constexpr int RB = 2;
  constexpr int NB = TT / RB;
  auto compute_tile = [&](int buf, int64_t ts, const Set& cur) {
    if (SUMMARY && ts < wg0) {
      // before this wavefront's window: only the chunk's delta sum
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) sd += xdl[buf][tt][ch].x;
      return;
    }
    const uint32_t ry = trow(ts);
    float bcv[2][RB][BCW];
    float2 dcv[2][RB];
    auto read_batch = [&](float(&dst)[RB][BCW], float2(&dd)[RB], int jb) {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const float* src = &bcs[buf][jb * RB + i][gs][0];
#pragma unroll
        for (int e = 0; e < BCW; ++e) dst[i][e] = src[e];
        dd[i] = xdl[buf][jb * RB + i][ch];
      }
    };
    read_batch(bcv[0], dcv[0], 0);
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
      if (jb + 1 < NB) read_batch(bcv[(jb + 1) & 1], dcv[(jb + 1) & 1], jb + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int tt = jb * RB + i;
        const float xv = HAS_DSKIP ? xxl[HAS_DSKIP ? buf : 0][HAS_DSKIP ? tt : 0][ch] : 0.f;
        const float ysum = step(xv, dcv[jb & 1][i].x, dcv[jb & 1][i].y, bcv[jb & 1][i]);
        emit(buf, tt, ry, ysum, cur);
      }
    }
  };
  // The ragged last tile of a chunk (nv < TT rows), once per chunk after the main loop: rows
  // past nv must leave the state alone, so each row is guarded (a uniform branch).
  auto compute_tail = [&](int buf, int64_t ts, int nv, const Set& cur) {
    const uint32_t ry = trow(ts);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if (tt < nv) {
        const float2 dc = xdl[buf][tt][ch];
        const float xv = HAS_DSKIP ? xxl[HAS_DSKIP ? buf : 0][HAS_DSKIP ? tt : 0][ch] : 0.f;
        const float ysum = step(xv, dc.x, dc.y, &bcs[buf][tt][gs][0]);
        emit(buf, tt, ry, ysum, cur);
      }
    }
  };
  // y of the tile whose partials are in ypart[buf]: thread tid takes rows tid / CW, + RPF, ...
  // of channel tid % CW (its own lane's channel), adds the GS partials in a fixed order and
  // stores, a fixed number of stores per wavefront.
  auto finalize = [&](int buf, int64_t ts, const Set& cur) {
    if (!YPART) return;
    const uint32_t rbytes = __builtin_amdgcn_readfirstlane(trow(ts) * row_bytes);
#pragma unroll
    for (int r = 0; r < FR; ++r) {
      const int tt = r * RPF + tid / CW;
      float s = ypart[YPART && YB == 2 ? buf : 0][0][tt][ch];
#pragma unroll
      for (int gg = 1; gg < GS; ++gg) s += ypart[YPART && YB == 2 ? buf : 0][YPART ? gg : 0][tt][ch];
      const uint32_t o = dvalid ? rbytes + fin_off[YPART ? r : 0] : kDrop;
      T::bstore(rsy, o, 0u, gate(s, cur.z[ZG ? r : 0]));
    }
  };

  // ---- main loop: the full tiles of the chunk, then the ragged tail, in steps of three ----
  const int64_t nfull = (t1 - t0) / TT;
  const int nrem = (int)((t1 - t0) - nfull * TT);
  const int64_t ntile = nfull + (nrem > 0 ? 1 : 0);
  Set sa, sb, sc;
  load_set(sa, t0);
  load_set(sb, t0 + TT);
  store_set(sa, 0);
  __syncthreads();

  // One step: issue the loads of tile k + 2, compute tile k (if it exists) from LDS, stage
  // tile k + 1 into the other LDS buffer, one barrier, store tile k's y.  `cur` still holds
  // tile k's inputs (its gate, in the fused variant).  No memory operation
  // depends on a branch (the compute issues none when there are y partials): past the chunk
  // end the loads read zeros, the staged buffer goes unused and the y stores are dropped.
  auto stepk = [&](int64_t k, Set& ld, const Set& st, const Set& cur) {
    const int64_t ts = t0 + k * TT;
    const int buf = (int)(k & 1);
    load_set(ld, ts + 2 * TT);
    if (k < nfull)
      compute_tile(buf, ts, cur);
    else if (k == nfull && nrem > 0)
      compute_tail(buf, ts, nrem, cur);
    // staging and the y finalize run at the highest wave priority: where two workgroups share a
    // SIMD, the one nearing its barriers gets the issue slots first (Bt=4 L=4096 D=4096 bf16:
    // 0.292 ms against 0.299 ms at priority 0 and 0.294 ms at 2; Bt=1 L=65536 D=2048 in 16
    // chunks: 0.720 against 0.732 ms)
    __builtin_amdgcn_s_setprio(3);
    store_set(st, buf ^ 1);
    __syncthreads();
    finalize(buf, ts, cur);
    if (YPART && YB == 1) __syncthreads();  // partials read before the next tile rewrites them
    __builtin_amdgcn_s_setprio(0);
  };
  // groups of three steps so the three register sets rotate without copies; one loop exit
  for (int64_t k = 0; k < ntile; k += 3) {
    stepk(k, sc, sb, sa);
    stepk(k + 1, sa, sc, sb);
    stepk(k + 2, sb, sa, sc);
  }

  if (SUMMARY) {
    if (dvalid) {
      const int64_t base = b * p.G + k;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int64_t n = (int64_t)gs * K + j;
        if (n < N) {
          const int64_t idx = (base * N + n) * D + d;
          p.s_bh[idx] = h[j];
          if (!BETA0) {
            p.s_bv[idx] = v[j];
            p.s_q[idx] = wg0 > tc0 ? 0.f : q[j];
          }
        }
      }
      if (g == 0) p.s_sd[base * D + d] = trunc ? INFINITY : sd;
    }
  } else if (k == p.G - 1 && dvalid) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t n = (int64_t)gs * K + j;
      if (n < N) {
        if (p.last_h) p.last_h[(b * D + d) * N + n] = h[j];
        if (p.last_v) p.last_v[(b * D + d) * N + n] = v[j];
      }
    }
  }
}

template <typename IO, int K, int S, bool BETA0, int EXT, int YBP, bool HW>
void launch_main(const FwdArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.Dskip)
    hipLaunchKernelGGL((fwd_kernel<IO, K, S, BETA0, false, true, EXT, YBP, HW>), grid, block, 0,
                       s, a);
  else
    hipLaunchKernelGGL((fwd_kernel<IO, K, S, BETA0, false, false, EXT, YBP, HW>), grid, block, 0,
                       s, a);
}

// SH: wavefronts per workgroup of the half-wavefront layout for this (NP, K), 0 if it has none
template <typename IO, int K, int S, bool BETA0, int EXT, int SH = 0>
hipError_t launch_ks(const FwdArgs& a, hipStream_t s) {
  const dim3 block(S * kWave);
  if (a.G > 1) {
    const dim3 grid((unsigned)(a.ncb * a.Bt * (a.G - 1)));
    hipLaunchKernelGGL((fwd_kernel<IO, K, S, BETA0, true, false, EXT, 1, false>), grid, block, 0,
                       s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if constexpr (SH > 0) {
    if (a.half_wave) {
      const dim3 grid((unsigned)(a.ncb_hw * a.Bt * a.G));
      launch_main<IO, K, SH, BETA0, EXT, 2, true>(a, grid, dim3(SH * kWave), s);
      return hipGetLastError();
    }
  }
  const dim3 grid((unsigned)(a.ncb * a.Bt * a.G));
  // single-buffered y partials when the grid has more workgroups than the GPU has CUs
  if constexpr (S >= 16) {
    launch_main<IO, K, S, BETA0, EXT, 1, false>(a, grid, block, s);
  } else {
    if ((int64_t)grid.x > a.cus)
      launch_main<IO, K, S, BETA0, EXT, 1, false>(a, grid, block, s);
    else
      launch_main<IO, K, S, BETA0, EXT, 2, false>(a, grid, block, s);
  }
  return hipGetLastError();
}

template <typename IO, bool BETA0, int EXT>
hipError_t launch_io(const FwdArgs& a, int K, hipStream_t s) {
  // padded state count NP = K * S is 4, 16, 32 or 64
  const int NP = a.N <= 4 ? 4 : (a.N <= 16 ? 16 : (a.N <= 32 ? 32 : 64));
  switch (NP * 100 + K) {
    case 401: return launch_ks<IO, 1, 4, BETA0, EXT>(a, s);
    case 402: return launch_ks<IO, 2, 2, BETA0, EXT>(a, s);
    case 404: return launch_ks<IO, 4, 1, BETA0, EXT>(a, s);
    case 1601: return launch_ks<IO, 1, 16, BETA0, EXT>(a, s);
    case 1602: return launch_ks<IO, 2, 8, BETA0, EXT, 4>(a, s);
    case 1604: return launch_ks<IO, 4, 4, BETA0, EXT, 2>(a, s);
    case 1608: return launch_ks<IO, 8, 2, BETA0, EXT>(a, s);
    case 1616: return launch_ks<IO, 16, 1, BETA0, EXT>(a, s);
    case 3204: return launch_ks<IO, 4, 8, BETA0, EXT>(a, s);
    case 3208: return launch_ks<IO, 8, 4, BETA0, EXT>(a, s);
    case 6404: return launch_ks<IO, 4, 16, BETA0, EXT>(a, s);
    case 6408: return launch_ks<IO, 8, 8, BETA0, EXT>(a, s);
    case 6416: return launch_ks<IO, 16, 4, BETA0, EXT>(a, s);
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

hipError_t MSM_FWD_PART(MSM_IO_BF16, MSM_EXT)(const FwdArgs& a, int K, bool beta0, hipStream_t s) {
  return beta0 ? launch_io<PartIO, true, MSM_EXT>(a, K, s)
               : launch_io<PartIO, false, MSM_EXT>(a, K, s);
}

}  // namespace msm
