// Forward of the complex-valued momentum scan (gfx950).
//
// Recurrence (Momentum Mamba README, "Complex Number Support": A, B and C complex, x, delta and
// y real; complextorch, "The diagonal SSM", for the complex diagonal state), per (b, d, n):
//   a_t = exp(delta_t A) = 2^(delta_t Re A log2 e) (cos + i sin)(delta_t Im A)
//   v_t = beta v_{t-1} + alpha delta_t x_t B_t,  h_t = a_t h_{t-1} + v_t
//   y_t = Re(sum_n C_t h_t) (+ Dskip x_t)
//
// Work decomposition (the backward's half-wavefront layout): a workgroup owns kBwdChans = 32
// channels of one batch row; lane l of wavefront g serves channel l % 32 and state group
// 2 g + l / 32, which holds K consecutive states in registers, so S wavefronts cover
// NP = 2 S K padded states.  32-channel blocks give Bt * D / 32 workgroups, which fills the
// 256 CUs at the usual training shapes without cutting the sequence into chunks.
//   * B_t, C_t (alpha B and C, widened to fp32) and (delta, delta x, x) are staged per tile of
//     kTile steps in LDS, one tile ahead: the loads of tile k + 1 are issued before tile k is
//     computed and written to the other LDS buffer after it;
//   * the readout sum over n: in-lane over K, across the two halves with v_permlane32_swap,
//     then across the S wavefronts through LDS in a fixed order (double-buffered partials,
//     one barrier per tile);
//   * the rotation e^(i delta Im A) comes from a 64-entry LDS table and short Taylor series
//     after an exact reduction of the phase in revolutions (cis_delta_tab), its modulus from
//     v_exp_f32.
// The recording pass (REC) writes h_t for every step to a history buffer laid out
// [b][t + 1][n][d] (row 0 = the initial state), which the backward reads instead of
// recomputing the forward; it produces no y.  It runs the recurrence in fp64 (a_t from an fp64
// exponential and rotation, fp64 states, alpha delta x B formed in fp64) and rounds each state
// to fp32 once, for the history.
#include "msm_complex.hpp"
#include "msm_internal.h"

namespace msm {
namespace {

template <typename IO, int K, int S, bool HAS_DSKIP, bool REC>
__global__ __launch_bounds__(S* kWave) void cfwd_kernel(const CFwdArgs p) {
  using T = io<IO>;
  using CT = cio<IO>;
  using raw = typename T::raw;
  using craw = typename CT::raw;
  constexpr int TT = kTile;
  constexpr int CB = kBwdChans;
  constexpr int NTHR = S * kWave;
  constexpr int NP = 2 * S * K;
  constexpr bool Y = !REC;
  constexpr int BCE = TT * NP;  // (row, state) elements of B / C per tile
  constexpr int NBC = (BCE + NTHR - 1) / NTHR;
  constexpr int XE = TT * CB;   // (row, channel) elements of x / delta per tile
  constexpr int NX = (XE + NTHR - 1) / NTHR;
  constexpr bool DSK = Y && HAS_DSKIP;

  __shared__ float4 bcs[2][TT][NP];  // alpha B (re, im), C (re, im)
  __shared__ float2 xdl[2][TT][CB];  // delta, delta * x
  __shared__ float xxl[DSK ? 2 : 1][DSK ? TT : 1][CB];
  __shared__ float ypart[Y ? 2 : 1][Y ? S : 1][TT][CB];
  __shared__ CTab ctab;  // fp64 exponential and rotation tables (recording pass)
  __shared__ float2 ctabf[64];  // fp32 rotation table (readout pass)

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int g = tid / kWave;
  const int c = lane & (CB - 1);
  const int gi = 2 * g + (lane >> 5);
  const int64_t b = blockIdx.x / (uint32_t)p.ncb;
  const int cb = (int)(blockIdx.x - b * (uint32_t)p.ncb);
  const int64_t L = p.L, D = p.D, N = p.N;
  const int64_t d = (int64_t)cb * CB + c;
  const bool dvalid = d < D;
  const int64_t dl = dvalid ? d : D - 1;
  const float beta = p.beta;

  // fp32 state for the readout pass, fp64 state for the recording pass (whose history feeds
  // the delta gradient, where fp32 rounding of a_t, compounded over the memory of the state
  // and multiplied by |A|, exceeds the fp32 tolerance)
  float Ar[K], hr[K], hi[K], vr[K], vi[K];
  RevPair Ai[K];
  double ArD[K], AiD[K], hdr[K], hdi[K], vdr[K], vdi[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t n = (int64_t)gi * K + j;
    const bool on = n < N;
    const int64_t ai = (dl * N + (on ? n : 0)) * 2;
    const float are = on ? p.A[ai] : 0.f, aim = on ? p.A[ai + 1] : 0.f;
    Ar[j] = are * kLog2e;  // padding states: a = 1, B = C = 0, h = v = 0
    Ai[j] = to_revolutions(aim);
    ArD[j] = are;
    AiD[j] = (double)aim / kTwoPiD;
    const int64_t si = ((b * D + dl) * N + (on ? n : 0)) * 2;
    hr[j] = (on && p.h0) ? p.h0[si] : 0.f;
    hi[j] = (on && p.h0) ? p.h0[si + 1] : 0.f;
    vr[j] = (on && p.v0) ? p.v0[si] : 0.f;
    vi[j] = (on && p.v0) ? p.v0[si + 1] : 0.f;
    hdr[j] = hr[j];
    hdi[j] = hi[j];
    vdr[j] = vr[j];
    vdi[j] = vi[j];
  }
  const float dsk = (DSK && gi == 0) ? p.Dskip[dl] : 0.f;

  // ---- addressing: every tile goes through buffer resources based at its first row, so rows
  // past L read as zero and stores there are dropped ----
  const int64_t row_bytes = D * T::es, bc_row_bytes = N * CT::es;
  const char* x0 = static_cast<const char*>(p.x) + b * L * row_bytes;
  const char* dl0 = static_cast<const char*>(p.delta) + b * L * row_bytes;
  const char* B0 = static_cast<const char*>(p.B) + b * L * bc_row_bytes;
  const char* C0 = static_cast<const char*>(p.C) + b * L * bc_row_bytes;
  char* y0 = Y ? static_cast<char*>(p.y) + b * L * row_bytes : nullptr;
  // resource for the TT rows from row r on (rows past L are out of range): the tile's own rows
  // only, so extent and offset are 32-bit (tile_rsrc; the host keeps L below 2^30), with the
  // clamped row count read back as a scalar so that the resource stays scalar
  auto tile_rows = [&](int64_t r) {
    return __builtin_amdgcn_readfirstlane(min(max((int32_t)L - (int32_t)r, 0), TT));
  };
  auto rows = [&](const void* base, int64_t r, int64_t rb) {
    return tile_rsrc(base, (int32_t)r, tile_rows(r), (uint32_t)rb);
  };
  // history rows (REC): row ts + 1 + tt holds h after step ts + tt
  const int64_t hrow_bytes = N * D * 8;
  float* hist0 = REC ? p.hist + b * (L + 1) * N * D * 2 : nullptr;
  float* hist1 = REC ? hist0 + N * D * 2 : nullptr;  // row 1: h after step 0
  uint32_t h_voff[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t n = (int64_t)gi * K + j;
    h_voff[j] = (dvalid && n < N) ? (uint32_t)((n * D + d) * 8) : 0x80000000u;
  }
  if (REC) {
    // row 0: the initial state
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t n = (int64_t)gi * K + j;
      if (dvalid && n < N) {
        hist0[(n * D + d) * 2] = hr[j];
        hist0[(n * D + d) * 2 + 1] = hi[j];
      }
    }
  }

  uint32_t bc_voff[NBC];
#pragma unroll
  for (int r = 0; r < NBC; ++r) {
    const int i = tid + r * NTHR;
    const int n = i % NP;
    bc_voff[r] = (i < BCE && n < N) ? (uint32_t)((i / NP) * bc_row_bytes + n * CT::es) : 0x80000000u;
  }
  uint32_t x_voff[NX];
#pragma unroll
  for (int r = 0; r < NX; ++r) {
    const int i = tid + r * NTHR;
    const int64_t dch = (int64_t)cb * CB + i % CB;
    x_voff[r] = (i < XE && dch < D) ? (uint32_t)((i / CB) * row_bytes + dch * T::es) : 0x80000000u;
  }
  struct Set {
    craw b[NBC], c[NBC];
    raw x[NX], d[NX];
  };
  auto load_set = [&](Set& st, int64_t ts) {
    const auto rb = rows(B0, ts, bc_row_bytes), rc = rows(C0, ts, bc_row_bytes);
#pragma unroll
    for (int r = 0; r < NBC; ++r) {
      st.b[r] = CT::bload(rb, bc_voff[r], 0u);
      st.c[r] = CT::bload(rc, bc_voff[r], 0u);
    }
    const auto rx = rows(x0, ts, row_bytes), rd = rows(dl0, ts, row_bytes);
#pragma unroll
    for (int r = 0; r < NX; ++r) {
      st.x[r] = T::bload(rx, x_voff[r], 0u);
      st.d[r] = T::bload(rd, x_voff[r], 0u);
    }
  };
  auto store_set = [&](const Set& st, int buf) {
#pragma unroll
    for (int r = 0; r < NBC; ++r) {
      const int i = tid + r * NTHR;
      if (NBC * NTHR == BCE || i < BCE) {
        if (REC)  // B as given (alpha enters in fp64)
          bcs[buf][i / NP][i % NP] = make_float4(CT::re(st.b[r]), CT::im(st.b[r]), 0.f, 0.f);
        else
          bcs[buf][i / NP][i % NP] = make_float4(CT::re(st.b[r]) * p.alpha,
                                                 CT::im(st.b[r]) * p.alpha, CT::re(st.c[r]),
                                                 CT::im(st.c[r]));
      }
    }
#pragma unroll
    for (int r = 0; r < NX; ++r) {
      const int i = tid + r * NTHR;
      if (NX * NTHR == XE || i < XE) {
        const float xv = T::widen(st.x[r]), dv = T::widen(st.d[r]);
        xdl[buf][i / CB][i % CB] = make_float2(dv, REC ? xv : dv * xv);  // recording: (delta, x)
        if (DSK) xxl[DSK ? buf : 0][DSK ? i / CB : 0][i % CB] = xv;
      }
    }
  };

  // one step for the K states of this lane; returns this lane's part of the readout
  auto step = [&](int buf, int tt, const __amdgpu_buffer_rsrc_t& rh) -> float {
    const float2 dd = xdl[buf][tt][c];
    if constexpr (REC) {
      const double dlt = dd.x, cw = (double)p.alpha * dlt * (double)dd.y;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const float4 q = bcs[buf][tt][gi * K + j];
        const double mag = exp_tab(dlt * ArD[j], ctab);
        const CisD e = cis_rev_tab(dlt * AiD[j], ctab);
        const double ar = mag * e.c, ai = mag * e.s;
        vdr[j] = __builtin_fma((double)beta, vdr[j], cw * q.x);
        vdi[j] = __builtin_fma((double)beta, vdi[j], cw * q.y);
        const double nr = __builtin_fma(ar, hdr[j], __builtin_fma(-ai, hdi[j], vdr[j]));
        const double ni = __builtin_fma(ar, hdi[j], __builtin_fma(ai, hdr[j], vdi[j]));
        hdr[j] = nr;
        hdi[j] = ni;
        const u32x2 hv = {__float_as_uint((float)nr), __float_as_uint((float)ni)};
        __builtin_amdgcn_raw_buffer_store_b64(hv, rh, h_voff[j], (uint32_t)(tt * hrow_bytes), 0);
      }
      return 0.f;
    }
    float ys = DSK ? dsk * xxl[DSK ? buf : 0][DSK ? tt : 0][c] : 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float4 q = bcs[buf][tt][gi * K + j];
      const float mag = exp2_fast(dd.x * Ar[j]);
      float co, si;
      cis_delta_tab(dd.x, Ai[j], ctabf, co, si);
      const float ar = mag * co, ai = mag * si;
      vr[j] = fmaf(beta, vr[j], dd.y * q.x);
      vi[j] = fmaf(beta, vi[j], dd.y * q.y);
      const float nr = fmaf(ar, hr[j], fmaf(-ai, hi[j], vr[j]));
      const float ni = fmaf(ar, hi[j], fmaf(ai, hr[j], vi[j]));
      hr[j] = nr;
      hi[j] = ni;
      ys = fmaf(q.z, nr, ys);
      ys = fmaf(-q.w, ni, ys);
    }
    return ys;
  };
  auto emit = [&](int buf, int tt, float ys) {
    if (Y) {
      const float s = half_sum(ys);
      if (lane < 32) ypart[Y ? buf : 0][Y ? g : 0][tt][c] = s;
    }
  };
  auto compute_full = [&](int buf, int64_t ts) {
    const auto rh = REC ? rows(hist1, ts, hrow_bytes) : make_rsrc(nullptr, 0);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) emit(buf, tt, step(buf, tt, rh));
  };
  // the ragged last tile: rows past L must leave the states alone (uniform branch per row)
  auto compute_tail = [&](int buf, int64_t ts, int nv) {
    const auto rh = REC ? rows(hist1, ts, hrow_bytes) : make_rsrc(nullptr, 0);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
      if (tt < nv) emit(buf, tt, step(buf, tt, rh));
  };
  // y of a tile: each thread adds the S partials of its (row, channel) outputs in a fixed
  // order and stores them (channels past D and rows past L are dropped by the resource)
  auto finalize = [&](int buf, int64_t ts) {
    if (!Y) return;
    const auto ry = rows(y0, ts, row_bytes);
#pragma unroll
    for (int r = 0; r < NX; ++r) {
      const int i = tid + r * NTHR;
      if (NX * NTHR == XE || i < XE) {
        float s = 0.f;
#pragma unroll
        for (int gg = 0; gg < S; ++gg) s += ypart[Y ? buf : 0][Y ? gg : 0][i / CB][i % CB];
        T::bstore(ry, x_voff[r], 0u, s);
      }
    }
  };

  const int64_t nfull = L / TT;
  const int nrem = (int)(L - nfull * TT);
  const int64_t ntile = nfull + (nrem > 0 ? 1 : 0);
  if constexpr (REC)
    ctab_build(ctab, threadIdx.x, NTHR);
  else
    ctab_build_f32(ctabf, threadIdx.x, NTHR);
  {
    Set s0;
    load_set(s0, 0);
    store_set(s0, 0);
  }
  __syncthreads();
  for (int64_t k = 0; k < ntile; ++k) {
    const int64_t ts = k * TT;
    const int buf = (int)(k & 1);
    Set nx;
    load_set(nx, ts + TT);  // past L this reads zeros; the buffer then goes unused
    if (k < nfull)
      compute_full(buf, ts);
    else
      compute_tail(buf, ts, nrem);
    store_set(nx, buf ^ 1);
    __syncthreads();
    finalize(buf, ts);
  }

  if (Y && dvalid) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t n = (int64_t)gi * K + j;
      if (n < N) {
        const int64_t si = ((b * D + d) * N + n) * 2;
        if (p.last_h) {
          p.last_h[si] = hr[j];
          p.last_h[si + 1] = hi[j];
        }
        if (p.last_v) {
          p.last_v[si] = vr[j];
          p.last_v[si + 1] = vi[j];
        }
      }
    }
  }
}

template <typename IO, int K, int S>
hipError_t launch_ks(const CFwdArgs& a, bool record, hipStream_t s) {
  const dim3 grid((unsigned)(a.ncb * a.Bt)), block(S * kWave);
  if (record)
    hipLaunchKernelGGL((cfwd_kernel<IO, K, S, false, true>), grid, block, 0, s, a);
  else if (a.Dskip)
    hipLaunchKernelGGL((cfwd_kernel<IO, K, S, true, false>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((cfwd_kernel<IO, K, S, false, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <typename IO>
hipError_t launch_io(const CFwdArgs& a, bool record, hipStream_t s) {
  switch (complex_padded_states(a.N)) {
    case 4: return launch_ks<IO, 2, 1>(a, record, s);
    // 2 wavefronts per SIMD: 0.39 ms against 0.47 ms with 2 states x 4 wavefronts
    case 16: return launch_ks<IO, 1, 8>(a, record, s);
    case 32: return launch_ks<IO, 1, 16>(a, record, s);
    case 64: return launch_ks<IO, 4, 8>(a, record, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_cfwd(const CFwdArgs& a, int io_bf16, bool record, hipStream_t s) {
  return io_bf16 ? launch_io<bf16_storage>(a, record, s) : launch_io<float>(a, record, s);
}

}  // namespace msm
