// Backward of the complex-valued momentum scan (gfx950): gradients of the real loss
//   sum(dy * y) + <dlast_h, last_h> + <dlast_v, last_v>   (<u, w> = Re sum conj(u) w).
//
// Gradients of complex inputs are returned as dL/dRe + i dL/dIm.  Adjoints (the real scan's
// "Gradient Flow" of the Momentum Mamba README carried to complex states; every product with a
// state adjoint takes the conjugate of the coefficient), per (b, d, n):
//   gh_t = dy_t conj(C_t) + conj(a_{t+1}) gh_{t+1}   (+ dlast_h at the last step)
//   gv_t = gh_t + beta gv_{t+1}                        (+ dlast_v at the last step)
//   dx_t     += alpha delta_t Re(conj(gv_t) B_t)
//   ddelta_t += alpha x_t Re(conj(gv_t) B_t) + Re(conj(gh_t) A a_t h_{t-1})
//   dA   += delta_t conj(a_t h_{t-1}) gh_t            dB_t += alpha delta_t x_t gv_t (sum over d)
//   dC_t += dy_t conj(h_t) (sum over d)               dh0 = conj(a_0) gh_0, dv0 = beta gv_0
//
// The states h_{t-1} come from the history that the recording forward pass wrote (one complex
// fp32 value per (b, t, n, d)): on a 288 GB device trading that buffer for the recompute of the
// real backward keeps this kernel a single reverse sweep.  The sweep computes a_t, the adjoints
// and the sums over n in fp64: the delta gradient carries a factor |A| (tens for a rotating
// state), and an fp32 a_t in the adjoint carry already exceeds the fp32 tolerance there.
// Layout as the complex forward: 32 channels per workgroup, state group 2 g + l / 32 of K
// states per lane.  Tiles of TT steps
// are swept in reverse; the inputs of the next (earlier) tile -- x, delta, dy, B, C through
// LDS, its TT history rows straight into registers -- are loaded while the current one is
// computed.  Reductions in a fixed order:
//   over n for dx / ddelta (in fp64): in-lane over K, across the halves with
//     v_permlane32_swap, across the S wavefronts through LDS;
//   over d for dB / dC: a reduce-scatter over each 32-lane half, then across channel blocks in
//     the finalize kernel; dA (accumulated in fp64 per lane) and dDskip across batch rows
//     there too.
#include <type_traits>

#include "msm_complex.hpp"
#include "msm_internal.h"
#include "msm_lanes.hpp"

namespace msm {
namespace {

// SPLIT: 0 = all states in one launch; otherwise this launch covers the 16 states n0 .. n0 + 15
// of 32 or 64 padded states (the 16-state plan runs without spills; wider plans do not), one of
// several launches: 1 = first, 2 = middle, 3 = last.  dx / ddelta are sums over the states, so
// the launches add their sums in an fp64 buffer ([Bt][L][2][D]) and the last one stores them;
// every other gradient comes from disjoint states.  The skip term belongs to the first launch.
template <typename IO, int K, int S, bool HAS_DSKIP, int SPLIT>
__global__ __launch_bounds__(S* kWave) void cbwd_kernel(const CBwdArgs p) {
  using T = io<IO>;
  using CT = cio<IO>;
  using raw = typename T::raw;
  using craw = typename CT::raw;
  // two tiles of history rows (the one swept and the one in flight) stay in registers: 64 of
  // them at two states per lane, 32 at four
  constexpr int TT = K >= 4 ? 2 : 16 / K;
  constexpr int CB = kBwdChans;
  constexpr int NTHR = S * kWave;
  constexpr int NP = 2 * S * K;
  constexpr int BCE = TT * NP;
  constexpr int NBC = (BCE + NTHR - 1) / NTHR;
  constexpr int XE = TT * CB;
  constexpr int NX = (XE + NTHR - 1) / NTHR;
  constexpr int M = 32;            // values per lane in one dB / dC reduce-scatter
  constexpr int RB = M / (4 * K);  // rows per reduce-scatter
  static_assert(RB >= 1 && TT % RB == 0, "tile must split into reduce blocks");

  __shared__ float4 bcs[2][TT][NP];       // alpha B (re, im), C (re, im)
  __shared__ float4 xs[2][TT][CB];        // delta, x, dy, alpha delta x
  __shared__ double2 gpart[2][S][TT][CB];  // (dx, ddelta) partial sums per wavefront
  __shared__ CTab ctab;                    // fp64 exponential and rotation tables

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
  const int64_t hrow_bytes = N * D * 8;
  const float* hist0 = p.hist + b * (L + 1) * N * D * 2;
  const int n0 = SPLIT ? p.n0 : 0;     // first state of this launch
  const int NPD = SPLIT ? p.NP : NP;   // states per row of the dB / dC partials

  // fp64: the rotation a_t, the adjoints and the sums over n (an fp32 a_t in the adjoint carry,
  // multiplied by |A| in the delta gradient, exceeds the fp32 tolerance); fp32: the history and
  // the per-element dB / dC terms
  double AiD[K], chr[K], chi[K], cvr[K], cvi[K], dAr[K], dAi[K];
  float Are[K], Aim[K], hcr[K], hci[K];  // A converts to fp64 exactly where it is used
  uint32_t h_voff[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t n = n0 + (int64_t)gi * K + j;
    const bool on = n < N;
    const bool live = on && dvalid;
    const int64_t ai = (dl * N + (on ? n : 0)) * 2;
    Are[j] = on ? p.A[ai] : 0.f;
    Aim[j] = on ? p.A[ai + 1] : 0.f;
    AiD[j] = Aim[j] / kTwoPiD;
    const int64_t si = ((b * D + dl) * N + (on ? n : 0)) * 2;
    chr[j] = (on && p.dlast_h) ? p.dlast_h[si] : 0.f;
    chi[j] = (on && p.dlast_h) ? p.dlast_h[si + 1] : 0.f;
    cvr[j] = (on && p.dlast_v) ? p.dlast_v[si] : 0.f;
    cvi[j] = (on && p.dlast_v) ? p.dlast_v[si + 1] : 0.f;
    // h_{L-1}: history row L
    const int64_t hi0 = (L * N * D + (on ? n : 0) * D + dl) * 2;
    hcr[j] = live ? hist0[hi0] : 0.f;
    hci[j] = live ? hist0[hi0 + 1] : 0.f;
    dAr[j] = dAi[j] = 0.0;
    h_voff[j] = live ? (uint32_t)((n * D + d) * 8) : 0x80000000u;
  }
  const float dsk = (HAS_DSKIP && gi == 0) ? p.Dskip[dl] : 0.f;
  double dsum = 0.0;  // sum of dy x over time, for dDskip

  const int64_t row_bytes = D * T::es, bc_row_bytes = N * CT::es;
  const char* x0 = static_cast<const char*>(p.x) + b * L * row_bytes;
  const char* dl0 = static_cast<const char*>(p.delta) + b * L * row_bytes;
  const char* dy0 = static_cast<const char*>(p.dy) + b * L * row_bytes;
  const char* B0 = static_cast<const char*>(p.B) + b * L * bc_row_bytes;
  const char* C0 = static_cast<const char*>(p.C) + b * L * bc_row_bytes;
  char* dx0 = static_cast<char*>(p.dx) + b * L * row_bytes;
  char* ddl0 = static_cast<char*>(p.ddelta) + b * L * row_bytes;
  const int64_t part_row_bytes = (int64_t)NPD * 16;
  char* part0 = reinterpret_cast<char*>(p.dbc_part) + (b * p.ncb + cb) * L * part_row_bytes;
  // Resource for the TT rows of a (nrows, rb) slab from row r on (rows past nrows are out of
  // range): the tile's own rows only, so extent and offset are 32-bit (tile_rsrc; the host keeps
  // L below 2^30).  The clamped row count is read back as a scalar (the compiler forms it with a
  // vector med3, and a resource built from a vector value loops over the lanes' values).
  auto rows = [&](const void* base, int64_t r, int64_t rb, int64_t nrows) {
    const int32_t nr = __builtin_amdgcn_readfirstlane(min(max((int32_t)nrows - (int32_t)r, 0), TT));
    return tile_rsrc(base, (int32_t)r, nr, (uint32_t)rb);
  };

  uint32_t bc_voff[NBC];
#pragma unroll
  for (int r = 0; r < NBC; ++r) {
    const int i = tid + r * NTHR;
    const int n = n0 + i % NP;
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
    raw x[NX], d[NX], g[NX];
    u32x2 h[TT][K];  // history rows ts .. ts + TT - 1, i.e. h_{t-1} of each step t of the tile
  };
  auto load_set = [&](Set& st, int64_t ts) {
    const auto rb = rows(B0, ts, bc_row_bytes, L), rc = rows(C0, ts, bc_row_bytes, L);
#pragma unroll
    for (int r = 0; r < NBC; ++r) {
      st.b[r] = CT::bload(rb, bc_voff[r], 0u);
      st.c[r] = CT::bload(rc, bc_voff[r], 0u);
    }
    const auto rx = rows(x0, ts, row_bytes, L), rd = rows(dl0, ts, row_bytes, L),
               rg = rows(dy0, ts, row_bytes, L);
#pragma unroll
    for (int r = 0; r < NX; ++r) {
      st.x[r] = T::bload(rx, x_voff[r], 0u);
      st.d[r] = T::bload(rd, x_voff[r], 0u);
      st.g[r] = T::bload(rg, x_voff[r], 0u);
    }
    const auto rh = rows(hist0, ts, hrow_bytes, L + 1);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int j = 0; j < K; ++j)
        // the row goes into the per-lane offset, which the range check covers (rows past L + 1
        // in the ragged tile read zeros)
        st.h[tt][j] = __builtin_amdgcn_raw_buffer_load_b64(
            rh, h_voff[j] + (uint32_t)(tt * hrow_bytes), 0u, 0);
  };
  auto store_set = [&](const Set& st, int buf) {
#pragma unroll
    for (int r = 0; r < NBC; ++r) {
      const int i = tid + r * NTHR;
      if (NBC * NTHR == BCE || i < BCE)
        bcs[buf][i / NP][i % NP] = make_float4(CT::re(st.b[r]) * p.alpha, CT::im(st.b[r]) * p.alpha,
                                               CT::re(st.c[r]), CT::im(st.c[r]));
    }
#pragma unroll
    for (int r = 0; r < NX; ++r) {
      const int i = tid + r * NTHR;
      if (NX * NTHR == XE || i < XE) {
        const float xv = T::widen(st.x[r]), dv = T::widen(st.d[r]), gv = T::widen(st.g[r]);
        xs[buf][i / CB][i % CB] = make_float4(dv, xv, gv, p.alpha * dv * xv);
      }
    }
  };

  // Steps of one tile, last row first.  Rows at or past nv (the ragged tile only) are skipped.
  auto compute = [&](auto tail_c, int buf, int64_t ts, const Set& cur, int nv) {
    constexpr bool TAIL = decltype(tail_c)::value;
    const auto rp = rows(part0, ts, part_row_bytes, L);
#pragma unroll
    for (int rb = 0; rb < TT / RB; ++rb) {
      float vals[M];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int tt = TT - 1 - (rb * RB + i);
        if (TAIL && tt >= nv) {
#pragma unroll
          for (int e = 0; e < 4 * K; ++e) vals[i * 4 * K + e] = 0.f;
          continue;
        }
        const float4 e = xs[buf][tt][c];
        const double dlt = e.x, xv = e.y, dyv = e.z;
        double sdx = 0.0, sdd = 0.0;
#pragma unroll
        for (int j = 0; j < K; ++j) {
          const float4 q = bcs[buf][tt][gi * K + j];
          const double hpr = __uint_as_float(cur.h[tt][j].x), hpi = __uint_as_float(cur.h[tt][j].y);
          const double ghr = __builtin_fma(dyv, (double)q.z, chr[j]);
          const double ghi = __builtin_fma(-dyv, (double)q.w, chi[j]);
          const double gvr = ghr + cvr[j], gvi = ghi + cvi[j];
          const double mag = exp_tab(dlt * (double)Are[j], ctab);
          const CisD ee = cis_rev_tab(dlt * AiD[j], ctab);
          const double ar = mag * ee.c, ai = mag * ee.s;
          const double Pr = __builtin_fma(ar, hpr, -ai * hpi);  // a h_{t-1}
          const double Pi = __builtin_fma(ar, hpi, ai * hpr);
          const double s1 = __builtin_fma(gvr, (double)q.x, gvi * q.y);  // Re(conj(gv) alpha B)
          sdx = __builtin_fma(dlt, s1, sdx);
          const double Qr = __builtin_fma((double)Are[j], Pr, -(double)Aim[j] * Pi);  // A a h_{t-1}
          const double Qi = __builtin_fma((double)Are[j], Pi, (double)Aim[j] * Pr);
          sdd = __builtin_fma(xv, s1, sdd);
          sdd = __builtin_fma(ghr, Qr, sdd);
          sdd = __builtin_fma(ghi, Qi, sdd);
          // dA += delta conj(a h_{t-1}) gh
          dAr[j] = __builtin_fma(dlt, __builtin_fma(Pr, ghr, Pi * ghi), dAr[j]);
          dAi[j] = __builtin_fma(dlt, __builtin_fma(Pr, ghi, -Pi * ghr), dAi[j]);
          vals[i * 4 * K + 4 * j + 0] = e.w * (float)gvr;
          vals[i * 4 * K + 4 * j + 1] = e.w * (float)gvi;
          vals[i * 4 * K + 4 * j + 2] = e.z * hcr[j];
          vals[i * 4 * K + 4 * j + 3] = -e.z * hci[j];
          chr[j] = __builtin_fma(ar, ghr, ai * ghi);  // conj(a_t) gh_t, carried to step t - 1
          chi[j] = __builtin_fma(ar, ghi, -ai * ghr);
          cvr[j] = (double)beta * gvr;
          cvi[j] = (double)beta * gvi;
          hcr[j] = (float)hpr;
          hci[j] = (float)hpi;
        }
        sdx = __builtin_fma((double)dsk, dyv, sdx);  // skip term, once per channel
        dsum = __builtin_fma(dyv, xv, dsum);
        sdx = half_sum_d(sdx);
        sdd = half_sum_d(sdd);
        if (lane < 32) gpart[buf][g][tt][c] = make_double2(sdx, sdd);
      }
      reduce_scatter32(vals, lane);
      // lane l of a half now holds value (l & 31) = (row r of the block, state j, component)
      const int q = lane & 31;
      const int r = q / (4 * K), j = (q / 4) % K, comp = q & 3;
      const int tt = TT - 1 - (rb * RB + r);
      const uint32_t off = (uint32_t)((tt * NPD + n0 + gi * K + j) * 16 + comp * 4);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(vals[0]), rp, off, 0u, 0);
    }
  };
  // split launches: per-thread offsets into the fp64 sums, [L][2][D] per batch row
  const int64_t acc_row_bytes = 2 * D * 8;
  char* acc0 = SPLIT ? reinterpret_cast<char*>(p.acc) + b * L * acc_row_bytes : dx0;
  uint32_t a_voff[NX];
#pragma unroll
  for (int r = 0; r < NX; ++r) {
    const int i = tid + r * NTHR;
    const int64_t dch = (int64_t)cb * CB + i % CB;
    a_voff[r] = (i < XE && dch < D) ? (uint32_t)(((i / CB) * 2 * D + dch) * 8) : 0x80000000u;
  }
  auto finalize = [&](int buf, int64_t ts) {
    const auto rdx = rows(dx0, ts, row_bytes, L), rdd = rows(ddl0, ts, row_bytes, L);
    const auto racc = SPLIT ? rows(acc0, ts, acc_row_bytes, L) : make_rsrc(acc0, 0);
#pragma unroll
    for (int r = 0; r < NX; ++r) {
      const int i = tid + r * NTHR;
      if (NX * NTHR == XE || i < XE) {
        // every partial read before the first sum: one LDS round trip
        double2 pv[S];
#pragma unroll
        for (int gg = 0; gg < S; ++gg) pv[gg] = gpart[buf][gg][i / CB][i % CB];
        double sx = pv[0].x, sd = pv[0].y;
#pragma unroll
        for (int gg = 1; gg < S; ++gg) {
          sx += pv[gg].x;
          sd += pv[gg].y;
        }
        if constexpr (SPLIT == 0) {
          T::bstore(rdx, x_voff[r], 0u, (float)sx);
          T::bstore(rdd, x_voff[r], 0u, (float)sd);
        } else {
          const uint32_t ox = a_voff[r], od = a_voff[r] + (uint32_t)(D * 8);
          if (SPLIT != 1) {
            const u32x2 wx = __builtin_amdgcn_raw_buffer_load_b64(racc, ox, 0u, 0);
            const u32x2 wd = __builtin_amdgcn_raw_buffer_load_b64(racc, od, 0u, 0);
            sx += __longlong_as_double((long long)(((uint64_t)wx.y << 32) | wx.x));
            sd += __longlong_as_double((long long)(((uint64_t)wd.y << 32) | wd.x));
          }
          if (SPLIT == 3) {
            T::bstore(rdx, x_voff[r], 0u, (float)sx);
            T::bstore(rdd, x_voff[r], 0u, (float)sd);
          } else {
            const uint64_t ux = (uint64_t)__double_as_longlong(sx);
            const uint64_t ud = (uint64_t)__double_as_longlong(sd);
            const u32x2 wx = {(uint32_t)ux, (uint32_t)(ux >> 32)};
            const u32x2 wd = {(uint32_t)ud, (uint32_t)(ud >> 32)};
            __builtin_amdgcn_raw_buffer_store_b64(wx, racc, ox, 0u, 0);
            __builtin_amdgcn_raw_buffer_store_b64(wd, racc, od, 0u, 0);
          }
        }
      }
    }
  };

  const int64_t nfull = L / TT;
  const int nrem = (int)(L - nfull * TT);
  const int64_t ntile = nfull + (nrem > 0 ? 1 : 0);
  const int64_t klast = ntile - 1;
  auto stepk = [&](int64_t k, const Set& cur, Set& nxt) {
    const int64_t ts = k * TT;
    const int buf = (int)(k & 1);
    load_set(nxt, (k > 0 ? k - 1 : 0) * TT);  // at k = 0 a harmless reload, left unused
    if (k == klast && nrem > 0)
      compute(std::true_type{}, buf, ts, cur, nrem);
    else
      compute(std::false_type{}, buf, ts, cur, TT);
    store_set(nxt, buf ^ 1);
    __syncthreads();
    finalize(buf, ts);
  };
  ctab_build(ctab, threadIdx.x, NTHR);
  Set sa, sb;
  load_set(sa, klast * TT);
  store_set(sa, (int)(klast & 1));
  __syncthreads();
  for (int64_t k = klast; k >= 0; k -= 2) {
    stepk(k, sa, sb);
    if (k >= 1) stepk(k - 1, sb, sa);
  }

  if (dvalid) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t n = n0 + (int64_t)gi * K + j;
      if (n < N) {
        const int64_t si = ((b * D + d) * N + n) * 2;
        if (p.dh0) {
          p.dh0[si] = chr[j];
          p.dh0[si + 1] = chi[j];
        }
        if (p.dv0) {
          p.dv0[si] = cvr[j];
          p.dv0[si + 1] = cvi[j];
        }
        const int64_t ai = ((b * D + d) * N + n) * 2;
        p.dA_part[ai] = (float)dAr[j];
        p.dA_part[ai + 1] = (float)dAi[j];
      }
    }
    if (HAS_DSKIP && gi == 0) p.dD_part[b * D + d] = (float)dsum;
  }
}

// Sums the per-block partials in a fixed order: dB, dC (over channel blocks), dA and dDskip
// (over batch rows).
template <typename IO>
__global__ __launch_bounds__(256) void cbwd_finalize_kernel(const CBwdArgs p) {
  using CT = cio<IO>;
  const int64_t n_bc = p.Bt * p.L * p.N;
  const int64_t n_a = p.D * p.N;
  const int64_t n_d = p.Dskip ? p.D : 0;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_bc) {
    const int64_t n = i % p.N;
    const int64_t bt = i / p.N;  // b * L + t
    const int64_t b = bt / p.L, t = bt % p.L;
    const float4* src = reinterpret_cast<const float4*>(p.dbc_part) + (b * p.ncb * p.L + t) * p.NP + n;
    const int64_t stride = p.L * p.NP;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    int cb = 0;
    for (; cb + 4 <= p.ncb; cb += 4) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = src[(cb + u) * stride];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s.x += v[u].x;
        s.y += v[u].y;
        s.z += v[u].z;
        s.w += v[u].w;
      }
    }
    for (; cb < p.ncb; ++cb) {
      const float4 v = src[cb * stride];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    CT::store(p.dB, i, s.x, s.y);
    CT::store(p.dC, i, s.z, s.w);
  } else if (i < n_bc + n_a) {
    const int64_t k = i - n_bc;  // d * N + n
    float sr = 0.f, si = 0.f;
    for (int64_t b = 0; b < p.Bt; ++b) {
      sr += p.dA_part[(b * n_a + k) * 2];
      si += p.dA_part[(b * n_a + k) * 2 + 1];
    }
    p.dA[2 * k] = sr;
    p.dA[2 * k + 1] = si;
  } else if (i < n_bc + n_a + n_d) {
    const int64_t dd = i - n_bc - n_a;
    float s = 0.f;
    for (int64_t b = 0; b < p.Bt; ++b) s += p.dD_part[b * p.D + dd];
    p.dDskip[dd] = s;
  }
}

template <typename IO, int K, int S, int SPLIT>
hipError_t launch_sweep(const CBwdArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.ncb * a.Bt)), block(S * kWave);
  if (a.Dskip)
    hipLaunchKernelGGL((cbwd_kernel<IO, K, S, true, SPLIT>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((cbwd_kernel<IO, K, S, false, SPLIT>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <typename IO>
hipError_t launch_io(const CBwdArgs& a, hipStream_t s) {
  hipError_t e;
  if (a.NP == 4) {
    e = launch_sweep<IO, 2, 1, 0>(a, s);
  } else if (a.NP == 16) {
    e = launch_sweep<IO, 2, 4, 0>(a, s);
  } else if (a.NP == 32 || a.NP == 64) {
    // 16 states per launch (the last launch stores dx / ddelta); the skip term in the first
    const int parts = a.NP / 16;
    e = hipSuccess;
    for (int k = 0; k < parts && e == hipSuccess; ++k) {
      CBwdArgs h = a;
      h.n0 = 16 * k;
      if (k > 0) h.Dskip = nullptr;
      if (k == 0)
        e = launch_sweep<IO, 2, 4, 1>(h, s);
      else if (k == parts - 1)
        e = launch_sweep<IO, 2, 4, 3>(h, s);
      else
        e = launch_sweep<IO, 2, 4, 2>(h, s);
    }
  } else {
    return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const int64_t total = a.Bt * a.L * a.N + a.D * a.N + (a.Dskip ? a.D : 0);
  hipLaunchKernelGGL((cbwd_finalize_kernel<IO>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cbwd(const CBwdArgs& a, int io_bf16, hipStream_t s) {
  return io_bf16 ? launch_io<bf16_storage>(a, s) : launch_io<float>(a, s);
}

}  // namespace msm
