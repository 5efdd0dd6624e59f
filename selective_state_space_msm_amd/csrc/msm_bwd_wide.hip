// Backward of the momentum selective scan for 64 padded states (17 <= N <= 64), gfx950.
//
// Same adjoints and the same two phases as the half-wavefront backward (msm_bwd.hip), with
// full-wavefront channel blocks: lane = channel (64 per workgroup), a wavefront keeps K = 4
// states and a workgroup of 16 wavefronts covers the 64 states.  The sums over channels for
// dB / dC use a butterfly reduce-scatter over the 64 lanes; dx / ddelta sum the 16 wavefront
// partials through LDS in a fixed order.  Partials go through the shared finalize kernel.
// The fused variant (EXT: delta bias + softplus, SiLU gate) re-forms delta_eff and the gated dy
// from the raw inputs wherever they are read, adds the wavefront partials of the pre-gate
// output C . h for dz, and sums the bias gradient per channel; it works in rounds of 4 rows
// so that the extra partials fit in LDS.  Its zero-order-hold form (EXT = 2) also carries the
// write coefficient g = delta phi(delta A) and its derivatives through dx, ddelta, dA and dB.
#include "msm_device.hpp"
#include "msm_internal.h"

namespace msm {
namespace {

// Butterfly reduce-scatter of M values over the 64 lanes of a wavefront.  Stage SMASK
// exchanges with lane ^ SMASK: lanes with that bit set keep the upper half of the remaining
// values, the others the lower half, and each adds what its partner sent.  Once one value is
// left, the remaining stages are a plain all-reduce.  On return lane l holds in v[0] the sum
// over all 64 lanes of value (l >> (6 - log2 M)).
template <int CNT, int SMASK, int M>
__device__ __forceinline__ void rs_stage(float (&v)[M], int lane) {
  if constexpr (SMASK >= 1) {
    if constexpr (CNT > 1) {
      constexpr int HALF = CNT / 2;
      const bool up = (lane & SMASK) != 0;
#pragma unroll
      for (int i = 0; i < HALF; ++i) {
        const float keep = up ? v[i + HALF] : v[i];
        const float send = up ? v[i] : v[i + HALF];
        v[i] = keep + __shfl_xor(send, SMASK);
      }
      rs_stage<HALF, SMASK / 2, M>(v, lane);
    } else {
      v[0] += __shfl_xor(v[0], SMASK);
      rs_stage<1, SMASK / 2, M>(v, lane);
    }
  }
}

template <int M>
__device__ __forceinline__ void reduce_scatter64(float (&v)[M], int lane) {
  static_assert(M >= 1 && M <= 64 && (M & (M - 1)) == 0, "M must be a power of two <= 64");
  rs_stage<M, 32, M>(v, lane);
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

template <typename IO, int K, int S, bool BETA0, bool HAS_DSKIP, int EXT>
__global__ __launch_bounds__(S* kWave) void bwd_wide_kernel(const BwdArgs p) {
  using T = io<IO>;
  using raw = typename T::raw;
  constexpr int TB = kBwdTile;
  constexpr int BCW = 2 * K;
  constexpr int BC_PER_TILE = TB * S * BCW;
  constexpr int NTHR = S * kWave;
  constexpr int NPER = (BC_PER_TILE + NTHR - 1) / NTHR;
  // rows whose per-wavefront partials sit in LDS at once (fp64, so fewer rows for big S)
  constexpr int SR = EXT ? 4 : (S >= 16 ? 8 : TB);
  constexpr bool ZOH = EXT == 2;  // zero-order-hold write coefficient g = delta phi(delta A)
  constexpr int NSR = TB / SR;
  // steps per lane-reduce block of dB/dC values (at most 64 values per block)
  constexpr int RB = (64 / (2 * K)) < SR ? (64 / (2 * K)) : SR;
  constexpr int M = 2 * K * RB;
  constexpr int NRB = SR / RB;
  static_assert(TB % SR == 0 && SR % RB == 0, "tile must split into rounds and reduce blocks");

  __shared__ float bcs[TB][S][BCW];       // fp32 B (alpha-scaled) | C, for the recompute
  __shared__ double bcs64[TB][S][BCW];    // the same values widened, for the adjoint sweep
  __shared__ double spart[2][S][SR][kWave];
  __shared__ float ypart[EXT ? S : 1][EXT ? SR : 1][kWave];  // fused: partials of C . h

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int g = tid / kWave;
  const int cb = (int)(blockIdx.x % p.ncb);
  const int64_t b = blockIdx.x / p.ncb;
  const int64_t L = p.L, D = p.D, N = p.N, NT = p.NT;
  const int64_t d = (int64_t)cb * kWave + lane;
  const bool dvalid = d < D;
  const int64_t dl = dvalid ? d : D - 1;
  const float beta = p.beta;
  const double beta64 = p.beta;

  float A2[K], v[K], h[K];
  double A64[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t n = (int64_t)g * K + j;
    const float an = n < N ? p.A[dl * N + n] : 0.f;
    A2[j] = an * kLog2e;
    A64[j] = an;
    const int64_t si = (b * D + dl) * N + n;
    v[j] = (p.v0 && n < N) ? p.v0[si] : 0.f;
    h[j] = (p.h0 && n < N) ? p.h0[si] : 0.f;
  }
  // fused extras of this lane's channel
  const float dbias = (EXT && p.delta_bias) ? p.delta_bias[dl] : 0.f;
  const bool softplus = EXT && p.delta_softplus != 0;
  const bool has_z = EXT && p.z != nullptr;
  auto delta_eff = [&](float dv) {
    if (!EXT) return dv;
    const float u = dv + dbias;
    return softplus ? softplus_f(u) : u;
  };
  // dy as the scan sees it: gated by silu(z)
  auto gated = [&](float gy, raw zr) { return has_z ? gy * silu_f(T::widen(zr)) : gy; };

  auto stage = [&](int64_t ts, int64_t nv) {
#pragma unroll
    for (int r = 0; r < NPER; ++r) {
      const int i = tid + r * NTHR;
      if (i < BC_PER_TILE) {
        const int tt = i / (S * BCW);
        const int rem = i % (S * BCW);
        const int gg = rem / BCW;
        const int r2 = rem % BCW;
        const int64_t n = (int64_t)gg * K + (r2 % K);
        float val = 0.f;
        if (tt < nv && n < N) {
          const int64_t idx = (b * L + ts + tt) * N + n;
          val = (r2 >= K) ? T::widen(T::load(p.C, idx)) : T::widen(T::load(p.B, idx)) * p.alpha;
        }
        (&bcs[0][0][0])[i] = val;
        (&bcs64[0][0][0])[i] = val;
      }
    }
  };
  auto ckpt_index = [&](int64_t tile, int which, int64_t n) {
    return (((b * NT + tile) * 2 + which) * N + n) * D + dl;
  };

  // ---------------- phase 1: forward with checkpoints ----------------
  for (int64_t tile = 0; tile < NT; ++tile) {
    const int64_t ts = tile * TB;
    const int64_t nv = (L - ts < TB) ? L - ts : TB;
    if (dvalid) {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int64_t n = (int64_t)g * K + j;
        if (n < N) {
          p.ckpt[ckpt_index(tile, 0, n)] = v[j];
          p.ckpt[ckpt_index(tile, 1, n)] = h[j];
        }
      }
    }
    raw xr[TB], dr[TB];
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) {
      const int64_t t = ts + (tt < nv ? tt : nv - 1);
      xr[tt] = T::load(p.x, (b * L + t) * D + dl);
      dr[tt] = T::load(p.delta, (b * L + t) * D + dl);
    }
    __syncthreads();
    stage(ts, nv);
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) {
      if (tt < nv) {
        const float xv = T::widen(xr[tt]), dv = delta_eff(T::widen(dr[tt]));
        const float c = dv * xv;
        const float* bc = &bcs[tt][g][0];
#pragma unroll
        for (int j = 0; j < K; ++j) {
          const float arg = dv * A2[j];
          const float a = exp2_fast(arg);
          float w = c * bc[j];
          if (ZOH) w *= zoh_phi(arg * kLn2, a);
          v[j] = BETA0 ? w : fmaf(beta, v[j], w);
          h[j] = fmaf(a, h[j], v[j]);
        }
      }
    }
  }

  // ---------------- phase 2: reverse sweep ----------------
  // The adjoint state and the sums that feed ddelta are kept in fp64: ddelta is a difference
  // of two large terms (x * sum B gv and sum A a h gh), and fp32 adjoints lose too many bits.
  double ghn[K], gvn[K], dAacc[K];  // ghn = a_{t+1} gh_{t+1}, gvn = beta gv_{t+1}
  // the adjoints of the final state enter as the carries into the last step
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t n = (int64_t)g * K + j;
    const int64_t si = (b * D + dl) * N + n;
    ghn[j] = (p.dlast_h && n < N) ? (double)p.dlast_h[si] : 0.0;
    gvn[j] = (p.dlast_v && n < N) ? (double)p.dlast_v[si] : 0.0;
    dAacc[j] = 0.0;
  }
  float dDacc = 0.f;
  double dbias64 = 0.0;  // fused: this lane's rows of the channel's bias gradient
  const float dsk = HAS_DSKIP ? p.Dskip[dl] : 0.f;
  float* dbc = p.dbc_part + (b * p.ncb + cb) * L * 2 * p.NP;

  for (int64_t tile = NT - 1; tile >= 0; --tile) {
    const int64_t ts = tile * TB;
    const int nv = (int)((L - ts < TB) ? L - ts : TB);
    raw xr[TB], dr[TB], gr[TB], zr[EXT ? TB : 1];
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) {
      const int64_t t = ts + (tt < nv ? tt : nv - 1);
      const int64_t idx = (b * L + t) * D + dl;
      xr[tt] = T::load(p.x, idx);
      dr[tt] = T::load(p.delta, idx);
      gr[tt] = T::load(p.dy, idx);
      if (EXT) zr[EXT ? tt : 0] = has_z ? T::load(p.z, idx) : raw{};
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t n = (int64_t)g * K + j;
      v[j] = n < N ? p.ckpt[ckpt_index(tile, 0, n)] : 0.f;
      h[j] = n < N ? p.ckpt[ckpt_index(tile, 1, n)] : 0.f;
    }
    __syncthreads();  // previous tile's readers of bcs / spart are done
    stage(ts, nv);
    __syncthreads();

    // recompute the tile: hs[tt] = h_{ts+tt-1}, av[tt] = a_{ts+tt}
    float hs[TB + 1][K], av[TB][K];
#pragma unroll
    for (int j = 0; j < K; ++j) hs[0][j] = h[j];
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) {
      if (tt < nv) {
        const float xv = T::widen(xr[tt]), dv = delta_eff(T::widen(dr[tt]));
        const float c = dv * xv;
        const float* bc = &bcs[tt][g][0];
#pragma unroll
        for (int j = 0; j < K; ++j) {
          const float arg = dv * A2[j];
          const float a = exp2_fast(arg);
          float w = c * bc[j];
          if (ZOH) w *= zoh_phi(arg * kLn2, a);
          v[j] = BETA0 ? w : fmaf(beta, v[j], w);
          h[j] = fmaf(a, h[j], v[j]);
          av[tt][j] = a;
          hs[tt + 1][j] = h[j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < K; ++j) {
          av[tt][j] = 0.f;
          hs[tt + 1][j] = 0.f;
        }
      }
    }

    // reverse sweep over the tile in rounds of SR rows, each split into reduce blocks of RB
#pragma unroll
    for (int sr = NSR - 1; sr >= 0; --sr) {
#pragma unroll
      for (int rb = NRB - 1; rb >= 0; --rb) {
        float vals[M];
#pragma unroll
        for (int tb = RB - 1; tb >= 0; --tb) {
          const int tr = rb * RB + tb;  // row within the round
          const int tt = sr * SR + tr;  // row within the tile
          if (tt < nv) {
            const float xv = T::widen(xr[tt]), dv = delta_eff(T::widen(dr[tt]));
            const float gy = EXT ? gated(T::widen(gr[tt]), zr[EXT ? tt : 0]) : T::widen(gr[tt]);
            const float c = dv * xv;
            float yq = 0.f;
            const double gy64 = gy, dv64 = dv;
            const double* bc = &bcs64[tt][g][0];
            double s1 = 0.0, s2 = 0.0, s1d = 0.0;
#pragma unroll
            for (int j = 0; j < K; ++j) {
              const double a64 = av[tt][j];
              const double gh = fma(bc[K + j], gy64, ghn[j]);
              const double gv = gh + gvn[j];
              const double gg = a64 * (double)hs[tt][j] * gh;
              s2 = fma(A64[j], gg, s2);
              dAacc[j] = fma(dv64, gg, dAacc[j]);
              if (!ZOH) {
                s1 = fma(bc[j], gv, s1);
                vals[(tb * 2 + 0) * K + j] = c * (float)gv;       // dB / alpha
              } else {
                // g = delta phi: dx and dB take phi, ddelta's write part dg/ddelta = a, and dA
                // gains alpha B x gv delta^2 psi
                const float u = dv * A2[j] * kLn2;
                const float ph = zoh_phi(u, av[tt][j]);
                const double bgv = bc[j] * gv;  // alpha B gv
                s1 = fma(bgv, (double)ph, s1);
                s1d = fma(bgv, a64, s1d);
                dAacc[j] = fma(bgv, (double)(xv * dv * dv * zoh_psi(u, av[tt][j], ph)), dAacc[j]);
                vals[(tb * 2 + 0) * K + j] = c * ph * (float)gv;  // dB / alpha
              }
              vals[(tb * 2 + 1) * K + j] = gy * hs[tt + 1][j];  // dC
              if (EXT) yq = fmaf(bcs[tt][g][K + j], hs[tt + 1][j], yq);
              ghn[j] = a64 * gh;
              gvn[j] = BETA0 ? 0.0 : beta64 * gv;
            }
            spart[0][g][tr][lane] = s1;
            // the zero-order hold's ddelta write part is not x times the dx sum: add it here
            spart[1][g][tr][lane] = ZOH ? fma((double)xv, s1d, s2) : s2;
            if (EXT) ypart[EXT ? g : 0][EXT ? tr : 0][lane] = yq;
            if (HAS_DSKIP) dDacc = fmaf(gy, xv, dDacc);
          } else {
#pragma unroll
            for (int j = 0; j < 2 * K; ++j) vals[tb * 2 * K + j] = 0.f;
          }
        }
        if (!dvalid) {
#pragma unroll
          for (int i = 0; i < M; ++i) vals[i] = 0.f;
        }
        reduce_scatter64<M>(vals, lane);
        constexpr int SH = 6 - ilog2(M);
        const int idx = lane >> SH;
        if ((lane & ((1 << SH) - 1)) == 0) {
          const int tb = idx / (2 * K);
          const int which = (idx / K) % 2;
          const int j = idx % K;
          const int tt = sr * SR + rb * RB + tb;
          const int64_t n = (int64_t)g * K + j;
          if (tt < nv && n < N) dbc[(ts + tt) * 2 * p.NP + which * p.NP + n] = vals[0];
        }
      }
      __syncthreads();
      // dx / ddelta for the rows of this round owned by this wavefront: add the S partials
      // in a fixed order, then combine in fp64 (the ddelta cancellation happens here)
      for (int tr = g; tr < SR; tr += S) {
        const int tt = sr * SR + tr;
        if (tt >= nv) break;
        double s1 = 0.0, s2 = 0.0;
#pragma unroll
        for (int gg = 0; gg < S; ++gg) {
          s1 += spart[0][gg][tr][lane];
          s2 += spart[1][gg][tr][lane];
        }
        if (dvalid) {
          const int64_t idx = (b * L + ts + tt) * D + d;
          if (!EXT) {
            const double xv = T::widen(T::load(p.x, idx)), dv = T::widen(T::load(p.delta, idx));
            double dxv = dv * s1;
            if (HAS_DSKIP) dxv = fma((double)dsk, (double)T::widen(T::load(p.dy, idx)), dxv);
            T::store(p.dx, idx, (float)dxv);
            T::store(p.ddelta, idx, (float)fma(xv, s1, s2));
          } else {
            const float xf = T::widen(T::load(p.x, idx)), draw = T::widen(T::load(p.delta, idx));
            const float gyr = T::widen(T::load(p.dy, idx));
            const float zv = has_z ? T::widen(T::load(p.z, idx)) : 0.f;
            const float gy = has_z ? gyr * silu_f(zv) : gyr;
            const double xv = xf, dv = delta_eff(draw);
            double dxv = dv * s1;
            if (HAS_DSKIP) dxv = fma((double)dsk, (double)gy, dxv);
            T::store(p.dx, idx, (float)dxv);
            // through softplus: d softplus(u) / du = logistic(u)
            const double dsp = softplus ? (double)logistic_f(draw + dbias).s : 1.0;
            const double qd = (ZOH ? s2 : fma(xv, s1, s2)) * dsp;
            T::store(p.ddelta, idx, (float)qd);
            dbias64 += qd;
            if (has_z) {
              // dz from the pre-gate output: the wavefront partials plus the skip term
              float yr = ypart[0][EXT ? tr : 0][lane];
#pragma unroll
              for (int gg = 1; gg < S; ++gg) yr += ypart[EXT ? gg : 0][EXT ? tr : 0][lane];
              if (HAS_DSKIP) yr = fmaf(dsk, xf, yr);
              T::store(p.dz, idx, gyr * silu_grad_f(zv) * yr);
            }
          }
        }
      }
      if (NSR > 1) __syncthreads();  // spart is reused by the next round of this tile
    }
  }

  // adjoints of the initial state: after step 0 the carries are a_0 gh_0 and beta gv_0
  if (dvalid) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t n = (int64_t)g * K + j;
      const int64_t si = (b * D + d) * N + n;
      if (n < N && p.dh0) p.dh0[si] = (float)ghn[j];
      if (n < N && p.dv0) p.dv0[si] = (float)gvn[j];
    }
  }
  if (dvalid) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t n = (int64_t)g * K + j;
      if (n < N) p.dA_part[(b * N + n) * D + d] = (float)dAacc[j];
    }
    if (HAS_DSKIP && g == 0) p.dD_part[b * D + d] = dDacc;
  }
  if (EXT && p.delta_bias) {
    // the bias gradient of the channel: each wavefront holds the sum over its rows
    __syncthreads();
    spart[0][g][0][lane] = dbias64;
    __syncthreads();
    if (g == 0 && dvalid) {
      double t = spart[0][0][0][lane];
#pragma unroll
      for (int gg = 1; gg < S; ++gg) t += spart[0][gg][0][lane];
      p.dbias_part[b * D + d] = (float)t;
    }
  }
}

template <typename IO, bool BETA0, int EXT>
hipError_t launch_wide(const BwdArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.ncb * a.Bt)), block(16 * kWave);
  if (a.Dskip)
    hipLaunchKernelGGL((bwd_wide_kernel<IO, 4, 16, BETA0, true, EXT>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((bwd_wide_kernel<IO, 4, 16, BETA0, false, EXT>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <typename IO, bool BETA0>
hipError_t launch_wide_ext(const BwdArgs& a, int ext, hipStream_t s) {
  switch (ext) {
    case 0: return launch_wide<IO, BETA0, 0>(a, s);
    case 1: return launch_wide<IO, BETA0, 1>(a, s);
    case 2: return launch_wide<IO, BETA0, 2>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_bwd_wide(const BwdArgs& a, int io_bf16, bool beta0, int ext, hipStream_t s) {
  if (a.NP != 64) return hipErrorInvalidValue;
  if (io_bf16)
    return beta0 ? launch_wide_ext<bf16_storage, true>(a, ext, s)
                 : launch_wide_ext<bf16_storage, false>(a, ext, s);
  return beta0 ? launch_wide_ext<float, true>(a, ext, s) : launch_wide_ext<float, false>(a, ext, s);
}

}  // namespace msm
