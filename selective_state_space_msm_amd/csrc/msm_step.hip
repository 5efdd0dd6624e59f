// Single-token decode step of the momentum selective scan (gfx950).
//
// The `step` of the Momentum Mamba README (one token in, the ssm and velocity states carried in
// and out), for the scan part of the block: with the fused op's extras,
//   delta_eff = softplus(delta + bias[d]) (or delta + bias[d]),
//   v' = beta v + alpha g B x,  h' = exp(delta_eff A) h + v',
//   (g = delta_eff, or (exp(delta_eff A) - 1) / A with the zero-order hold),
//   y  = (C . h' + Dskip x) * silu(z)   (the gate when z is given),
// with h and v, (Bt, D, N) fp32, updated in place.
//
// The step reads and writes every state once and does a handful of flops per state: it is
// bound by HBM bandwidth (16 bytes of state traffic per (b, d, n)).  The layout follows that:
// a channel's N states are contiguous, G = ceil(N / 4) rounded up to a power of two lanes
// share a channel and each lane moves four consecutive states with 16-byte loads and stores,
// so a wavefront streams one contiguous block of both state arrays.  The readout sum over the
// channel's lanes is a butterfly of lane swaps inside the group.  B, C (per batch row), A (per
// channel) and x / delta / z (per channel) are shared between lanes and come from cache.  The
// state loads and stores are marked nontemporal: every state is touched once per step, and
// keeping them out of the caches leaves those to the shared operands (measured: 5.5 TB/s with
// the hint against 5.1 TB/s without, at 1024 x 4096 x 16 states).
#include "msm_device.hpp"
#include "msm_internal.h"

namespace msm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename IO, bool VEC>
__global__ __launch_bounds__(256) void step_kernel(const StepArgs p) {
  using T = io<IO>;
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int G = p.G;
  const int64_t npair = p.Bt * p.D;
  const int64_t pr_raw = gtid / G;
  const bool valid = pr_raw < npair;
  // lanes past the last channel compute on the last one and store nothing (the butterfly
  // below needs every lane of a group)
  const int64_t pr = valid ? pr_raw : npair - 1;
  const int q = (int)(gtid - pr_raw * G);
  const int64_t N = p.N, D = p.D;
  const int64_t b = pr / D, d = pr - b * D;
  const int n0 = 4 * q;

  const float xv = T::widen(T::load(p.x, pr));
  const float draw = T::widen(T::load(p.delta, pr));
  const float u = draw + (p.delta_bias ? p.delta_bias[d] : 0.f);
  const float de = p.delta_softplus ? softplus_f(u) : u;
  const float c = p.alpha * de * xv;

  float hs[4], vs[4], As[4], Bs[4], Cs[4];
  float* hp = p.h + pr * N + n0;
  float* vp = p.v + pr * N + n0;
  if (VEC) {
    // N is a multiple of 4 here, so a lane's four states are all real or all padding
    if (n0 < N) {
      const f32x4 h4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(hp));
      const f32x4 v4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(vp));
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(p.A + d * N + n0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hs[j] = h4[j];
        vs[j] = v4[j];
        As[j] = a4[j];
        Bs[j] = T::widen(T::load(p.B, b * N + n0 + j));
        Cs[j] = T::widen(T::load(p.C, b * N + n0 + j));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) hs[j] = vs[j] = As[j] = Bs[j] = Cs[j] = 0.f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool on = n0 + j < N;
      hs[j] = on ? hp[j] : 0.f;
      vs[j] = on ? vp[j] : 0.f;
      As[j] = on ? p.A[d * N + n0 + j] : 0.f;
      Bs[j] = on ? T::widen(T::load(p.B, b * N + n0 + j)) : 0.f;
      Cs[j] = on ? T::widen(T::load(p.C, b * N + n0 + j)) : 0.f;
    }
  }

  float ys = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float arg = de * (As[j] * kLog2e);
    const float a = exp2_fast(arg);
    float w = c * Bs[j];
    if (p.zoh) w *= zoh_phi_fwd(arg * kLn2, a);  // zero-order hold: g = delta phi(delta A)
    vs[j] = fmaf(p.beta, vs[j], w);
    hs[j] = fmaf(a, hs[j], vs[j]);
    ys = fmaf(Cs[j], hs[j], ys);  // padding states have C = 0
  }

  if (valid) {
    if (VEC) {
      if (n0 < N) {
        const f32x4 h4 = {hs[0], hs[1], hs[2], hs[3]};
        const f32x4 v4 = {vs[0], vs[1], vs[2], vs[3]};
        __builtin_nontemporal_store(h4, reinterpret_cast<f32x4*>(hp));
        __builtin_nontemporal_store(v4, reinterpret_cast<f32x4*>(vp));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (n0 + j < N) {
          hp[j] = hs[j];
          vp[j] = vs[j];
        }
      }
    }
  }

  // readout: sum over the G lanes of the channel (groups are aligned inside the wavefront)
  for (int m = G >> 1; m > 0; m >>= 1) ys += __shfl_xor(ys, m, 64);
  if (valid && q == 0) {
    float yv = p.Dskip ? fmaf(p.Dskip[d], xv, ys) : ys;
    if (p.z) yv *= silu_f(T::widen(T::load(p.z, pr)));
    T::store(p.y, pr, yv);
  }
}

template <typename IO>
hipError_t launch_io(const StepArgs& a, bool vec, hipStream_t s) {
  const int64_t threads = a.Bt * a.D * a.G;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (vec)
    hipLaunchKernelGGL((step_kernel<IO, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((step_kernel<IO, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step(const StepArgs& a, int io_bf16, bool vec, hipStream_t s) {
  return io_bf16 ? launch_io<bf16_storage>(a, vec, s) : launch_io<float>(a, vec, s);
}

}  // namespace msm
