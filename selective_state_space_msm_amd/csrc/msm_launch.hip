// Launchers: the forward and backward recurrence kernels (one build of msm_fwd.hip /
// msm_bwd.hip per I/O dtype and variant; the full-wave backward for 64 padded states), and
// the kernel that finishes the backward by summing its per-block partials.
#include <mutex>

#include "msm_device.hpp"
#include "msm_internal.h"

namespace msm {
namespace {

// Sums the per-block partials in a fixed order and writes dB, dC (I/O dtype), dA, dDskip and
// the delta-bias gradient.
template <typename IO>
__global__ __launch_bounds__(256) void bwd_finalize_kernel(const BwdArgs p) {
  using T = io<IO>;
  const int64_t n_bc = p.Bt * p.L * 2 * p.N;
  const int64_t n_a = p.D * p.N;
  const int64_t n_d = p.Dskip ? p.D : 0;
  const int64_t n_g = p.ddelta_bias ? p.D : 0;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_bc) {
    const int64_t n = i % p.N;
    const int64_t which = (i / p.N) % 2;
    const int64_t bt = i / (2 * p.N);  // b * L + t
    const int64_t b = bt / p.L, t = bt % p.L;
    // the channel blocks' partials sit L * 2 * NP floats apart; eight loads are issued before
    // they are added (in the same fixed order), which keeps several in flight per thread
    const float* src = p.dbc_part + ((b * p.ncb) * p.L + t) * 2 * p.NP + which * p.NP + n;
    const int64_t stride = p.L * 2 * p.NP;
    float s = 0.f;
    int cb = 0;
    for (; cb + 8 <= p.ncb; cb += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = src[(cb + u) * stride];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; cb < p.ncb; ++cb) s += src[cb * stride];
    if (which == 0)
      T::store(p.dB, bt * p.N + n, s * p.alpha);
    else
      T::store(p.dC, bt * p.N + n, s);
  } else if (i < n_bc + n_a) {
    const int64_t k = i - n_bc;  // d * N + n
    const int64_t dd = k / p.N, n = k % p.N;
    float s = 0.f;
    for (int64_t b = 0; b < p.Bt; ++b) s += p.dA_part[(b * p.N + n) * p.D + dd];
    p.dA[k] = s;
  } else if (i < n_bc + n_a + n_d) {
    const int64_t dd = i - n_bc - n_a;
    float s = 0.f;
    for (int64_t b = 0; b < p.Bt; ++b) s += p.dD_part[b * p.D + dd];
    p.dDskip[dd] = s;
  } else if (i < n_bc + n_a + n_d + n_g) {
    const int64_t dd = i - n_bc - n_a - n_d;
    float s = 0.f;
    for (int64_t b = 0; b < p.Bt; ++b) s += p.dbias_part[b * p.D + dd];
    p.ddelta_bias[dd] = s;
  }
}

template <typename IO>
hipError_t launch_finalize(const BwdArgs& a, hipStream_t s) {
  const int64_t total =
      a.Bt * a.L * 2 * a.N + a.D * a.N + (a.Dskip ? a.D : 0) + (a.ddelta_bias ? a.D : 0);
  hipLaunchKernelGGL((bwd_finalize_kernel<IO>), dim3((unsigned)((total + 255) / 256)), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int io_bf16, int K, bool beta0, int ext, hipStream_t s) {
  hipError_t e;
  if (a.NP == 64 && K == 2) {
    // two halves of 32 states through the half-wavefront kernel: the second runs without the
    // skip term (the first adds it) and adds the first's dx / ddelta / dz sums
    auto part = [&](const BwdArgs& h) {
      if (io_bf16)
        return ext == 2 ? launch_bwd_part_1_2(h, 2, beta0, s)
               : ext == 1 ? launch_bwd_part_1_1(h, 2, beta0, s)
                          : launch_bwd_part_1_0(h, 2, beta0, s);
      return ext == 2 ? launch_bwd_part_0_2(h, 2, beta0, s)
             : ext == 1 ? launch_bwd_part_0_1(h, 2, beta0, s)
                        : launch_bwd_part_0_0(h, 2, beta0, s);
    };
    BwdArgs h1 = a;
    h1.n0 = 0;
    h1.split_pass = 1;
    e = part(h1);
    if (e != hipSuccess) return e;
    BwdArgs h2 = a;
    h2.n0 = 32;
    h2.split_pass = 2;
    h2.Dskip = nullptr;
    e = part(h2);
  } else if (a.NP == 64) {
    e = launch_bwd_wide(a, io_bf16, beta0, ext, s);
  } else if (io_bf16) {
    e = ext == 2 ? launch_bwd_part_1_2(a, K, beta0, s)
        : ext == 1 ? launch_bwd_part_1_1(a, K, beta0, s)
                   : launch_bwd_part_1_0(a, K, beta0, s);
  } else {
    e = ext == 2 ? launch_bwd_part_0_2(a, K, beta0, s)
        : ext == 1 ? launch_bwd_part_0_1(a, K, beta0, s)
                   : launch_bwd_part_0_0(a, K, beta0, s);
  }
  if (e != hipSuccess) return e;
  return io_bf16 ? launch_finalize<bf16_storage>(a, s) : launch_finalize<float>(a, s);
}

// Scratch of the allocation-free forward (msm_scan_fwd_noalloc): a file-scope device array, one
// copy per GPU the library runs on, held until the process ends.  Host code never uses the
// array's name as an address: the device address comes from hipGetSymbolAddress, looked up once
// per device with that device current and kept in `scratch_dev`.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_dev[dev] = p;
  }
  *ptr = scratch_dev[dev];
  return hipSuccess;
}

hipError_t launch_fwd(const FwdArgs& a, int io_bf16, int K, bool beta0, int ext, hipStream_t s) {
  if (io_bf16)
    return ext == 2   ? launch_fwd_part_1_2(a, K, beta0, s)
           : ext == 1 ? launch_fwd_part_1_1(a, K, beta0, s)
                      : launch_fwd_part_1_0(a, K, beta0, s);
  return ext == 2   ? launch_fwd_part_0_2(a, K, beta0, s)
         : ext == 1 ? launch_fwd_part_0_1(a, K, beta0, s)
                    : launch_fwd_part_0_0(a, K, beta0, s);
}

}  // namespace msm
