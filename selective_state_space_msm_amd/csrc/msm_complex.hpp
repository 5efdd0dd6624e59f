// Complex-valued elements for the complex scan kernels (gfx950): interleaved (re, im) pairs.
#pragma once

#include "msm_device.hpp"

namespace msm {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr double kTwoPiD = 6.283185307179586;

// Im A in revolutions, split into a float pair (hi + lo) so that the phase delta * Im A / 2 pi
// keeps its accuracy when it spans several turns.
struct RevPair {
  float hi, lo;
};
__device__ __forceinline__ RevPair to_revolutions(float im_a) {
  const double r = (double)im_a / kTwoPiD;
  const float hi = (float)r;
  return RevPair{hi, (float)(r - (double)hi)};
}

// e^(i delta Im A) = (c, s) with a table of e^(2 pi i m / 64), m < 64, in fp32 (each entry
// rounded from the fp64 rotation).  The phase in revolutions is formed as p + lo with
// p = fl(delta hi) and lo carrying the rounding error of that product (exact, from an FMA) plus
// delta lo.  k = rint(64 p) is split off exactly (Sterbenz), leaving |2 pi u| <= pi/64 + tiny,
// where sin to the 3rd and cos to the 4th power of 2 pi u are truncated below 3e-9.  One complex
// product with the entry of k mod 64 finishes it: about 1e-7 absolute error in a CPU emulation
// over phases up to 16 turns.  The hardware v_sin_f32 / v_cos_f32 are not used: their error
// (about 1e-6 absolute, judging by the parity errors they caused) is carried into the delta
// gradient with a factor |A|, beyond the fp32 tolerance.
__device__ __forceinline__ void cis_delta_tab(float delta, RevPair a, const float2* tab, float& c,
                                              float& s) {
  constexpr float S1 = (float)kTwoPiD;
  constexpr float S3 = (float)(-kTwoPiD * kTwoPiD * kTwoPiD / 6.0);
  constexpr float C2 = (float)(-kTwoPiD * kTwoPiD / 2.0);
  constexpr float C4 = (float)(kTwoPiD * kTwoPiD * kTwoPiD * kTwoPiD / 24.0);
  const float p = delta * a.hi;
  const float lo = fmaf(delta, a.lo, fmaf(delta, a.hi, -p));
  const float k = __builtin_rintf(64.f * p);
  const float u = fmaf(k, -1.f / 64.f, p) + lo;
  const float z = u * u;
  const float su = u * fmaf(z, S3, S1);
  const float cu = fmaf(z, fmaf(z, C4, C2), 1.f);
  const float2 e = tab[(int)k & 63];
  c = fmaf(e.x, cu, -e.y * su);
  s = fmaf(e.y, cu, e.x * su);
}

// (2 pi)^m / m! and 1 / m!, the Taylor coefficients of the fp64 rotation and exponential.
constexpr double taylor_2pi(int m) {
  double r = 1.0;
  for (int i = 1; i <= m; ++i) r *= kTwoPiD / i;
  return r;
}
constexpr double inv_fact(int m) {
  double r = 1.0;
  for (int i = 1; i <= m; ++i) r /= i;
  return r;
}

// e^(2 pi i r) in fp64 for r in revolutions (it builds the rotation tables below): k = rint(4 r)
// quarter turns are split off exactly, then the Taylor series of sin to the 15th and of cos to
// the 16th power of 2 pi u (truncated below 5e-17 for |2 pi u| <= pi/4), and k mod 4 rotates
// the pair by quarter turns (bit 1 of k and of k + 1 give the signs).
struct CisD {
  double c, s;
};
__device__ __forceinline__ CisD cis_rev_d(double r) {
  const double k = __builtin_rint(4.0 * r);
  const double u = __builtin_fma(k, -0.25, r);
  const double z = u * u;
  double ps = __builtin_fma(z, -taylor_2pi(15), taylor_2pi(13));
  ps = __builtin_fma(z, ps, -taylor_2pi(11));
  ps = __builtin_fma(z, ps, taylor_2pi(9));
  ps = __builtin_fma(z, ps, -taylor_2pi(7));
  ps = __builtin_fma(z, ps, taylor_2pi(5));
  ps = __builtin_fma(z, ps, -taylor_2pi(3));
  ps = __builtin_fma(z, ps, taylor_2pi(1));
  const double sn = u * ps;
  double pc = __builtin_fma(z, taylor_2pi(16), -taylor_2pi(14));
  pc = __builtin_fma(z, pc, taylor_2pi(12));
  pc = __builtin_fma(z, pc, -taylor_2pi(10));
  pc = __builtin_fma(z, pc, taylor_2pi(8));
  pc = __builtin_fma(z, pc, -taylor_2pi(6));
  pc = __builtin_fma(z, pc, taylor_2pi(4));
  pc = __builtin_fma(z, pc, -taylor_2pi(2));
  const double cs = __builtin_fma(z, pc, 1.0);
  const int q = (int)k;
  const bool odd = (q & 1) != 0;
  const double cr = odd ? sn : cs, sr = odd ? cs : sn;
  return CisD{((q + 1) & 2) ? -cr : cr, (q & 2) ? -sr : sr};
}

constexpr double kLn2D = 0.6931471805599453;

// e^x in fp64 (it builds the table of 2^(j/32) below): x = k ln 2 + g with
// k = rint(x log2 e), |g| <= ln(2) / 2 + tiny, e^g from its Taylor series to g^13 (truncated
// below 5e-18), scaled by 2^k.  The reduction's rounding (k times the error of ln 2 in fp64) is
// below 1e-13 relative for |x| < 1000; results under the fp64 range flush to zero through
// ldexp.
__device__ __forceinline__ double exp_d(double x) {
  constexpr double kLog2eD = 1.4426950408889634;
  const double k = __builtin_rint(x * kLog2eD);
  const double g = __builtin_fma(-k, kLn2D, x);
  double p = __builtin_fma(g, inv_fact(13), inv_fact(12));
  p = __builtin_fma(p, g, inv_fact(11));
  p = __builtin_fma(p, g, inv_fact(10));
  p = __builtin_fma(p, g, inv_fact(9));
  p = __builtin_fma(p, g, inv_fact(8));
  p = __builtin_fma(p, g, inv_fact(7));
  p = __builtin_fma(p, g, inv_fact(6));
  p = __builtin_fma(p, g, inv_fact(5));
  p = __builtin_fma(p, g, inv_fact(4));
  p = __builtin_fma(p, g, inv_fact(3));
  p = __builtin_fma(p, g, 0.5);
  p = __builtin_fma(p, g, 1.0);
  p = __builtin_fma(p, g, 1.0);
  const double kc = k < -2000.0 ? -2000.0 : k;  // keeps the int conversion in range
  return ldexp(p, (int)kc);
}

// Tables for the fp64 exponential and rotation of the training path, built once per workgroup
// in LDS from exp_d and cis_rev_d: e^(2 pi i m / 64) for m < 64 and 2^(j / 32) for j < 32.  They
// make the reduced arguments 16 (rotation) and 32 (exponential) times smaller than in the
// functions above, so shorter series reach fp64 accuracy and the quarter-turn selects go away.
struct CTab {
  double2 cis[64];
  double p2[32];
};
// the fp32 rotation table of cis_delta_tab
__device__ inline void ctab_build_f32(float2* t, int tid, int nthr) {
  for (int m = tid; m < 64; m += nthr) {
    const CisD e = cis_rev_d(m / 64.0);
    t[m] = make_float2((float)e.c, (float)e.s);
  }
}
__device__ inline void ctab_build(CTab& t, int tid, int nthr) {
  for (int m = tid; m < 64; m += nthr) {
    const CisD e = cis_rev_d(m / 64.0);
    t.cis[m] = make_double2(e.c, e.s);
  }
  for (int j = tid; j < 32; j += nthr) t.p2[j] = exp_d(j * (kLn2D / 32.0));
}

// e^(2 pi i r) with the table: r = k/64 + u, k = rint(64 r), u exact (Sterbenz) with
// |2 pi u| <= pi/64; sin to the 9th and cos to the 8th power of 2 pi u (truncated below 1e-20),
// then one complex product with the table entry of k mod 64.
__device__ __forceinline__ CisD cis_rev_tab(double r, const CTab& t) {
  const double k = __builtin_rint(64.0 * r);
  const double u = __builtin_fma(k, -1.0 / 64.0, r);
  const double z = u * u;
  double ps = __builtin_fma(z, taylor_2pi(9), -taylor_2pi(7));
  ps = __builtin_fma(z, ps, taylor_2pi(5));
  ps = __builtin_fma(z, ps, -taylor_2pi(3));
  ps = __builtin_fma(z, ps, taylor_2pi(1));
  const double su = u * ps;
  double pc = __builtin_fma(z, taylor_2pi(8), -taylor_2pi(6));
  pc = __builtin_fma(z, pc, taylor_2pi(4));
  pc = __builtin_fma(z, pc, -taylor_2pi(2));
  const double cu = __builtin_fma(z, pc, 1.0);
  const double2 e = t.cis[(int)k & 63];
  return CisD{__builtin_fma(e.x, cu, -e.y * su), __builtin_fma(e.y, cu, e.x * su)};
}

// e^x with the table: x = (32 m + j) ln2/32 + g, k = 32 m + j = rint(32 x / ln 2),
// |g| <= ln2/64 + tiny; e^g from its series to g^6 (truncated below 4e-18), times 2^(j/32) from
// the table, scaled by 2^m.  The reduction's rounding is k times the error of ln2/32 in fp64,
// the same bound as exp_d's; results under the fp64 range flush to zero through ldexp.
__device__ __forceinline__ double exp_tab(double x, const CTab& t) {
  constexpr double kScale = 32.0 * 1.4426950408889634;  // 32 / ln 2
  double k = __builtin_rint(x * kScale);
  k = k < -1073741824.0 ? -1073741824.0 : k;  // keeps the int conversion in range
  const double g = __builtin_fma(-k, kLn2D / 32.0, x);
  double p = __builtin_fma(g, inv_fact(6), inv_fact(5));
  p = __builtin_fma(p, g, inv_fact(4));
  p = __builtin_fma(p, g, inv_fact(3));
  p = __builtin_fma(p, g, 0.5);
  p = __builtin_fma(p, g, 1.0);
  p = __builtin_fma(p, g, 1.0);
  const int ki = (int)k;
  return ldexp(p * t.p2[ki & 31], ki >> 5);
}

// Adds an fp64 value across the two 32-lane halves (both halves get the same sum).
__device__ __forceinline__ double half_sum_d(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  const auto rl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto rh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  const double a = __longlong_as_double((long long)(((uint64_t)rh[0] << 32) | rl[0]));
  const double b = __longlong_as_double((long long)(((uint64_t)rh[1] << 32) | rl[1]));
  return a + b;
}

// One complex element of an I/O array (B, C and their gradients) as it sits in a register
// between its load and its first use.
template <typename IO>
struct cio;

template <>
struct cio<float> {
  using raw = u32x2;
  static constexpr int es = 8;  // bytes per complex element
  static __device__ __forceinline__ raw bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  }
  static __device__ __forceinline__ float re(raw v) { return __uint_as_float(v.x); }
  static __device__ __forceinline__ float im(raw v) { return __uint_as_float(v.y); }
  static __device__ __forceinline__ void store(void* p, int64_t i, float re, float im) {
    float* q = static_cast<float*>(p) + 2 * i;
    q[0] = re;
    q[1] = im;
  }
};

template <>
struct cio<bf16_storage> {
  using raw = uint32_t;  // re in the low half, im in the high half (little-endian pair)
  static constexpr int es = 4;
  static __device__ __forceinline__ raw bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
  }
  static __device__ __forceinline__ float re(raw v) { return __uint_as_float(v << 16); }
  static __device__ __forceinline__ float im(raw v) { return __uint_as_float(v & 0xffff0000u); }
  // fp32 -> bf16 round to nearest even, each part
  static __device__ __forceinline__ void store(void* p, int64_t i, float re, float im) {
    __bf16* q = static_cast<__bf16*>(p) + 2 * i;
    q[0] = static_cast<__bf16>(re);
    q[1] = static_cast<__bf16>(im);
  }
};

// Adds v across the two 32-lane halves of a wavefront (lanes l and l ^ 32 both get the sum).
__device__ __forceinline__ float half_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace msm
