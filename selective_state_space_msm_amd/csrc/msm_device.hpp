// Device-side helpers shared by the forward and backward kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msm {

constexpr float kLog2e = 1.4426950408889634f;  // A is rescaled once so that a = 2^(delta*A2)

// 2^x on the transcendental unit (v_exp_f32, half rate on gfx950).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// log2(x) and 1/x on the transcendental unit (v_log_f32, v_rcp_f32; about 1 ulp each).
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

constexpr float kLn2 = 0.6931471805599453f;

// softplus(u) = log(1 + e^u) = max(u, 0) + log1p(e^-|u|).  log1p(e) is formed as
// log(w) * e / (w - 1) with w = 1 + e (Goldberg, "What every computer scientist should know
// about floating-point arithmetic", Theorem 4): the quotient cancels the rounding of 1 + e,
// so tiny e keep their relative accuracy; nothing overflows for any u.
__device__ __forceinline__ float softplus_f(float u) {
  const float e = exp2_fast(-fabsf(u) * kLog2e);
  const float w = 1.f + e;
  const float l1p = w == 1.f ? e : log2_fast(w) * kLn2 * (e * rcp_fast(w - 1.f));
  return fmaxf(u, 0.f) + l1p;
}

// logistic(z) = 1 / (1 + e^-z) and 1 - logistic(z), both from e = e^-|z| <= 1 (no overflow,
// no cancellation in the complement).
struct Logistic {
  float s, sc;
};
__device__ __forceinline__ Logistic logistic_f(float z) {
  const float e = exp2_fast(-fabsf(z) * kLog2e);
  const float r = rcp_fast(1.f + e);
  const float er = e * r;
  return z >= 0.f ? Logistic{r, er} : Logistic{er, r};
}

// SiLU gate z * logistic(z) and its derivative logistic(z) (1 + z (1 - logistic(z))).
__device__ __forceinline__ float silu_f(float z) { return z * logistic_f(z).s; }
__device__ __forceinline__ float silu_grad_f(float z) {
  const Logistic l = logistic_f(z);
  return l.s * fmaf(z, l.sc, 1.f);
}

// Zero-order hold.  The write coefficient is g = (e^u - 1) / A = delta phi(u) with u = delta A,
// phi(u) = (e^u - 1) / u, and dg/dA = delta^2 psi(u) with psi(u) = (u e^u - e^u + 1) / u^2.
// Near u = 0 both quotients cancel, so they come from their Taylor series there
// (phi = sum u^k / (k+1)!, psi = sum (k+1) u^k / (k+2)!, truncated below 2e-9 relative for
// |u| < 1/4); elsewhere from a = e^u, which keeps its relative accuracy in a - 1 and a - phi.
__device__ __forceinline__ float zoh_phi(float u, float a) {
  float p = fmaf(u, 1.f / 5040.f, 1.f / 720.f);
  p = fmaf(p, u, 1.f / 120.f);
  p = fmaf(p, u, 1.f / 24.f);
  p = fmaf(p, u, 1.f / 6.f);
  p = fmaf(p, u, 0.5f);
  p = fmaf(p, u, 1.f);
  const float q = (a - 1.f) * rcp_fast(u);
  return fabsf(u) < 0.25f ? p : q;
}
// phi alone, for the kernels that never need psi (forward and decode step): the series switches
// at |u| = 1/8 and stops at u^4 (truncation below 5e-8 relative).  Above the switch a - 1 >= 0.117
// in magnitude, so its rounding stays below about 1e-6 relative.  psi's (a - phi) / u would lose
// more than that to cancellation at the lower switch, so the backward keeps zoh_phi.
__device__ __forceinline__ float zoh_phi_fwd(float u, float a) {
  float p = fmaf(u, 1.f / 120.f, 1.f / 24.f);
  p = fmaf(p, u, 1.f / 6.f);
  p = fmaf(p, u, 0.5f);
  p = fmaf(p, u, 1.f);
  const float q = (a - 1.f) * rcp_fast(u);
  return fabsf(u) < 0.125f ? p : q;
}
// The forward's write coefficient g = delta phi(delta A) = (e^(delta A) - 1) / A itself, from
// arg = delta A log2 e, a = 2^arg and invA = 1 / A (0 for A = 0).  Below |delta A| = 1/8 it is
// delta times the same degree-4 series, evaluated in arg (coefficient k is ln 2^k / (k + 1)!);
// above, (a - 1) / A = a invA - invA in one FMA, with the same rounding as (a - 1) / u above:
// no reciprocal per update.
__device__ __forceinline__ float zoh_g_fwd(float arg, float a, float delta, float invA) {
  float p = fmaf(arg, 0.0019236258215256953f, 0.013876027166205394f);
  p = fmaf(p, arg, 0.08007550231970023f);
  p = fmaf(p, arg, 0.34657359027997264f);
  p = fmaf(p, arg, 1.f);
  const float q = fmaf(a, invA, -invA);
  return fabsf(arg) < 0.18033688f ? delta * p : q;
}
__device__ __forceinline__ float zoh_psi(float u, float a, float phi) {
  float p = fmaf(u, 1.f / 5760.f, 1.f / 840.f);
  p = fmaf(p, u, 1.f / 144.f);
  p = fmaf(p, u, 1.f / 30.f);
  p = fmaf(p, u, 1.f / 8.f);
  p = fmaf(p, u, 1.f / 3.f);
  p = fmaf(p, u, 0.5f);
  const float q = (a - phi) * rcp_fast(u);
  return fabsf(u) < 0.25f ? p : q;
}

// The backward's zero-order-hold quantities from arg = delta A log2 e, a = 2^arg, delta and
// invA = 1 / A (0 for A = 0): the write coefficient g = delta phi(delta A) and its derivative
// dg/dA = delta^2 psi(delta A).  Below |delta A| = 1/4 they come from the degree-6 series of
// zoh_phi and zoh_psi, evaluated in arg (coefficient k carries ln 2^k); above it from
// g = (a - 1) / A and dg/dA = (delta a - g) / A, with no reciprocal per update.
constexpr float kZohSwitchArg = 0.36067376f;  // |delta A| = 1/4 in units of log2 e
__device__ __forceinline__ float zoh_g_bwd(float arg, float a, float delta, float invA) {
  float p = fmaf(arg, 2.2005043419116583e-05f, 0.0002222259691071407f);
  p = fmaf(p, arg, 0.0019236258215256953f);
  p = fmaf(p, arg, 0.013876027166205394f);
  p = fmaf(p, arg, 0.08007550231970023f);
  p = fmaf(p, arg, 0.34657359027997264f);
  p = fmaf(p, arg, 1.f);
  const float q = fmaf(a, invA, -invA);
  return fabsf(arg) < kZohSwitchArg ? delta * p : q;
}
// g as zoh_g_bwd returned it
__device__ __forceinline__ float zoh_gA_bwd(float arg, float a, float delta, float invA, float g) {
  float p = fmaf(arg, 1.9254412991727008e-05f, 0.0001904794020918349f);
  p = fmaf(p, arg, 0.0016030215179380794f);
  p = fmaf(p, arg, 0.011100821732964315f);
  p = fmaf(p, arg, 0.06005662673977517f);
  p = fmaf(p, arg, 0.23104906018664842f);
  p = fmaf(p, arg, 0.5f);
  const float q = fmaf(delta, a, -g) * invA;
  return fabsf(arg) < kZohSwitchArg ? (delta * delta) * p : q;
}

struct bf16_storage {
  uint16_t bits;
};

// Raw buffer resource over `bytes` bytes starting at `base` (gfx9-family descriptor word 3).
// A load whose per-lane offset is at or past the extent returns 0 without touching memory and
// a store there is dropped; the kernels use this for rows past the end of a chunk.  Extents
// are clamped to [0, 2^31 - 1]; every offset a kernel uses stays far below that bound.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_u32(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}
// Buffer resource for the `rows` rows of a slab that start at row r (0 <= r < 2^31; rows <= 0
// gives an empty resource).  The resource spans that tile alone, so its extent and the row
// offset need 32-bit arithmetic only, whatever the slab's size, as long as the tile's bytes fit
// in 31 bits; accesses at or past `rows` rows are dropped (stores) or read zero (loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int32_t r,
                                                             int32_t rows, uint32_t row_bytes) {
  const uint64_t off = (uint64_t)(uint32_t)r * row_bytes;
  return make_rsrc_u32(static_cast<const char*>(base) + off,
                       rows > 0 ? (uint32_t)rows * row_bytes : 0u);
}

// I/O element access.  "raw" is what sits in a register between the load and its first use.
template <typename IO>
struct io;

template <>
struct io<float> {
  using raw = float;
  static constexpr int es = 4;
  // delta * x from the raw values
  static __device__ __forceinline__ float mul_raw(raw a, raw b) { return a * b; }
  static __device__ __forceinline__ raw load(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  // element `lane` of the row starting at element `row` (row is wavefront-uniform, so the
  // address is a scalar base plus a 32-bit per-lane offset)
  static __device__ __forceinline__ raw load_row(const void* p, int64_t row, uint32_t lane) {
    return (static_cast<const float*>(p) + row)[lane];
  }
  static __device__ __forceinline__ void store_row(void* p, int64_t row, uint32_t lane, float v) {
    (static_cast<float*>(p) + row)[lane] = v;
  }
  static __device__ __forceinline__ raw bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
  }
  static __device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                uint32_t soff, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
  }
  static __device__ __forceinline__ float widen(raw r) { return r; }
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
};

template <>
struct io<bf16_storage> {
  using raw = uint32_t;  // the 16 bf16 bits, zero-extended
  static constexpr int es = 2;
  // delta * x from the raw bits: widen both (exact) and multiply
  static __device__ __forceinline__ float mul_raw(raw a, raw b) {
    return __uint_as_float(a << 16) * __uint_as_float(b << 16);
  }
  static __device__ __forceinline__ raw load(const void* p, int64_t i) {
    return static_cast<const uint16_t*>(p)[i];
  }
  static __device__ __forceinline__ raw load_row(const void* p, int64_t row, uint32_t lane) {
    return (static_cast<const uint16_t*>(p) + row)[lane];
  }
  static __device__ __forceinline__ void store_row(void* p, int64_t row, uint32_t lane, float v) {
    (static_cast<__bf16*>(p) + row)[lane] = static_cast<__bf16>(v);
  }
  static __device__ __forceinline__ raw bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
  }
  static __device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                uint32_t soff, float v) {
    const __bf16 hv = static_cast<__bf16>(v);
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, hv), r, voff, soff, 0);
  }
  // bf16 -> fp32 is exact: the bf16 bits are the upper half of the fp32 pattern.
  static __device__ __forceinline__ float widen(raw r) { return __uint_as_float(r << 16); }
  // fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32).
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    static_cast<__bf16*>(p)[i] = static_cast<__bf16>(v);
  }
};

}  // namespace msm
