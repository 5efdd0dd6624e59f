// Cross-lane reductions and row-window buffer resources shared by the backward kernels
// (gfx950, wave64).
#pragma once

#include "msm_device.hpp"

namespace msm {

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// One reduce-scatter stage inside a 16-lane row: lanes are paired by the DPP pattern CTRL,
// partners differ in lane bit MASK; the lane with the bit set keeps the upper half.
template <int CTRL, int MASK, int H, int M>
__device__ __forceinline__ void rs_dpp(float (&v)[M], int lane) {
  const bool up = (lane & MASK) != 0;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float lo = v[i] + dpp<CTRL>(v[i]);
    const float hi = v[i + H] + dpp<CTRL>(v[i + H]);
    v[i] = up ? hi : lo;
  }
}

// Reduce-scatter of 32 values over each 32-lane half of a wavefront.  The pairings are
// lane^16 (permlane16 swap), lane^15 (row mirror), lane^7 within 8 (half-row mirror), lane^2
// and lane^1 (quad permutes); each pairs lanes that agree on the bits decided so far and
// differ in the next one (16, 8, 4, 2, 1), and together they cover all 32 lanes.  On return
// lane l holds in v[0] the sum over its half of value (l & 31).
__device__ __forceinline__ void reduce_scatter32(float (&v)[32], int lane) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    // after the swap, lanes 0-15 of each 32 hold (their v[i], partner's v[i]) and lanes 16-31
    // hold (partner's v[i+16], their v[i+16])
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]),
                                                    __float_as_uint(v[i + 16]), false, false);
    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  rs_dpp<0x140, 8, 8>(v, lane);  // row_mirror
  rs_dpp<0x141, 4, 4>(v, lane);  // row_half_mirror
  rs_dpp<0x4E, 2, 2>(v, lane);   // quad_perm [2,3,0,1]
  rs_dpp<0xB1, 1, 1>(v, lane);   // quad_perm [1,0,3,2]
}

// Adds a across the two halves of the wavefront for lanes 0-31 and b for lanes 32-63 (the
// same pairing trick as above, with v_permlane32_swap).
__device__ __forceinline__ float swap_add32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource for the rows of a (L, row_bytes) slab starting at row r; rows at or past
// the end read as zero and are never written.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int64_t r,
                                                             int64_t row_bytes, int64_t total) {
  const int64_t off = r * row_bytes;
  return make_rsrc(static_cast<const char*>(base) + off, total - off);
}

}  // namespace msm
