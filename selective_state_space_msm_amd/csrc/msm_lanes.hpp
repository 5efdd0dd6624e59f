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

// The stages paired by lane bit 8 (row_mirror) and lane bit 4 (row_half_mirror) split the
// lanes along DPP banks (groups of 4 lanes of a 16-lane row): lanes 8-15 of a row are banks
// 2-3, lanes with bit 4 set are banks 1 and 3.  There each output is two DPP adds, one per
// bank mask, each writing only the lanes that keep that half: 2 instructions instead of the 2
// adds and a select of rs_dpp (the compiler folds a DPP move into its add only with full
// masks, hence the inline assembly).  A DPP read of a VGPR needs 2 wait states after the VALU
// instruction that wrote it, and the hazard check does not look inside inline assembly, so
// each block starts and ends with s_nop 1.  Outputs are early-clobber: a bank-masked write
// leaves the other lanes of its destination unchanged until the second add fills them.
#define MSM_RS_PAIR(CTRL, LO, UP, o, a, b)                                               \
  "v_add_f32_dpp %" #o ", %" #a ", %" #a " " CTRL " row_mask:0xf bank_mask:" LO "\n\t" \
  "v_add_f32_dpp %" #o ", %" #b ", %" #b " " CTRL " row_mask:0xf bank_mask:" UP "\n\t"

__device__ __forceinline__ void rs_bank8(float (&v)[32]) {
  float o[8];
  asm("s_nop 1\n\t"
      MSM_RS_PAIR("row_mirror", "0x3", "0xc", 0, 8, 16)
      MSM_RS_PAIR("row_mirror", "0x3", "0xc", 1, 9, 17)
      MSM_RS_PAIR("row_mirror", "0x3", "0xc", 2, 10, 18)
      MSM_RS_PAIR("row_mirror", "0x3", "0xc", 3, 11, 19)
      MSM_RS_PAIR("row_mirror", "0x3", "0xc", 4, 12, 20)
      MSM_RS_PAIR("row_mirror", "0x3", "0xc", 5, 13, 21)
      MSM_RS_PAIR("row_mirror", "0x3", "0xc", 6, 14, 22)
      MSM_RS_PAIR("row_mirror", "0x3", "0xc", 7, 15, 23)
      "s_nop 1"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7])
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]),
        "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]),
        "v"(v[15]));
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = o[i];
}

__device__ __forceinline__ void rs_bank4(float (&v)[32]) {
  float o[4];
  asm("s_nop 1\n\t"
      MSM_RS_PAIR("row_half_mirror", "0x5", "0xa", 0, 4, 8)
      MSM_RS_PAIR("row_half_mirror", "0x5", "0xa", 1, 5, 9)
      MSM_RS_PAIR("row_half_mirror", "0x5", "0xa", 2, 6, 10)
      MSM_RS_PAIR("row_half_mirror", "0x5", "0xa", 3, 7, 11)
      "s_nop 1"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = o[i];
}
#undef MSM_RS_PAIR

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
  rs_bank8(v);                   // row_mirror
  rs_bank4(v);                   // row_half_mirror
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
