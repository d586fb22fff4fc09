// Lane exchanges within groups of 8 lanes through DPP, an operand modifier
// of the vector ALU: the value moves between lanes inside the instruction,
// with no LDS round trip and no wait (a __shfl_xor is a ds_bpermute, an LDS
// instruction the next use must wait for).  The epilogues reduce over the 8
// lanes that hold one row's 64 columns, once or twice per 16-row slab.
//
// DPP controls used (CDNA3/CDNA4 ISA, DPP_CTRL):
//   quad_perm [1,0,3,2] = 0xB1   lane i reads lane i ^ 1
//   quad_perm [2,3,0,1] = 0x4E   lane i reads lane i ^ 2
//   row_shl:4 = 0x104            lane i reads lane i + 4 of its 16-lane row
//   row_shr:4 = 0x114            lane i reads lane i - 4 of its 16-lane row
//   row_half_mirror = 0x141      lane i reads lane 7 - i of its 8-lane half row
// The bank mask selects which groups of 4 lanes of a row are written; the
// others keep the `old` operand.
#pragma once

#include <hip/hip_runtime.h>

namespace coda {

template <int CTRL, int BANKS = 0xF>
__device__ __forceinline__ float dpp_move(float old, float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, x), CTRL, 0xF, BANKS, false));
}

// x of lane i ^ 1, i ^ 2 and i ^ 4.
__device__ __forceinline__ float lane_xor1(float x) { return dpp_move<0xB1>(x, x); }
__device__ __forceinline__ float lane_xor2(float x) { return dpp_move<0x4E>(x, x); }
__device__ __forceinline__ float lane_xor4(float x) {
  // lanes 0-3 of each 8 read 4 lanes up (banks 0 and 2 of the row), lanes
  // 4-7 read 4 lanes down (banks 1 and 3)
  return dpp_move<0x114, 0xA>(dpp_move<0x104, 0x5>(x, x), x);
}
// x of the lane holding the same position in the other quad of the 8-lane
// group, mirrored: lane i reads lane 7 - i.  After a reduction over each
// quad every lane of a quad holds the same value, so this gives each lane
// the other quad's result, as lane_xor4 would, in one instruction.
__device__ __forceinline__ float lane_other_quad(float x) { return dpp_move<0x141>(x, x); }

// The sum over the 8 lanes of each group, in every lane.  Each lane adds the
// same pairs as with exchanges i ^ 1, i ^ 2, i ^ 4 (a + b = b + a exactly),
// so the result is bit-identical to that order.
__device__ __forceinline__ float sum8(float s) {
  s += lane_xor1(s);
  s += lane_xor2(s);
  return s + lane_other_quad(s);
}

// The maximum over the 4 lanes of each quad, in every lane.
__device__ __forceinline__ float max4(float a) {
  a = fmaxf(a, lane_xor1(a));
  return fmaxf(a, lane_xor2(a));
}

}  // namespace coda
