// Index arithmetic shared by the GEMM kernels and their host-side checks.
//
// Everything here is pure integer math, usable from device code and from a
// plain C++ host compiler (the unit test builds it with g++ and checks that
// every map is a bijection that stays inside its buffer).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define CODA_HD __host__ __device__ __forceinline__
#else
#define CODA_HD inline
#endif

namespace coda {

// Macro tile: 256 x 256 outputs per workgroup of 4 wavefronts (2 x 2), each
// wavefront owning a 128 x 128 sub-tile.  One k-tile is 128 bytes of the
// contraction per operand row (64 bf16 or 32 fp32), i.e. eight 16-byte chunks.
constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kThreads = 256;
constexpr int kRowBytes = 128;
constexpr int kChunks = 8;
constexpr int kStageBytes = kTileM * kRowBytes;  // one operand, one k-tile: 32 KiB
constexpr int kEpiPitch = 132;                   // floats per row of the epilogue slab
constexpr int kPartialCols = 128;                // columns per partial-RMS tile

// LDS placement of chunk `c` (0..7) of tile row `row`.  The chunk index is
// XOR-swizzled with a function of the row so that the 16 rows one MFMA
// fragment read touches land on distinct banks for both 32- and 64-bank
// views of the LDS (rows r and r+8 get different swizzles).
CODA_HD int lds_swizzle(int row) { return (row ^ (row >> 3)) & 7; }
CODA_HD int lds_offset(int row, int c) { return row * kRowBytes + ((c ^ lds_swizzle(row)) << 4); }

// Workgroup -> output tile.  The dispatcher places workgroup b on XCD b % 8;
// each XCD is given a contiguous range of logical tile ids so that tiles
// sharing A rows / B columns share that XCD's L2.  Logical ids are then laid
// out in groups of `group_m` tile rows that sweep the tile columns together.
CODA_HD void map_tile(int b, int tiles_m, int tiles_n, int group_m, int* tm, int* tn) {
  const int nb = tiles_m * tiles_n;
  const int q = nb / 8, rem = nb % 8, x = b % 8, i = b / 8;
  const int logical = (x < rem) ? x * (q + 1) + i : rem * (q + 1) + (x - rem) * q + i;
  const int per_group = group_m * tiles_n;
  const int gidx = logical / per_group;
  const int first_m = gidx * group_m;
  const int gsize = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const int within = logical - gidx * per_group;
  *tm = first_m + within % gsize;
  *tn = within / gsize;
}

// Staging of one k-tile of one operand (kTileM rows x kRowBytes) by the
// workgroup's 256 threads, eight 16-byte registers per thread.
//
// Contraction-contiguous operand: thread t, slot i handles chunk id = i*256+t,
// row id/8, chunk id%8 (one global 16-byte load, one LDS 16-byte store).
CODA_HD void kc_slot(int tid, int i, int* row, int* chunk) {
  const int id = i * kThreads + tid;
  *row = id >> 3;
  *chunk = id & 7;
}

// Row-contiguous operand (the contraction runs across rows of memory): the
// tile is cut into E x E element blocks (E elements per chunk); block id
// = i*256 + t covers tile rows [rb*E, rb*E+E) and contraction chunk kb.  The
// thread loads E global chunks (one per contraction index), transposes the
// E x E block in registers and stores E LDS chunks (one per tile row).
CODA_HD void rc_block(int tid, int i, int E, int* rb, int* kb) {
  const int id = i * kThreads + tid;
  const int per_k = kTileM / E;
  *rb = id % per_k;
  *kb = id / per_k;
}

// Byte permute of two dwords (the semantics of v_perm_b32 for selector bytes
// 0..7): byte b of the result is byte sel.b of the 8-byte value {hi, lo}, lo
// supplying bytes 0..3.
CODA_HD uint32_t perm_bytes(uint32_t hi, uint32_t lo, uint32_t sel) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_perm(hi, lo, sel);
#else
  const uint64_t v = ((uint64_t)hi << 32) | lo;
  uint32_t r = 0;
  for (int b = 0; b < 4; ++b) r |= (uint32_t)((v >> (8 * ((sel >> (8 * b)) & 7))) & 0xff) << (8 * b);
  return r;
#endif
}

// Transpose of an 8 x 8 block of 16-bit values held as 8 rows of 4 dwords
// (two values per dword, the lower column in the low half): out[c] is column
// c of `in`, packed the same way.
CODA_HD void transpose8x8_b16(const uint32_t (&in)[8][4], uint32_t (&out)[8][4]) {
  for (int c = 0; c < 8; ++c)
    for (int p = 0; p < 4; ++p)
      out[c][p] = perm_bytes(in[2 * p + 1][c >> 1], in[2 * p][c >> 1], (c & 1) ? 0x07060302u : 0x05040100u);
}

}  // namespace coda
