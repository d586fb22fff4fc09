// Index arithmetic shared by the GEMM kernels and their host-side checks.
//
// Everything here is pure integer math, usable from device code and from a
// plain C++ host compiler (the unit test builds it with g++ and checks that
// every map is a bijection that stays inside its buffer and that fragment
// reads spread over distinct LDS banks).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define CODA_HD __host__ __device__ __forceinline__
#else
#define CODA_HD inline
#endif

namespace coda {

// Macro tile: 256 x 256 outputs per workgroup of 8 wavefronts (2 x 4, two per
// SIMD), each wavefront owning a 128 x 64 sub-tile.  One k-tile is 64 bytes of
// the contraction per operand row (32 bf16 or 16 fp32).  Four LDS stages
// (4 x 32 KiB of a CU's 160 KiB).  A fifth stage, which gives the loads one
// more step to land, measured 0.6-2.7% slower at the 7B, 70B and 1B second
// GEMM shapes (bf16 and fp8) with bit-identical results.
constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveM = 128;                         // rows of a wavefront's sub-tile
constexpr int kWaveN = 64;                          // columns of a wavefront's sub-tile
constexpr int kFragM = kWaveM / 16;                 // 16-row A fragments per wavefront: 8
constexpr int kFragN = kWaveN / 16;                 // 16-column B fragments per wavefront: 4
constexpr int kKTBytes = 64;                        // contraction bytes per row per k-tile
constexpr int kOperandBytes = kTileM * kKTBytes;    // one operand, one k-tile: 16 KiB
constexpr int kStageBytes = 2 * kOperandBytes;      // A + B: 32 KiB
constexpr int kStages = 4;
constexpr int kDmaSlots = kOperandBytes / (kWaves * 1024);  // 1 KiB DMA blocks per wave per operand: 2
constexpr int kEpiPitch = kWaveN + 4;               // floats per row of the epilogue slab
constexpr int kEpiSlabBytes = 16 * kEpiPitch * 4;   // one wavefront's 16-row slab
constexpr int kPartialCols = kWaveN;                // columns per partial-RMS tile

// ---- contraction-contiguous ("KC") operand tile ---------------------------
// 256 operand rows x 64 bytes (four 16-byte chunks).  Chunk c of row r is
// stored at chunk position c ^ ((r ^ (r >> 2)) & 3).  A fragment read takes
// one chunk of 16 consecutive rows; with this swizzle every 4, 8 and 16
// consecutive lanes of it hit distinct 16-byte bank groups within a 64-,
// 128- and 256-byte window, so the read is conflict-free however the LDS
// groups the lanes of a 16-byte read.  (With (r >> 2) & 3 alone only the
// 16-lane window is conflict-free; 8 consecutive lanes then meet 2-way.)
CODA_HD int kc_swizzle(int r) { return (r ^ (r >> 2)) & 3; }
CODA_HD int kc_offset(int r, int c) { return r * kKTBytes + ((c ^ kc_swizzle(r)) << 4); }

// ---- tile-packed contraction-contiguous ("KP") operand -----------------
// A contraction-contiguous bf16 matrix may also be stored tile-packed, in the
// order the fragment reads want: for row block R = row / 16 and 16-byte chunk
// c of the contraction (8 bf16), the chunks of the block's 16 rows lie
// together,
//   element (row, 8 c + e) at 16-byte unit (R nck + c) 16 + row % 16, byte 2 e,
// with nck chunks per row and the rows padded to a multiple of 16.  One
// k-tile of 16 rows is then 1 KiB contiguous in memory, and the LDS tile
// keeps that order: [row block][chunk 0..3][row % 16][16 B].  The 16 lanes
// of a fragment read take 256 contiguous bytes, which the LDS serves at full
// rate (the KC layout's 16-byte reads gather 16 rows 64 bytes apart and run
// at half rate), and every direct load reads 1 KiB of consecutive memory.
CODA_HD int kp_offset(int r, int c) { return ((r >> 4) * 4 + c) * 256 + (r & 15) * 16; }
// KP direct loads: block b of the tile is row block b; lane L -> row
// 16 b + L % 16, chunk L / 16 (position 16 L of the block, as kp_offset).
CODA_HD void dma_kp(int s, int w, int L, int* row, int* chunk) {
  const int b = s * kWaves + w;
  *row = 16 * b + (L & 15);
  *chunk = L >> 4;
}
// 16-byte unit holding chunk c of row r in a packed matrix of nck chunks per row.
CODA_HD int64_t kp_unit(int64_t r, int64_t c, int64_t nck) { return ((r >> 4) * nck + c) * 16 + (r & 15); }

// ---- row-contiguous ("RC") operand tile --------------------------------
// The contraction runs across memory rows: KTE contraction rows (32 bf16 /
// 16 fp32) of 256 operand elements (512 / 1024 bytes).  16-byte chunk c of
// contraction row k is stored at chunk position c ^ rc_swizzle(k), an even
// XOR (whole 32-byte segments move) that spreads the 16 rows one transposing
// fragment read touches over all banks, each bank exactly twice.
CODA_HD int rc_swizzle(int k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }
CODA_HD int rc_row_bytes(int E) { return kTileM * (16 / E); }  // E elements per chunk
CODA_HD int rc_offset(int k, int c, int E) { return k * rc_row_bytes(E) + ((c ^ rc_swizzle(k)) << 4); }

// ---- HBM -> LDS direct loads ---------------------------------------------
// Each load instruction of a wavefront writes one contiguous 1 KiB LDS block,
// lane L's 16 bytes at block + 16 L.  Slot s of wavefront w fills block
// b = kWaves s + w of the operand tile; the maps below give the logical
// element each lane must fetch so that the block holds the swizzled layout.
//
// KC: block b holds rows 16 b .. 16 b + 15; lane L -> row 16 b + L/4,
//     logical chunk (L % 4) ^ kc_swizzle(row).
CODA_HD void dma_kc(int s, int w, int L, int* row, int* chunk) {
  const int b = s * kWaves + w;
  *row = 16 * b + (L >> 2);
  *chunk = (L & 3) ^ kc_swizzle(*row);
}
// RC: block b holds 1024 / row_bytes contraction rows; lane L -> contraction
//     row k and logical chunk c (operand elements c*E .. c*E + E - 1).
CODA_HD void dma_rc(int s, int w, int L, int E, int* k, int* chunk) {
  const int b = s * kWaves + w;
  const int chunks_per_row = rc_row_bytes(E) / 16;  // 32 (bf16) or 64 (fp32)
  const int pos = b * 64 + L;                        // 16-byte position within the tile
  *k = pos / chunks_per_row;
  *chunk = (pos % chunks_per_row) ^ rc_swizzle(*k);
}

// ---- MFMA fragment reads (16 x 16 x 32 bf16 / 16 x 16 x 4 fp32) -----------
// Lane l = 16 g + i.  Fragment t of a wavefront covers operand rows
// base + 16 t .. + 15; lane l supplies operand row base + 16 t + i and
// contraction elements [g*E, g*E + E) of the k-tile (E = 8 bf16, 4 fp32).
//
// KC: one 16-byte read at kc_offset(base + 16 t + i, g).
//
// RC bf16: two 8-byte transposing reads (ds_read_b64_tr_b16), h = 0, 1.
// Within each 16-lane group the hardware hands lane i the i-th 16-bit value
// of every 16-lane stripe of the group's concatenated reads.  Lane j of the
// group reads 4 consecutive operand elements at contraction row
// 8 g + 4 h + j / 4, operand columns base + 16 t + 4 (j % 4) .. + 3; lane i
// then receives operand column base + 16 t + i at contraction rows
// 8 g + 4 h .. + 3, exactly the MFMA operand layout.
CODA_HD int rc_tr_offset(int base, int t, int h, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int k = 8 * g + 4 * h + (j >> 2);
  const int col = base + 16 * t + 4 * (j & 3);  // first of 4 bf16 elements
  const int c = col >> 3, within = (col & 7) * 2;
  return rc_offset(k, c, 8) + within;
}
// For bf16 the t dependence is a single XOR: the swizzle and t both act on
// address bits 5..7 only and every other term leaves those bits clear, so
// rc_tr_offset(base, t, h, lane) == rc_tr_offset(base, 0, h, lane) ^ (32 t)
// for base a multiple of 128 (checked on the host).
CODA_HD int rc_tr_lane_base(int base, int h, int lane) { return rc_tr_offset(base, 0, h, lane); }
// RC fp32: four 4-byte reads, u = 0..3: contraction row 4 g + u, operand
// column base + 16 t + i (feeding the u-th K=4 product).
CODA_HD int rc_f32_offset(int base, int t, int u, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int k = 4 * g + u;
  const int col = base + 16 * t + i;
  return rc_offset(k, col >> 2, 4) + (col & 3) * 4;
}

// SwiGLU operand order.  For the gated second GEMM the B operand is
// W2 = [W_gate | W_up] (columns [0, F) and [F, 2F)); the kernel reads it in
// a logical column order that alternates kSwiGLURun-column runs of the two
// halves: logical run 2m holds gate columns kSwiGLURun m .. + kSwiGLURun - 1
// and run 2m+1 the matching up columns F + kSwiGLURun m ...  Runs of 32
// columns keep 4 consecutive lanes of a direct load on one contiguous 64-byte
// segment.  An epilogue lane holding 8 columns of run 2m and lane l ^ 4
// (8 columns further in run 2m+1) then have the gate and up values of the
// same 8 output columns.  F must be a multiple of kSwiGLURun.
constexpr int kSwiGLURun = 32;
CODA_HD int swiglu_col(int n, int F) {
  const int c = n / kSwiGLURun;
  return ((c & 1) ? F : 0) + (c >> 1) * kSwiGLURun + n % kSwiGLURun;
}
// Output column of logical column n (gate or up), and whether n is an up column.
CODA_HD int swiglu_out_col(int n) { return (n / (2 * kSwiGLURun)) * kSwiGLURun + n % kSwiGLURun; }
CODA_HD bool swiglu_is_up(int n) { return ((n / kSwiGLURun) & 1) != 0; }
// The epilogue lane holding the up values for a gate lane (and vice versa).
constexpr int kSwiGLUPartner = kSwiGLURun / 8;

// ---- fp8 (e4m3) operands: v_mfma_f32_32x32x64_f8f6f4 ---------------------
// One k-tile is 64 bytes = 64 fp8 elements per operand row, so both operands
// use the contraction-contiguous layout above unchanged.  A wavefront's
// 128 x 64 sub-tile is 4 x 2 products of 32 x 32.  Lane l = 32 g + i of a
// 32-row fragment t supplies operand row base + 32 t + i and two 16-byte
// chunks of the k-tile: chunk g in its first four registers (half 0) and
// chunk 2 + g in its last four (half 1).  The matrix core takes the first
// registers of both lane halves as contraction block 0 and the last as block
// 1, with block 0's scale from lane i and block 1's from lane 32 + i (a GPU
// probe with a different exponent per block showed this), so the k-tile's
// bytes [0, 32) and [32, 64) are exactly its two scale blocks, as the
// microscaling formats need.  Unscaled products only need the same
// (lane, byte) -> k assignment on both operands.
constexpr int kFrag8M = kWaveM / 32;  // 4 fragments of 32 A rows
constexpr int kFrag8N = kWaveN / 32;  // 2 fragments of 32 B rows
CODA_HD int kc8_offset(int base, int t, int half, int lane) {
  return kc_offset(base + 32 * t + (lane & 31), (lane >> 5) + 2 * half);
}
// MX block exponents (one E8M0 byte per row and 32 contraction columns), in
// the order the second GEMM's lanes take them.  Rows come in blocks of 128
// (a wavefront's A rows); within a block, row 32 mt + l of k-tile t, half h
// is the scale that lane 32 h + l supplies for A fragment mt (tile_map's
// 32-row fragments).  Byte mx_byte(i, t, h, M) of an array for M rows:
//   ((t / 4 * ceil(M / 128) + i / 128) * 64 + 32 h + i % 32) * 16
//     + ((i / 32) % 4) * 4 + t % 4
// so a lane's 16 bytes hold, for one group of 4 k-tiles, its 4 fragments'
// dwords (one k-tile per byte), and a wavefront's 64 lanes read one 1 KiB
// block per group.  The array spans 1024 ceil(M / 128) ceil(cols / 256)
// bytes; the rows past M in the last block are padding.
CODA_HD int64_t mx_row_blocks(int64_t M) { return (M + 127) / 128; }
CODA_HD int64_t mx_byte(int64_t i, int t, int h, int64_t M) {
  return (((int64_t)(t >> 2) * mx_row_blocks(M) + (i >> 7)) * 64 + 32 * h + (i & 31)) * 16 + ((i >> 5) & 3) * 4 +
         (t & 3);
}
// Accumulator element e (0..15) of lane l in a 32 x 32 product is output
// row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32 (established by a GPU
// probe against a host product).  Epilogue slab s (16 rows) is half s % 2 of
// row fragment s / 2 and holds elements e = 8 (s % 2) .. 8 (s % 2) + 7.
CODA_HD int acc32_row(int e, int lane) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

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

}  // namespace coda
