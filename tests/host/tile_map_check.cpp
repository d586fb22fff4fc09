// Host-side checks of the GEMM kernels' index maps (built with g++, no GPU):
// every map is a bijection onto its buffer and never leaves it, the LDS
// swizzle spreads MFMA fragment reads over distinct banks, and the register
// transpose used for row-contiguous operands is a true transpose.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../transformer_gemm_epilogue_gemm1_amd/csrc/tile_map.hpp"

using namespace coda;

static int failures = 0;
#define CHECK(cond, ...)                   \
  do {                                     \
    if (!(cond)) {                         \
      if (failures < 20) {                 \
        fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
        fprintf(stderr, __VA_ARGS__);      \
        fprintf(stderr, "\n");             \
      }                                    \
      ++failures;                          \
    }                                      \
  } while (0)

static void check_map_tile() {
  const int shapes[][2] = {{1, 1}, {1, 2}, {2, 1}, {3, 5}, {64, 16}, {64, 112}, {32, 224}, {33, 17},
                           {7, 9}, {8, 8}, {9, 1}, {1, 9}, {64, 64}, {65, 113}};
  const int groups[] = {1, 2, 4, 8, 16};
  for (auto& sh : shapes)
    for (int gm : groups) {
      const int tm_n = sh[0], tn_n = sh[1], nb = tm_n * tn_n;
      std::vector<int> seen(nb, 0);
      for (int b = 0; b < nb; ++b) {
        int tm = -1, tn = -1;
        map_tile(b, tm_n, tn_n, gm, &tm, &tn);
        CHECK(tm >= 0 && tm < tm_n && tn >= 0 && tn < tn_n, "map_tile(%d,%d,%d,%d) -> (%d,%d) out of range", b, tm_n,
              tn_n, gm, tm, tn);
        if (tm >= 0 && tm < tm_n && tn >= 0 && tn < tn_n) seen[tm * tn_n + tn]++;
      }
      for (int i = 0; i < nb; ++i) CHECK(seen[i] == 1, "tile %d of %dx%d (group %d) hit %d times", i, tm_n, tn_n, gm, seen[i]);
    }
}

static void check_lds_layout() {
  std::vector<int> seen(kStageBytes / 16, 0);
  for (int row = 0; row < kTileM; ++row)
    for (int c = 0; c < kChunks; ++c) {
      const int off = lds_offset(row, c);
      CHECK(off >= 0 && off + 16 <= kStageBytes && off % 16 == 0, "lds_offset(%d,%d)=%d", row, c, off);
      seen[off / 16]++;
    }
  for (size_t i = 0; i < seen.size(); ++i) CHECK(seen[i] == 1, "LDS slot %zu used %d times", i, seen[i]);
  // fragment reads: 16 consecutive rows (one per lane) at one logical chunk;
  // 16-byte reads use 4 consecutive 4-byte banks.
  for (int r0 = 0; r0 < kTileM; r0 += 16)
    for (int c = 0; c < kChunks; ++c) {
      int used64[64] = {0};
      for (int i = 0; i < 16; ++i) {
        const int bank = (lds_offset(r0 + i, c) / 4) % 64;
        for (int w = 0; w < 4; ++w) used64[(bank + w) % 64]++;
      }
      for (int b = 0; b < 64; ++b) CHECK(used64[b] == 1, "64-bank conflict rows %d.. chunk %d bank %d", r0, c, b);
      for (int h = 0; h < 16; h += 8) {
        int used32[32] = {0};
        for (int i = h; i < h + 8; ++i) {
          const int bank = (lds_offset(r0 + i, c) / 4) % 32;
          for (int w = 0; w < 4; ++w) used32[(bank + w) % 32]++;
        }
        for (int b = 0; b < 32; ++b) CHECK(used32[b] == 1, "32-bank conflict rows %d.. chunk %d bank %d", r0 + h, c, b);
      }
    }
}

static void check_staging() {
  // contraction-contiguous operand: 256 threads x 8 slots cover 256 rows x 8 chunks once
  std::vector<int> seen(kTileM * kChunks, 0);
  for (int t = 0; t < kThreads; ++t)
    for (int i = 0; i < 8; ++i) {
      int row, c;
      kc_slot(t, i, &row, &c);
      CHECK(row >= 0 && row < kTileM && c >= 0 && c < kChunks, "kc_slot(%d,%d)", t, i);
      seen[row * kChunks + c]++;
    }
  for (size_t i = 0; i < seen.size(); ++i) CHECK(seen[i] == 1, "kc chunk %zu hit %d", i, seen[i]);
  // row-contiguous operand: E x E blocks
  for (int E : {8, 4}) {
    std::fill(seen.begin(), seen.end(), 0);
    const int nb = 8 / E;
    for (int t = 0; t < kThreads; ++t)
      for (int i = 0; i < nb; ++i) {
        int rb, kb;
        rc_block(t, i, E, &rb, &kb);
        CHECK(rb >= 0 && rb < kTileM / E && kb >= 0 && kb < kChunks, "rc_block(%d,%d,E=%d)", t, i, E);
        for (int c = 0; c < E; ++c) seen[(rb * E + c) * kChunks + kb]++;
      }
    for (size_t i = 0; i < seen.size(); ++i) CHECK(seen[i] == 1, "rc E=%d chunk %zu hit %d", E, i, seen[i]);
  }
}

static void check_transpose() {
  uint32_t in[8][4], out[8][4];
  uint16_t val[8][8];
  srand(1);
  for (int trial = 0; trial < 100; ++trial) {
    for (int r = 0; r < 8; ++r)
      for (int c = 0; c < 8; ++c) val[r][c] = (uint16_t)(rand() & 0xffff);
    for (int r = 0; r < 8; ++r)
      for (int p = 0; p < 4; ++p) in[r][p] = (uint32_t)val[r][2 * p] | ((uint32_t)val[r][2 * p + 1] << 16);
    transpose8x8_b16(in, out);
    for (int c = 0; c < 8; ++c)
      for (int k = 0; k < 8; ++k) {
        const uint16_t got = (uint16_t)(out[c][k / 2] >> (16 * (k & 1)));
        CHECK(got == val[k][c], "transpose: out[%d] elem %d = %04x, want %04x", c, k, got, val[k][c]);
      }
  }
}

static void check_epilogue_slab() {
  // each wavefront's 16 x kEpiPitch float slab stays inside its own region
  // and inside the first LDS stage; lane writes and reads stay in the slab
  const int slab_floats = 16 * kEpiPitch;
  CHECK(4 * slab_floats * 4 <= 2 * kStageBytes * 2, "slabs exceed LDS");
  for (int lane = 0; lane < 64; ++lane) {
    for (int nt = 0; nt < 8; ++nt)
      for (int e = 0; e < 4; ++e) {
        const int idx = (4 * (lane >> 4) + e) * kEpiPitch + nt * 16 + (lane & 15);
        CHECK(idx >= 0 && idx < slab_floats, "slab write lane %d", lane);
      }
    for (int q = 0; q < 4; ++q) {
      const int idx = ((lane >> 4) + 4 * q) * kEpiPitch + (lane & 15) * 8;
      CHECK(idx >= 0 && idx + 8 <= slab_floats && idx % 4 == 0, "slab read lane %d", lane);
    }
  }
}

int main() {
  check_map_tile();
  check_lds_layout();
  check_staging();
  check_transpose();
  check_epilogue_slab();
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("tile_map checks passed\n");
  return 0;
}
