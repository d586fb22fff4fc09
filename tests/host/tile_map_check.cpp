// Host-side checks of the GEMM kernels' index maps (built with g++, no GPU):
//  - the workgroup -> tile map is a bijection,
//  - every direct HBM->LDS load lands where the fragment reads expect the
//    logical element (KC and RC layouts, bf16 and fp32), covering each LDS
//    slot of a stage exactly once,
//  - fragment reads stay inside their operand tile, return the right logical
//    elements (the transposing read is emulated with the lane mapping the GPU
//    probe established: within each 16-lane group, lane i receives the i-th
//    16-bit value of every 16-lane stripe of the group's concatenated reads),
//  - the address shortcuts the kernel uses hold (fragment t at +1 KiB for KC,
//    at ^ 32 t for RC bf16, h = 1 at +2 KiB),
//  - fragment reads are LDS-bank-conflict free (KC) or at most 2-way (RC),
//  - the epilogue slabs stay inside their LDS region.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../transformer_gemm_epilogue_gemm1_amd/csrc/tile_map.hpp"

using namespace coda;

static int failures = 0;
#define CHECK(cond, ...)                                     \
  do {                                                       \
    if (!(cond)) {                                           \
      if (failures < 20) {                                   \
        fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
        fprintf(stderr, __VA_ARGS__);                        \
        fprintf(stderr, "\n");                               \
      }                                                      \
      ++failures;                                            \
    }                                                        \
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
        CHECK(tm >= 0 && tm < tm_n && tn >= 0 && tn < tn_n, "map_tile(%d,%d,%d,%d) -> (%d,%d)", b, tm_n, tn_n, gm, tm,
              tn);
        if (tm >= 0 && tm < tm_n && tn >= 0 && tn < tn_n) seen[tm * tn_n + tn]++;
      }
      for (int i = 0; i < nb; ++i) CHECK(seen[i] == 1, "tile %d of %dx%d (group %d) hit %d times", i, tm_n, tn_n, gm, seen[i]);
    }
}

// ---- contraction-contiguous layout --------------------------------------
static void check_kc() {
  // DMA placement == fragment-read placement, full coverage
  std::vector<int> pos_of(kTileM * 4, -1), hits(kOperandBytes / 16, 0);
  for (int s = 0; s < kDmaSlots; ++s)
    for (int w = 0; w < kWaves; ++w)
      for (int L = 0; L < 64; ++L) {
        int r, c;
        dma_kc(s, w, L, &r, &c);
        CHECK(r >= 0 && r < kTileM && c >= 0 && c < 4, "dma_kc(%d,%d,%d) -> (%d,%d)", s, w, L, r, c);
        const int pos = (s * kWaves + w) * 1024 + 16 * L;
        CHECK(pos + 16 <= kOperandBytes, "KC DMA block out of tile");
        CHECK(kc_offset(r, c) == pos, "KC: DMA writes (%d,%d) at %d, reads expect %d", r, c, pos, kc_offset(r, c));
        hits[pos / 16]++;
        pos_of[r * 4 + c] = pos;
        // a lane's chunk is the same in every slot (the kernel keeps one index)
        int r0, c0;
        dma_kc(0, w, L, &r0, &c0);
        CHECK(c0 == c, "KC chunk differs between slots");
      }
  for (size_t i = 0; i < hits.size(); ++i) CHECK(hits[i] == 1, "KC LDS slot %zu written %d times", i, hits[i]);
  for (size_t i = 0; i < pos_of.size(); ++i) CHECK(pos_of[i] >= 0, "KC element chunk %zu never loaded", i);
  // fragment reads: the lane reads logical (base + 16 t + i, chunk g); +1 KiB per t; banks
  for (int base = 0; base < kTileM; base += 64)
    for (int t = 0; t < 8 && base + 16 * t < kTileM; ++t) {
      for (int lane = 0; lane < 64; ++lane) {
        const int off = kc_offset(base + 16 * t + (lane & 15), lane >> 4);
        CHECK(off == kc_offset(base + (lane & 15), lane >> 4) + 1024 * t, "KC fragment stride");
        CHECK(off >= 0 && off + 16 <= kOperandBytes, "KC fragment read out of tile");
      }
      for (int g = 0; g < 4; ++g) {  // one 16-lane group = one pass of a 16-byte read
        int used[64] = {0};
        for (int i = 0; i < 16; ++i) {
          const int bank = (kc_offset(base + 16 * t + i, g) / 4) % 64;
          for (int q = 0; q < 4; ++q) used[(bank + q) % 64]++;
        }
        for (int b = 0; b < 64; ++b) CHECK(used[b] == 1, "KC fragment bank conflict base %d t %d g %d", base, t, g);
        // also conflict-free when the LDS serves 8 or 4 lanes (128 or 64 bytes) at a time
        for (int w : {4, 8})
          for (int i0 = 0; i0 < 16; i0 += w) {
            std::vector<int> slot(w, 0);
            for (int i = i0; i < i0 + w; ++i) slot[(kc_offset(base + 16 * t + i, g) % (16 * w)) / 16]++;
            for (int q = 0; q < w; ++q) CHECK(slot[q] == 1, "KC fragment: %d-lane window conflict at base %d t %d g %d", w, base, t, g);
          }
      }
    }
}

// ---- tile-packed contraction-contiguous layout --------------------------
// The DMA of a k-tile fills the same LDS positions kp_offset reads back; a
// lane's 16 bytes come from consecutive global units (each 1 KiB block is
// one contiguous 1 KiB of the packed matrix); fragment reads are 256
// contiguous bytes per 16 lanes (every bank once); kp_unit is a bijection
// from (row, chunk) onto the packed units.
static void check_kp() {
  std::vector<int> hits(kOperandBytes / 16, 0), pos_of(kTileM * 4, -1);
  const int nck = 40;  // chunks per row of a packed matrix (D = 320)
  for (int s = 0; s < kDmaSlots; ++s)
    for (int w = 0; w < kWaves; ++w) {
      int64_t unit0[3] = {-1, -1, -1};
      for (int L = 0; L < 64; ++L) {
        int r, c;
        dma_kp(s, w, L, &r, &c);
        CHECK(r >= 0 && r < kTileM && c >= 0 && c < 4, "dma_kp(%d,%d,%d) -> (%d,%d)", s, w, L, r, c);
        const int pos = (s * kWaves + w) * 1024 + 16 * L;
        CHECK(kp_offset(r, c) == pos, "KP: DMA writes (%d,%d) at %d, reads expect %d", r, c, pos, kp_offset(r, c));
        hits[pos / 16]++;
        pos_of[r * 4 + c] = pos;
        int r0, c0;
        dma_kp(0, w, L, &r0, &c0);
        CHECK(c0 == c, "KP chunk differs between slots");
        // k-tile kt of tile row m0 = 256: chunk 4 kt + c; consecutive lanes read consecutive units
        for (int kt = 0; kt < 3; ++kt) {
          const int64_t u = kp_unit(256 + r, 4 * kt + c, nck);
          if (L == 0) unit0[kt] = u;
          CHECK(u == unit0[kt] + L, "KP DMA block not contiguous (s %d w %d L %d kt %d)", s, w, L, kt);
          // the kernel adds 1 KiB per k-tile to the k-tile-0 offset
          CHECK(u * 16 == kp_unit(256 + r, c, nck) * 16 + 1024 * kt, "KP k-tile stride");
        }
      }
    }
  for (size_t i = 0; i < hits.size(); ++i) CHECK(hits[i] == 1, "KP LDS slot %zu written %d times", i, hits[i]);
  for (size_t i = 0; i < pos_of.size(); ++i) CHECK(pos_of[i] >= 0, "KP element chunk %zu never loaded", i);
  for (int base = 0; base < kTileM; base += 128)
    for (int t = 0; t < kFragM; ++t)
      for (int g = 0; g < 4; ++g) {
        int used[64] = {0};
        for (int i = 0; i < 16; ++i) {
          const int off = kp_offset(base + 16 * t + i, g);
          CHECK(off == kp_offset(base + i, g) + 1024 * t, "KP fragment stride");
          CHECK(off == kp_offset(base + 16 * t, g) + 16 * i, "KP fragment not contiguous");
          const int bank = (off / 4) % 64;
          for (int q = 0; q < 4; ++q) used[(bank + q) % 64]++;
        }
        for (int b = 0; b < 64; ++b) CHECK(used[b] == 1, "KP fragment bank conflict base %d t %d g %d", base, t, g);
      }
  // kp_unit: a bijection from 37 rows x nck chunks onto 48 x nck units (rows padded to 16)
  std::vector<int> seen(48 * nck, 0);
  for (int r = 0; r < 37; ++r)
    for (int c = 0; c < nck; ++c) {
      const int64_t u = kp_unit(r, c, nck);
      CHECK(u >= 0 && u < 48 * nck, "kp_unit out of range");
      seen[u]++;
    }
  int total = 0;
  for (int v : seen) {
    CHECK(v <= 1, "kp_unit not injective");
    total += v;
  }
  CHECK(total == 37 * nck, "kp_unit count");
}

// ---- row-contiguous layout ----------------------------------------------
static void check_rc(int E) {
  const int KTE = kKTBytes / (16 / E);  // contraction rows per k-tile (32 bf16, 16 fp32)
  const int cpr = rc_row_bytes(E) / 16;
  std::vector<int> hits(kOperandBytes / 16, 0), loaded(KTE * cpr, 0);
  // element id at each 2-byte (bf16) / 4-byte (fp32) LDS position: k * 256 + col
  std::vector<int> lds(kOperandBytes / (16 / E) * 0 + kOperandBytes, -1);
  const int es = 16 / E;
  for (int s = 0; s < kDmaSlots; ++s)
    for (int w = 0; w < kWaves; ++w)
      for (int L = 0; L < 64; ++L) {
        int k, c;
        dma_rc(s, w, L, E, &k, &c);
        CHECK(k >= 0 && k < KTE && c >= 0 && c < cpr, "dma_rc E=%d (%d,%d,%d) -> (%d,%d)", E, s, w, L, k, c);
        const int pos = (s * kWaves + w) * 1024 + 16 * L;
        CHECK(rc_offset(k, c, E) == pos, "RC E=%d: DMA writes (%d,%d) at %d, layout says %d", E, k, c, pos,
              rc_offset(k, c, E));
        hits[pos / 16]++;
        loaded[k * cpr + c]++;
        // the kernel derives slot s's contraction row as row(slot 0) + s * kslot
        int k0, c0;
        dma_rc(0, w, L, E, &k0, &c0);
        CHECK(k == k0 + s * ((kWaves * 1024) / rc_row_bytes(E)), "RC E=%d slot row stride", E);
        for (int e = 0; e < E; ++e) lds[pos + e * es] = k * kTileM + c * E + e;
      }
  for (size_t i = 0; i < hits.size(); ++i) CHECK(hits[i] == 1, "RC E=%d LDS slot %zu written %d times", E, i, hits[i]);
  for (size_t i = 0; i < loaded.size(); ++i) CHECK(loaded[i] == 1, "RC E=%d element chunk %zu loaded %d times", E, i,
                                                   loaded[i]);
  const int nfrag[2] = {kFragM, kFragN};
  const int bases_step[2] = {kWaveM, kWaveN};
  for (int which = 0; which < 2; ++which)
    for (int base = 0; base < kTileM; base += bases_step[which])
      for (int t = 0; t < nfrag[which]; ++t) {
        if (E == 8) {
          for (int h = 0; h < 2; ++h) {
            int bank_hits[64] = {0};
            int got[64][4];
            for (int lane = 0; lane < 64; ++lane) {
              const int off = rc_tr_offset(base, t, h, lane);
              CHECK(off == (rc_tr_lane_base(base, 0, lane) ^ (32 * t)) + 2048 * h, "RC tr address shortcut base %d t %d h %d lane %d",
                    base, t, h, lane);
              CHECK(off >= 0 && off + 8 <= kOperandBytes && off % 8 == 0, "RC tr read out of tile");
              for (int e = 0; e < 4; ++e) got[lane][e] = lds[off + 2 * e];
              for (int q = 0; q < 2; ++q) bank_hits[(off / 4 + q) % 64]++;
            }
            for (int b = 0; b < 64; ++b) CHECK(bank_hits[b] <= 2, "RC tr read bank %d hit %d times", b, bank_hits[b]);
            // emulate the transposing read and check the MFMA operand layout
            for (int lane = 0; lane < 64; ++lane) {
              const int g = lane >> 4, i = lane & 15;
              for (int u = 0; u < 4; ++u) {
                const int src = 16 * u + i;  // stripe index within the group's 64 values
                const int v = got[16 * g + src / 4][src % 4];
                const int want = (8 * g + 4 * h + u) * kTileM + base + 16 * t + i;
                CHECK(v == want, "RC tr lane %d u %d: got %d want %d (base %d t %d h %d)", lane, u, v, want, base, t, h);
              }
            }
          }
        } else {
          for (int u = 0; u < 4; ++u)
            for (int lane = 0; lane < 64; ++lane) {
              const int off = rc_f32_offset(base, t, u, lane);
              CHECK(off >= 0 && off + 4 <= kOperandBytes, "RC f32 read out of tile");
              const int want = (4 * (lane >> 4) + u) * kTileM + base + 16 * t + (lane & 15);
              CHECK(lds[off] == want, "RC f32 lane %d u %d: got %d want %d", lane, u, lds[off], want);
            }
        }
      }
}

// SwiGLU column order: a bijection of [0, 2F) onto itself whose run pair
// (2m, 2m+1) holds gate columns R m.. and up columns F + R m.. (R =
// kSwiGLURun), with every DMA chunk (8 bf16 or 4 fp32 elements) contiguous in
// memory, and output columns / up flags consistent with it.
static void check_swiglu_col() {
  const int R = kSwiGLURun;
  const int Fs[] = {32, 64, 96, 256, 288, 1024, 14336};
  for (int F : Fs) {
    std::vector<int> seen(2 * F, 0);
    for (int n = 0; n < 2 * F; ++n) {
      const int p = swiglu_col(n, F);
      CHECK(p >= 0 && p < 2 * F, "swiglu_col(%d, %d) = %d out of range", n, F, p);
      if (p >= 0 && p < 2 * F) seen[p]++;
      const int c = n / R, m = c / 2, i = n % R;
      CHECK(p == (c % 2 ? F : 0) + R * m + i, "swiglu_col(%d, %d) = %d", n, F, p);
      CHECK(swiglu_is_up(n) == (c % 2 == 1), "swiglu_is_up(%d)", n);
      CHECK(swiglu_out_col(n) == R * m + i && p == (swiglu_is_up(n) ? F : 0) + swiglu_out_col(n), "swiglu_out_col(%d)", n);
      if (n % 4 != 0) CHECK(p == swiglu_col(n - 1, F) + 1, "SwiGLU chunk not contiguous at %d", n);
    }
    for (int p = 0; p < 2 * F; ++p) CHECK(seen[p] == 1, "SwiGLU column %d of F=%d hit %d times", p, F, seen[p]);
  }
  // the epilogue pairs lane l (gate) with lane l ^ kSwiGLUPartner (up): same
  // row group (l / 8) and the same output columns
  for (int n0 = 0; n0 < 1024; n0 += kTileN)
    for (int wn = 0; wn < 4; ++wn)
      for (int lane = 0; lane < 64; ++lane) {
        const int pl = lane ^ kSwiGLUPartner;
        const int col = n0 + wn * kWaveN + (lane & 7) * 8, col_p = n0 + wn * kWaveN + (pl & 7) * 8;
        CHECK((pl >> 3) == (lane >> 3), "SwiGLU partner in another row group");
        CHECK(swiglu_is_up(col) != swiglu_is_up(col_p), "SwiGLU partner of the same kind");
        CHECK(swiglu_out_col(col) == swiglu_out_col(col_p), "SwiGLU partner covers different output columns");
      }
}

// fp8 fragments: 32-row fragments read as two 16-byte chunks per lane; the
// lane gets operand row base + 32 t + l % 32 and chunks l/32 and 2 + l/32
// (each 32-byte scale block of the k-tile spread over both lane halves);
// every 16-lane pass of a read hits each bank once; reads stay in the tile;
// the second chunk is the first XOR 32 bytes, fragment t is 2 KiB further;
// over a fragment every (row, chunk) of the 32 rows is read exactly once.
static void check_kc8() {
  for (int base = 0; base < kTileM; base += kWaveM)
    for (int t = 0; t < kFrag8M && base + 32 * t < kTileM; ++t)
      for (int half = 0; half < 2; ++half) {
        for (int lane = 0; lane < 64; ++lane) {
          const int off = kc8_offset(base, t, half, lane);
          CHECK(off >= 0 && off + 16 <= kOperandBytes, "kc8 read out of tile");
          CHECK(off == (kc8_offset(base, 0, 0, lane) ^ (32 * half)) + 2048 * t, "kc8 address shortcut");
          const int row = base + 32 * t + (lane & 31), chunk = (lane >> 5) + 2 * half;
          CHECK(off == kc_offset(row, chunk), "kc8 element");
        }
        if (half == 1) {
          std::vector<int> seen(32 * 4, 0);
          for (int lane = 0; lane < 64; ++lane)
            for (int h = 0; h < 2; ++h) seen[(lane & 31) * 4 + (lane >> 5) + 2 * h]++;
          for (int v : seen) CHECK(v == 1, "kc8: a (row, chunk) of the fragment read twice or never");
        }
        for (int g = 0; g < 4; ++g) {
          int used[64] = {0};
          for (int i = 0; i < 16; ++i) {
            const int bank = (kc8_offset(base, t, half, 16 * g + i) / 4) % 64;
            for (int q = 0; q < 4; ++q) used[(bank + q) % 64]++;
          }
          for (int b = 0; b < 64; ++b) CHECK(used[b] == 1, "kc8 bank conflict");
          for (int w : {4, 8})
            for (int i0 = 0; i0 < 16; i0 += w) {
              std::vector<int> slot(w, 0);
              for (int i = i0; i < i0 + w; ++i) slot[(kc8_offset(base, t, half, 16 * g + i) % (16 * w)) / 16]++;
              for (int q = 0; q < w; ++q) CHECK(slot[q] == 1, "kc8: %d-lane window conflict", w);
            }
        }
      }
  // 32 x 32 accumulators into 16-row slabs: every slab cell written once
  for (int s = 0; s < 8; ++s) {
    std::vector<int> cell(16 * 64, 0);
    for (int lane = 0; lane < 64; ++lane)
      for (int nt = 0; nt < kFrag8N; ++nt)
        for (int e = 8 * (s & 1); e < 8 * (s & 1) + 8; ++e) {
          const int r = acc32_row(e, lane) - 16 * (s & 1), c = 32 * nt + (lane & 31);
          CHECK(r >= 0 && r < 16 && c >= 0 && c < 64, "acc32 slab cell out of range");
          if (r >= 0 && r < 16) cell[r * 64 + c]++;
        }
    for (int i = 0; i < 16 * 64; ++i) CHECK(cell[i] == 1, "acc32 slab cell %d of slab %d written %d times", i, s, cell[i]);
  }
}

static void check_epilogue_slab() {
  const int slab_floats = 16 * kEpiPitch;
  CHECK((kWaves / 4) * kEpiSlabBytes <= kStageBytes, "slabs exceed their stage");
  for (int lane = 0; lane < 64; ++lane) {
    for (int nt = 0; nt < kFragN; ++nt)
      for (int e = 0; e < 4; ++e) {
        const int idx = (4 * (lane >> 4) + e) * kEpiPitch + nt * 16 + (lane & 15);
        CHECK(idx >= 0 && idx < slab_floats, "slab write lane %d", lane);
      }
    for (int q = 0; q < 2; ++q) {
      const int idx = ((lane >> 3) + 8 * q) * kEpiPitch + (lane & 7) * 8;
      CHECK(idx >= 0 && idx + 8 <= slab_floats && idx % 4 == 0, "slab read lane %d", lane);
    }
  }
}

// MX exponent bytes: every (row, k-tile, half) of an array for M rows and
// G groups lands on its own byte inside 8 M G bytes; a group's dword of one
// (row, half) holds its 4 k-tiles in order; the dwords the 64 lanes of a
// 32-row fragment read for one group are 256 contiguous bytes.
static void check_mx_byte() {
  for (int M : {1, 3, 32, 37, 128, 300})
    for (int G : {1, 2, 5}) {
      const int64_t RB = mx_row_blocks(M), bytes = 1024 * RB * G;
      CHECK(RB == (M + 127) / 128, "mx_row_blocks");
      std::vector<int> hit(bytes, 0);
      // every (row up to M rounded up to 128, k-tile, half) owns one byte
      for (int i = 0; i < 128 * RB; ++i)
        for (int t = 0; t < 4 * G; ++t)
          for (int h = 0; h < 2; ++h) {
            const int64_t o = mx_byte(i, t, h, M);
            CHECK(o >= 0 && o < bytes, "mx_byte outside the array");
            if (o >= 0 && o < bytes) hit[o]++;
          }
      for (int v : hit) CHECK(v == 1, "mx_byte: a byte used twice or never");
      // a wave's read of group g for its 128 rows: lane l takes the 16 bytes
      // at mx_byte(row0 + l % 32, 4g, l / 32); dword f of them holds the 4
      // k-tiles of fragment f's row row0 + 32f + l % 32, and the 64 lanes'
      // reads tile 1 KiB
      for (int row0 = 0; row0 < 128 * RB; row0 += 128)
        for (int g = 0; g < G; ++g) {
          std::vector<int> w(64, 0);
          const int64_t lo = mx_byte(row0, 4 * g, 0, M);
          CHECK(lo % 1024 == 0, "mx_byte: wave read not 1 KiB aligned");
          for (int lane = 0; lane < 64; ++lane) {
            const int64_t off = mx_byte(row0 + (lane & 31), 4 * g, lane >> 5, M);
            CHECK(off % 16 == 0 && off - lo >= 0 && off - lo < 1024, "mx_byte: lane read misplaced");
            if (off - lo >= 0 && off - lo < 1024) w[(off - lo) / 16]++;
            for (int f = 0; f < 4; ++f)
              for (int tt = 0; tt < 4; ++tt)
                CHECK(mx_byte(row0 + 32 * f + (lane & 31), 4 * g + tt, lane >> 5, M) == off + 4 * f + tt,
                      "mx_byte: lane's 16 bytes not its fragments' k-tiles");
          }
          for (int v : w) CHECK(v == 1, "mx_byte: wave read does not cover its 1 KiB");
        }
    }
}

int main() {
  check_map_tile();
  check_kc();
  check_kp();
  check_rc(8);
  check_rc(4);
  check_epilogue_slab();
  check_swiglu_col();
  check_kc8();
  check_mx_byte();
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("tile_map checks passed\n");
  return 0;
}
