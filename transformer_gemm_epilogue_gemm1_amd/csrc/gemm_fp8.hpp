// MFMA GEMM main loop for fp8 (OCP e4m3) operands on gfx950.
//
//   C[m, n] = sum_k A[m, k] B[n, k],  both operands contraction-contiguous
//   (A[M, K] row-major, B stored [N, K]), fp32 accumulation.
//
// The loop is the bf16 one (gemm.hpp) with fp8 fragments: the same 64-byte
// k-tiles (64 elements), direct HBM->LDS loads into the same four stages, the
// same barrier, tile order and epilogue interface.  What differs: a
// wavefront's 128 x 64 sub-tile is 4 x 2 products v_mfma_f32_32x32x64_f8f6f4
// (16 accumulators per lane each, 128 in all), each k-tile is one product per
// fragment pair, and fragments are 32 rows (two 16-byte reads per lane,
// kc8_offset).  Per k-tile a wavefront moves the same bytes as in bf16 for
// twice the flops.
#pragma once

#include "gemm.hpp"

namespace coda {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <>
struct Elem<uint8_t> {  // OCP e4m3, stored as its 8-bit code
  static constexpr int E = 16;
};

// 32-row fragment t of a contraction-contiguous operand tile (chunks g and
// 2 + g of the lane's row, kc8_offset); PK: the tile is in the packed LDS
// order (kp_offset in tile_map.hpp).
template <bool PK = false>
struct FragReader8 {
  int off0;  // lane's byte offset of fragment 0, first chunk
  __device__ __forceinline__ FragReader8(int base, int lane)
      : off0(PK ? kp_offset(base + (lane & 31), lane >> 5) : kc8_offset(base, 0, 0, lane)) {}
  __device__ __forceinline__ void refresh() { opaque(off0); }
  __device__ __forceinline__ i32x8 read(const char* tile, int t) const {
    // KC: the second chunk (chunk index + 2) is the first XOR 32 bytes (the
    // swizzle XORs the chunk index); packed: two chunks of the row block
    // further, 512 bytes on.  Fragment t lies 32 rows (2 KiB) further in
    // both layouts.
    const u32x4 lo = *(const u32x4*)(tile + off0 + 2048 * t);
    const u32x4 hi = *(const u32x4*)(tile + (PK ? off0 + 512 : (off0 ^ 32)) + 2048 * t);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
};

__device__ __forceinline__ void mac8(f32x16& acc, const i32x8& a, const i32x8& b) {
  // formats 0, 0: both operands e4m3; zero scale selectors: unscaled
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
}

// Which operands carry block exponents (MX): a mask of these bits.
constexpr int kMxA = 1, kMxB = 2;

// The same product with block scales: contraction block h of A's row i (the
// k-tile's bytes [32 h, 32 h + 32), the half-h registers of lanes i and
// 32 + i) is multiplied by 2^(a - 127), a the byte SEL of lane 32 h + i's
// sa; block h of B's row j (output column j) likewise by the byte SEL of
// lane 32 h + j's sb.  An unscaled operand passes 0x7F7F7F7F (2^0 in every
// byte).
template <int SEL>
__device__ __forceinline__ void mac8_mx(f32x16& acc, const i32x8& a, const i32x8& b, uint32_t sa, uint32_t sb) {
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, SEL, (int)sa, SEL, (int)sb);
}
constexpr uint32_t kMxUnit = 0x7F7F7F7Fu;

// Block exponents of an operand (E8M0 bytes in the mx_byte layout of
// tile_map.hpp, as the first GEMM's fp8 epilogue and the MX quantiser write
// them).  Lane l supplies, per fragment f of the wavefront's rows, the
// scales of row row0 + 32 f + l % 32 for block l / 32.  The layout puts the
// dwords of the 4 fragments of a 128-row block in a lane's 16 consecutive
// bytes (one byte per k-tile of a group of 4): an A wavefront (128 rows, 4
// fragments) loads all 16, a B wavefront (64 rows, 2 fragments, half of a
// 128-row block) the 8 of its half.  A group costs the lane one load; the
// wavefront reads 1 KiB (A) or 512 bytes (B) of consecutive memory.  (With
// one dword load per fragment the scaled GEMM ran 3.5% slower than with the
// exponents recycled in registers, wherever the dwords lay.)  Wavefronts
// whose rows all lie past the operand's end read 0 through the buffer
// descriptor's range check; their products are never stored.
struct MxArgs {
  const uint8_t* e;  // null: the operand is unscaled
  int64_t M;         // rows of the array (the operand's rows: the GEMM's M for A, N for B)
  uint32_t span;     // bytes of the array
};

template <int NF>
struct MxReader {
  static_assert(NF == 4 || NF == 2, "a wavefront's operand rows are 4 or 2 fragments");
  static constexpr int kLoads = 1;  // vector memory instructions per load() (the barrier counts them)
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off;    // byte offset of the lane's dwords of group 0, or kOutOfRange
  uint32_t gstep;  // bytes between groups
  // row0: the wavefront's first operand row (a multiple of 32 NF)
  __device__ __forceinline__ void init(const MxArgs& mx, int row0, int lane) {
    rsrc = make_rsrc(mx.e, mx.span);
    gstep = (uint32_t)(1024 * mx_row_blocks(mx.M));
    off = row0 < mx.M ? (uint32_t)mx_byte(row0 + (lane & 31), 0, lane >> 5, mx.M) : kOutOfRange;
  }
  // group grp's dwords; a group past the last one reads 0 (past the array)
  __device__ __forceinline__ void load(int grp, uint32_t (&out)[NF]) const {
    const int o = (int)(off + gstep * (uint32_t)grp);
    if constexpr (NF == 4) {
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, o, 0, 0));
#pragma unroll
      for (int f = 0; f < 4; ++f) out[f] = v[f];
    } else {
      const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rsrc, o, 0, 0));
      out[0] = v[0];
      out[1] = v[1];
    }
  }
};

// Block exponents held across a group of 4 k-tiles: cur for the group being
// multiplied, nxt for the next one, loaded during the group's first step.
template <int NF>
struct MxRegs {
  uint32_t cur[NF], nxt[NF];
};

// The exponent readers and registers of both operands (those not scaled stay
// unused).
struct MxState {
  MxReader<kFrag8M> ra;
  MxReader<kFrag8N> rb;
  MxRegs<kFrag8M> a;
  MxRegs<kFrag8N> b;
};

constexpr int kDmaIssueAfter8 = 1;

struct Frags8 {
  i32x8 a[kFrag8M], b[kFrag8N];
};

// One k-step, k-tile kt in stage S (the schedule of kstep in gemm.hpp): B
// fragments of tile kt + 1, then per A fragment its 2 products of tile kt and
// its reload for tile kt + 1; the loads of tile kt + kStages - 1 go out
// after the products of A fragment kDmaIssueAfter8 (4 products, 256
// matrix-core cycles, as in the bf16 step).
//
// MX (a mask of kMxA, kMxB: the operands that are block-scaled): k-tile kt
// uses byte kt % 4 = S of the group's exponent dwords.  The first step of a
// group moves the prefetched dwords into use and, behind the direct loads,
// loads the next group's (NEXT: the steps after the main loop belong to the
// last group and load none); its barrier then allows those loads in flight
// as well (they have a whole group of steps to land).  The barrier's count
// must equal the instructions issued after the direct loads: a larger one
// lets the oldest tile's loads through unlanded.
template <int S, int L = kLayKC, int MX = 0, bool NEXT = true>
__device__ __forceinline__ void kstep8(char* const (&st)[kStages], const Dma<uint8_t, true, L>& da,
                                       const Dma<uint8_t, true, L>& db, FragReader8<lds_packed(L)>& ra,
                                       FragReader8<lds_packed(L)>& rb,
                                       f32x16 (&acc)[kFrag8M][kFrag8N], Frags8& cur, int kt, int K, int wave,
                                       MxState& ms) {
  constexpr bool MA = (MX & kMxA) != 0, MB = (MX & kMxB) != 0;
  constexpr int kMxLoads = (MA ? MxReader<kFrag8M>::kLoads : 0) + (MB ? MxReader<kFrag8N>::kLoads : 0);
  constexpr int SL = (S + kStages - 1) % kStages;
  constexpr int SN = (S + 1) % kStages;
  static_assert(MX == 0 || kStages == 4, "a group of exponent bytes is one pass over the four stages");
  if constexpr (MA && S == 0) {
#pragma unroll
    for (int mt = 0; mt < kFrag8M; ++mt) ms.a.cur[mt] = ms.a.nxt[mt];
  }
  if constexpr (MB && S == 0) {
#pragma unroll
    for (int nt = 0; nt < kFrag8N; ++nt) ms.b.cur[nt] = ms.b.nxt[nt];
  }
  ra.refresh();
  rb.refresh();
  i32x8 nb[kFrag8N];
#pragma unroll
  for (int nt = 0; nt < kFrag8N; ++nt) nb[nt] = rb.read(st[SN] + kOperandBytes, nt);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int mt = 0; mt < kFrag8M; ++mt) {
#pragma unroll
    for (int nt = 0; nt < kFrag8N; ++nt) {
      if constexpr (MX != 0)
        mac8_mx<S>(acc[mt][nt], cur.a[mt], cur.b[nt], MA ? ms.a.cur[mt] : kMxUnit, MB ? ms.b.cur[nt] : kMxUnit);
      else
        mac8(acc[mt][nt], cur.a[mt], cur.b[nt]);
    }
    cur.a[mt] = ra.read(st[SN], mt);
    if (mt == kDmaIssueAfter8) {
      da.issue(st[SL], kt + kStages - 1, K, wave);
      db.issue(st[SL] + kOperandBytes, kt + kStages - 1, K, wave);
      if constexpr (MA && S == 0 && NEXT) ms.ra.load(kt / 4 + 1, ms.a.nxt);
      if constexpr (MB && S == 0 && NEXT) ms.rb.load(kt / 4 + 1, ms.b.nxt);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int nt = 0; nt < kFrag8N; ++nt) cur.b[nt] = nb[nt];
  if constexpr (MX != 0 && S == 0 && NEXT)
    stage_barrier_n<kLoadsPerTile + kMxLoads>();
  else
    stage_barrier();
}

// C = A B^T for fp8 A[M, K] (g.a, g.lda) and B[N, K] (g.b, g.ldb); the
// epilogue interface is the bf16 kernel's (16-row slabs, apply / end_slab /
// finish), and an epilogue that declares kLdsBytes gets that much LDS per
// wavefront through set_lds, in the stage that holds its slab.
// L: OpLayout of both operands (kLayPacked: tile-packed, kp_unit, with g.lda /
// g.ldb counting 16-byte chunks per row).
// MX: a mask of kMxA, kMxB, the operands that carry block exponents (mxa,
// mxb, MxReader's layout) that the products apply; the others' MxArgs are
// unused.
template <class Epi, int L = kLayKC, int MX = 0>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_fp8_kernel(
    GemmArgs g, typename Epi::Params ep, MxArgs mxa, MxArgs mxb) {
  static_assert(kStages == 4, "the stage arrays and the unrolled steps below assume four stages");
  __shared__ __attribute__((aligned(1024))) char st0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char st1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char st2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char st3[kStageBytes];
  char* const st[kStages] = {st0, st1, st2, st3};
  constexpr int KTE = kKTBytes;  // fp8 elements per k-tile
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  int tm, tn;
  map_tile(blockIdx.x, g.tiles_m, g.tiles_n, g.group_m, &tm, &tn);
  const int m0 = tm * kTileM, n0 = tn * kTileN;

  Dma<uint8_t, true, L> da, db;
  da.init(g.a, g.a_span, g.lda, m0, g.M, wave, lane);
  db.init(g.b, g.b_span, g.ldb, n0, g.N, wave, lane);
  FragReader8<lds_packed(L)> ra(wm * kWaveM, lane), rb(wn * kWaveN, lane);
  f32x16 acc[kFrag8M][kFrag8N];
#pragma unroll
  for (int i = 0; i < kFrag8M; ++i)
#pragma unroll
    for (int j = 0; j < kFrag8N; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = (g.K + KTE - 1) / KTE;
  MxState ms;
  if constexpr ((MX & kMxA) != 0) {
    ms.ra.init(mxa, m0 + wm * kWaveM, lane);
    ms.ra.load(0, ms.a.nxt);  // landed by the prologue's wait below
  }
  if constexpr ((MX & kMxB) != 0) {
    ms.rb.init(mxb, n0 + wn * kWaveN, lane);
    ms.rb.load(0, ms.b.nxt);
  }
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t) {
    da.issue(st[t], t, g.K, wave);
    db.issue(st[t] + kOperandBytes, t, g.K, wave);
  }
  static_assert((kStages - 3) * kLoadsPerTile == 4, "the prologue vmcnt literal assumes kStages - 3 tiles in flight");
  asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
  Frags8 cur;
#pragma unroll
  for (int mt = 0; mt < kFrag8M; ++mt) cur.a[mt] = ra.read(st[0], mt);
#pragma unroll
  for (int nt = 0; nt < kFrag8N; ++nt) cur.b[nt] = rb.read(st[0] + kOperandBytes, nt);
  int kt = 0;
  for (; kt + kStages <= nk; kt += kStages) {
    kstep8<0, L, MX>(st, da, db, ra, rb, acc, cur, kt, g.K, wave, ms);
    kstep8<1, L, MX>(st, da, db, ra, rb, acc, cur, kt + 1, g.K, wave, ms);
    kstep8<2, L, MX>(st, da, db, ra, rb, acc, cur, kt + 2, g.K, wave, ms);
    kstep8<3, L, MX>(st, da, db, ra, rb, acc, cur, kt + 3, g.K, wave, ms);
  }
  const int rem = nk - kt;
  if (rem > 0) kstep8<0, L, MX, false>(st, da, db, ra, rb, acc, cur, kt, g.K, wave, ms);
  if (rem > 1) kstep8<1, L, MX, false>(st, da, db, ra, rb, acc, cur, kt + 1, g.K, wave, ms);
  if (rem > 2) kstep8<2, L, MX, false>(st, da, db, ra, rb, acc, cur, kt + 2, g.K, wave, ms);
  drain_barrier();  // no direct load may land in the LDS the epilogue reuses

  // ---- epilogue: slab s = rows 16 s .. 16 s + 15 of the wavefront's 128 =
  // half s % 2 of row fragment s / 2 (acc32_row) ----
  Epi epi(ep, lane, wm, wn, m0, n0, tn, g.M, g.N);
  char* const stw = (wave & 3) == 0 ? st0 : (wave & 3) == 1 ? st1 : (wave & 3) == 2 ? st2 : st3;
  float* slab = (float*)(stw + (wave >> 2) * kEpiSlabBytes);
  if constexpr (epi_lds_bytes<Epi>::value > 0) {
    // the two wavefronts of a stage: their slabs, then the epilogue's own room
    static_assert(2 * kEpiSlabBytes + 2 * epi_lds_bytes<Epi>::value <= kStageBytes, "epilogue LDS exceeds a stage");
    static_assert(kEpiSlabBytes % 16 == 0 && epi_lds_bytes<Epi>::value % 16 == 0, "16-byte LDS alignment");
    epi.set_lds(stw + 2 * kEpiSlabBytes + (wave >> 2) * epi_lds_bytes<Epi>::value);
  }
  const int row_base = m0 + wm * kWaveM;
  const int col = n0 + wn * kWaveN + (lane & 7) * 8;
#pragma unroll
  for (int s = 0; s < 2 * kFrag8M; ++s) {
#pragma unroll
    for (int nt = 0; nt < kFrag8N; ++nt)
#pragma unroll
      for (int e = 8 * (s & 1); e < 8 * (s & 1) + 8; ++e)
        slab[(acc32_row(e, lane) - 16 * (s & 1)) * kEpiPitch + 32 * nt + (lane & 31)] = acc[s >> 1][nt][e];
    wave_lds_fence();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int rl = (lane >> 3) + 8 * q;
      const float* src = slab + rl * kEpiPitch + (lane & 7) * 8;
      const f32x4 lo = *(const f32x4*)src, hi = *(const f32x4*)(src + 4);
      float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const int row = row_base + s * 16 + rl;
      if (row < g.M && col < g.N) epi.apply(s, q, row, col, v);
    }
    epi.end_slab(s, row_base + s * 16);
    wave_lds_fence();
  }
  epi.finish();
}

}  // namespace coda
