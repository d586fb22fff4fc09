// MFMA GEMM main loop for gfx950 with pluggable epilogues.
//
// A GEMM kernel splits into a main loop (tiled multiply-accumulate) and an
// epilogue that post-processes the accumulators while they are still in
// registers, before anything is written to HBM (CODA news article by Synced,
// section "CODA：「尾声」里藏着宝藏").  Here the main loop is fixed and the
// epilogue is a template parameter.
//
//   C[m, n] = sum_k A(m, k) B(k, n),  fp32 accumulation.
//
// Operand storage (row-major with leading dimension ld, in elements):
//   A_KC = true : A(m, k) at a[m * lda + k]   (contraction contiguous)
//   A_KC = false: A(m, k) at a[k * lda + m]   (M contiguous, i.e. A^T stored)
//   B_KC = true : B(k, n) at b[n * ldb + k]   (contraction contiguous)
//   B_KC = false: B(k, n) at b[k * ldb + n]   (N contiguous: a [K, N] matrix)
//
// Workgroup: 512 threads = 8 wavefronts (2 x 4, two per SIMD), a 256 x 256
// output tile, each wavefront a 128 x 64 sub-tile held as 8 x 4 MFMA 16x16
// accumulators (128 fp32 per lane).  Two wavefronts per SIMD let one issue
// MFMAs while the other waits on LDS or the barrier.  The contraction is cut
// into k-tiles of 64 bytes per operand row (32 bf16 / 16 fp32).  Each k-tile
// of both operands goes from HBM straight into one of four LDS stages
// (buffer loads with an LDS destination; no registers, no LDS write
// instructions), contraction-contiguous operands as [row][k] and
// row-contiguous operands as they lie in memory ([k][row]), both XOR
// swizzled.  Fragments are read back with 16-byte reads ([row][k]) or 8-byte
// transposing reads ([k][row], bf16) and feed
//   bf16: v_mfma_f32_16x16x32_bf16
//   fp32: v_mfma_f32_16x16x4_f32, the 4 floats of a fragment feed 4 MFMAs
// Lane l of a 16x16 fragment holds operand row (l % 16) and contraction
// elements of group (l / 16); accumulator element e of lane l is output
// (4*(l/16)+e, l%16).  The contraction order inside one MFMA is the same for
// A and B, so the product does not depend on how the hardware orders k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tile_map.hpp"

namespace coda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {  // bfloat16, stored as its 16-bit pattern
  static constexpr int E = 8;
};
template <>
struct Elem<float> {
  static constexpr int E = 4;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {  // round to nearest even
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ---- element-chunk helpers: 8 values <-> storage -------------------------
// A "chunk" of the epilogue is 8 consecutive columns of one row.
template <typename T>
struct Chunk8;
template <>
struct Chunk8<uint16_t> {
  __device__ static void load(const uint16_t* p, float v[8]) {
    const u32x4 u = *(const u32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
  __device__ static void store(uint16_t* p, const float v[8]) {
    u32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *(u32x4*)p = u;
  }
  // value after a round trip through storage (rounding to the stored dtype)
  __device__ static float round(float x) { return bf16_to_f32(f32_to_bf16(x)); }
  // the 8 values as stored (16 bytes), and their expansion
  __device__ static u32x4 load_raw(const uint16_t* p) { return *(const u32x4*)p; }
  __device__ static void unpack(const u32x4& u, float v[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
};
template <>
struct Chunk8<float> {
  __device__ static void load(const float* p, float v[8]) {
    const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
  __device__ static void store(float* p, const float v[8]) {
    *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
  __device__ static float round(float x) { return x; }
};

// ---- operand staging: HBM -> LDS directly --------------------------------
// Global reads go through a raw buffer descriptor spanning exactly the
// operand's bytes.  A slot that falls outside the matrix (row >= rows,
// contraction index >= K) gets an offset past the descriptor's extent, for
// which the hardware returns zeros: no load ever leaves the operand.
constexpr uint32_t kOutOfRange = 0x80000000u;  // every operand spans < 2 GiB

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t span_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)span_bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;

// How a contraction-contiguous operand lies in memory and in the LDS stages.
//   kLayKC:     row-major in memory; LDS [row][k], XOR swizzled (kc_offset).
//               A direct load covers 16 rows x 64 bytes.
//   kLayPacked: tile-packed in memory (kp_unit, ld = 16-byte chunks per
//               row); LDS in the packed order (kp_offset).  Every direct load
//               copies 1 KiB of consecutive memory.
// (Loading a row-major operand into the packed LDS order, each lane fetching
// its own row's 16-byte chunk, made the second GEMM 7% and the backward 13%
// slower at 7B: the memory side wants 4 consecutive lanes on one row.)
enum OpLayout : int { kLayKC = 0, kLayPacked = 1 };
__host__ __device__ constexpr bool lds_packed(int layout) { return layout != kLayKC; }

// L (contraction-contiguous operands only): one of OpLayout.
template <typename T, bool KC, int L = kLayKC>
struct Dma {
  static constexpr int E = Elem<T>::E;
  static constexpr int KTE = kKTBytes / (int)sizeof(T);  // contraction elements per k-tile
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff[kDmaSlots];  // byte offset of each slot at k-tile 0, or kOutOfRange (row outside)
  int kidx0;                 // contraction index of slot 0 at k-tile 0
  int kslot;                 // contraction index step between slots (KC: 0, RC: rows per slot)
  uint32_t kstep;            // bytes between consecutive k-tiles

  // split > 0 (row-contiguous operands only): operand rows are read in the
  // SwiGLU order of swiglu_col(row, split) (nrows counts logical rows).
  __device__ __forceinline__ void init(const void* p, uint32_t span_bytes, int64_t ld, int row0, int nrows,
                                       int wave, int lane, int split = 0) {
    rsrc = make_rsrc(p, span_bytes);
#pragma unroll
    for (int s = 0; s < kDmaSlots; ++s) {
      if constexpr (KC && lds_packed(L)) {
        int r, c;
        dma_kp(s, wave, lane, &r, &c);
        const int gr = row0 + r;
        if (s == 0) kidx0 = c * E;  // the chunk of a lane is the same in every slot
        voff[s] = gr < nrows ? (uint32_t)(kp_unit(gr, c, ld) * 16) : kOutOfRange;
      } else if constexpr (KC) {
        int r, c;
        dma_kc(s, wave, lane, &r, &c);
        const int gr = row0 + r;
        if (s == 0) kidx0 = c * E;  // the chunk of a lane is the same in every slot
        voff[s] = gr < nrows ? (uint32_t)(((int64_t)gr * ld + c * E) * (int64_t)sizeof(T)) : kOutOfRange;
      } else {
        int k, c;
        dma_rc(s, wave, lane, E, &k, &c);
        const int gr = row0 + c * E;
        const int pr = split > 0 ? swiglu_col(gr, split) : gr;  // E elements stay contiguous
        if (s == 0) kidx0 = k;  // slot s: contraction row k + s * kslot
        voff[s] = gr < nrows ? (uint32_t)(((int64_t)k * ld + pr) * (int64_t)sizeof(T)) : kOutOfRange;
      }
    }
    kslot = KC ? 0 : (kWaves * 1024) / rc_row_bytes(E);
    // tile-packed: a k-tile is 4 chunks of 16 rows further
    kstep = KC ? (uint32_t)(L == kLayPacked ? 4 * 256 : kKTBytes) : (uint32_t)(KTE * ld * (int64_t)sizeof(T));
  }

  // Loads k-tile kt into the operand tile at `dst`.  `wave` is wave-uniform;
  // each slot fills the 1 KiB block (4 s + wave) of the tile.
  __device__ __forceinline__ void issue(char* dst, int kt, int K, int wave) const {
    const uint32_t kb = (uint32_t)kt * kstep;
    const int k0 = kt * KTE + kidx0;
#pragma unroll
    for (int s = 0; s < kDmaSlots; ++s) {
      const bool ok = (voff[s] != kOutOfRange) & (k0 + s * kslot < K);
      const uint32_t o = ok ? voff[s] + kb : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + (s * kWaves + wave) * 1024), 16, o, 0, 0,
                                               0);
    }
  }
};

// ---- MFMA fragments ----------------------------------------------------
// Eight fragments (t = 0..7) of the wavefront's 128 operand rows for one
// k-tile, 16 bytes per lane each (fragment maps in tile_map.hpp).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Keeps the compiler from treating v as loop-invariant, so addresses derived
// from it are recomputed where used instead of all being hoisted into
// registers (four stages x eight fragments would not fit).
__device__ __forceinline__ void opaque(int& v) { asm volatile("" : "+v"(v)); }

// PK: the tile is in the packed LDS order (lds_packed of its layout).
template <typename T, bool KC, bool PK = false>
struct FragReader {
  int off0;  // lane's byte offset of fragment 0 in the operand tile (RC bf16: h = 0 base)
  int base, lane;
  __device__ __forceinline__ FragReader(int base_, int lane_) : base(base_), lane(lane_) {
    off0 = KC ? (PK ? kp_offset(base_ + (lane_ & 15), lane_ >> 4) : kc_offset(base_ + (lane_ & 15), lane_ >> 4))
              : (sizeof(T) == 2 ? rc_tr_lane_base(base_, 0, lane_) : 0);
  }
  __device__ __forceinline__ void refresh() { opaque(off0); }
  // fragment t (compile-time after unrolling) of the operand tile at `tile`
  __device__ __forceinline__ u32x4 read(const char* tile, int t) const {
    if constexpr (KC) {
      // the swizzle depends on row % 16 only: fragment t lies 16 rows (1 KiB) further
      return *(const u32x4*)(tile + off0 + t * 1024);
    } else if constexpr (sizeof(T) == 2) {
      // fragment t at lane base ^ 32 t; h = 1 is 4 contraction rows (2 KiB)
      // further.  The address stays a pointer into the stage array: with an
      // integer-made address the compiler cannot tell which direct loads the
      // read depends on and waits for all of them.
      const lds_char* q = (const lds_char*)tile + (off0 ^ (32 * t));
      const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)q));
      const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(q + 2048)));
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    } else {
      u32x4 f;
#pragma unroll
      for (int u = 0; u < 4; ++u) f[u] = *(const uint32_t*)(tile + rc_f32_offset(base, t, u, lane));
      return f;
    }
  }
};

template <typename T>
struct Mma;

template <>
struct Mma<uint16_t> {
  __device__ __forceinline__ static void mac(f32x4& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                  0, 0, 0);
  }
};

template <>
struct Mma<float> {
  __device__ __forceinline__ static void mac(f32x4& acc, const u32x4& a, const u32x4& b) {
    // the four floats of each fragment feed four K=4 products
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[j]), __uint_as_float(b[j]), acc, 0, 0, 0);
  }
};

// Workgroup barriers of the pipeline.  stage_barrier waits until at most one
// k-tile of this wavefront's direct loads (kDmaSlots per operand each) is
// still in flight, then meets the other wavefronts: after it, every
// wavefront's loads of all older k-tiles have landed.  LDS reads may stay in
// flight across it (their stage is not overwritten before the step that
// uses them).  The scheduling fence keeps the compiler from moving any
// instruction across, so every product of a step, and the wait for the
// fragment reads it uses, comes before that step's barrier.
// drain_barrier waits for everything.
constexpr int kLoadsPerTile = 2 * kDmaSlots;  // direct loads per wavefront per k-tile
__device__ __forceinline__ void stage_barrier() {
  static_assert(kLoadsPerTile == 4, "the vmcnt literal assumes one k-tile of 2 x kDmaSlots loads");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// The same with N loads of the wavefront allowed in flight (the k-tile's
// direct loads issued last, plus N - kLoadsPerTile loads issued after them).
template <int N>
__device__ __forceinline__ void stage_barrier_n() {
  static_assert(N >= kLoadsPerTile && N < 64, "vmcnt holds 0..63");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void drain_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Orders a wavefront's own LDS accesses for the compiler.  The hardware
// performs one wavefront's LDS instructions in order, so a slab that only its
// own wavefront touches needs no barrier between writing and reading it.
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

struct GemmArgs {
  int M, N, K;
  int tiles_m, tiles_n, group_m;
  const void* a;
  int64_t lda;
  uint32_t a_span;  // bytes the A operand spans (< 2 GiB)
  const void* b;
  int64_t ldb;
  uint32_t b_span;
  int b_split;  // > 0: B (row-contiguous) read in the SwiGLU column order, gate/up halves at b_split
};

// A fragment index after whose products a k-step issues its direct loads
// (see kstep), for every operand layout.
constexpr int kDmaIssueAfter = 3;

// Fragments of one k-tile held in registers.
struct Frags {
  u32x4 a[kFragM], b[kFragN];
};

// One step of the k-pipeline, k-tile kt held in stage S = kt % kStages, its
// fragments already in `cur`:
//   read tile kt + 1's B fragments from stage S + 1 into a second set;
//   for each A fragment mt: run its 4 products of tile kt, then read tile
//   kt + 1's fragment mt into the same registers, so each read has about a
//   whole step to land before its products in the next step;
//   after the products of A fragment kDmaIssueAfter, issue the direct loads of tile
//   kt + kStages - 1 into stage (S - 1) mod kStages, which held tile kt - 1
//   (read in step kt - 2, used before the barrier of step kt - 1);
//   stage_barrier: at most tile kt + 3 is still in flight, so tile kt + 2,
//   which the next step reads, has landed everywhere.
// The scheduling fences pin this order (left alone, the scheduler sinks the
// reads behind the products).  Tiles past the end of K load as zeros; their
// fragments are read but never multiplied.
//
// Why the loads are issued mid-step: every wavefront of the workgroup leaves
// the barrier together, and the two wavefronts of a SIMD would otherwise
// both spend their first ~40 instructions on load addressing while the
// matrix unit idles.  Issued behind 16 products (256 matrix-core cycles),
// the addressing overlaps them; measured at the 7B second-GEMM shape under
// the power cap, 1.7-2.4% faster than issuing first (after 1 fragment: 1.2%,
// after 4-7: 0.3-0.8%; the A and B loads split over two points: 0.6-1.7%).
// The weight-gradient products (both operands row-contiguous) gain more: the
// 7B backward is 4.3% faster with their loads after fragment 3 than first
// (after 2: 3.9%, 4: 2.8%, 5: 2.3%).
template <typename T, bool A_KC, bool B_KC, int S, int A_L = kLayKC, int B_L = kLayKC>
__device__ __forceinline__ void kstep(char* const (&st)[kStages], const Dma<T, A_KC, A_L>& da,
                                      const Dma<T, B_KC, B_L>& db, FragReader<T, A_KC, lds_packed(A_L)>& ra,
                                      FragReader<T, B_KC, lds_packed(B_L)>& rb,
                                      f32x4 (&acc)[kFragM][kFragN], Frags& cur, int kt, int K, int wave) {
  constexpr int SL = (S + kStages - 1) % kStages;
  constexpr int SN = (S + 1) % kStages;
  constexpr int issue_at = kDmaIssueAfter;
  ra.refresh();
  rb.refresh();
  u32x4 nb[kFragN];
#pragma unroll
  for (int nt = 0; nt < kFragN; ++nt) nb[nt] = rb.read(st[SN] + kOperandBytes, nt);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int mt = 0; mt < kFragM; ++mt) {
#pragma unroll
    for (int nt = 0; nt < kFragN; ++nt) Mma<T>::mac(acc[mt][nt], cur.a[mt], cur.b[nt]);
    cur.a[mt] = ra.read(st[SN], mt);
    if (mt == issue_at) {
      da.issue(st[SL], kt + kStages - 1, K, wave);
      db.issue(st[SL] + kOperandBytes, kt + kStages - 1, K, wave);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int nt = 0; nt < kFragN; ++nt) cur.b[nt] = nb[nt];
  stage_barrier();
}

// The epilogue sees the wavefront's accumulators 16 rows at a time, staged
// through a slab of LDS private to the wavefront (after drain_barrier the
// stages are free), so that each lane holds 8 consecutive columns of one row:
// lane l, slot q (0..1) gets row (l/8 + 8q) of the 16-row slab and columns
// [8*(l%8), 8*(l%8)+8) of the wavefront's 64.  Epi provides
//   apply(mt, q, row, col, v)  for rows < M and columns < N (col % 8 == 0);
//                              row = row_base + 16 mt + l/8 + 8 q
//                              (epi_row), v[8] the accumulators
//   end_slab(mt, slab_row0)    after all lanes applied 16-row slab mt
//   finish()                   on every lane after the last slab
// An epilogue that stages data of its own in LDS declares kLdsBytes (per
// wavefront) and set_lds(char*); only the fp8 kernel hands out such room.
// A_L, B_L: OpLayout of a contraction-contiguous operand.
template <class E, class = void>
struct epi_lds_bytes {
  static constexpr int value = 0;
};
template <class E>
struct epi_lds_bytes<E, std::void_t<decltype(E::kLdsBytes)>> {
  static constexpr int value = E::kLdsBytes;
};

template <typename T, bool A_KC, bool B_KC, class Epi, int A_L = kLayKC, int B_L = kLayKC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_kernel(
    GemmArgs g, typename Epi::Params ep) {
  static_assert(kStages == 4, "the stage arrays and the unrolled steps below assume four stages");
  static_assert((A_L == kLayKC || A_KC) && (B_L == kLayKC || B_KC), "only contraction-contiguous operands are packed");
  static_assert((A_L != kLayPacked && B_L != kLayPacked) || sizeof(T) == 2, "tile-packed operands are bf16");
  static_assert(epi_lds_bytes<Epi>::value == 0, "this kernel gives its epilogues no LDS of their own");
  __shared__ __attribute__((aligned(1024))) char st0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char st1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char st2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char st3[kStageBytes];
  char* const st[kStages] = {st0, st1, st2, st3};
  constexpr int KTE = kKTBytes / (int)sizeof(T);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  int tm, tn;
  map_tile(blockIdx.x, g.tiles_m, g.tiles_n, g.group_m, &tm, &tn);
  const int m0 = tm * kTileM, n0 = tn * kTileN;

  Dma<T, A_KC, A_L> da;
  Dma<T, B_KC, B_L> db;
  da.init(g.a, g.a_span, g.lda, m0, g.M, wave, lane);
  db.init(g.b, g.b_span, g.ldb, n0, g.N, wave, lane, B_KC ? 0 : g.b_split);
  FragReader<T, A_KC, lds_packed(A_L)> ra(wm * kWaveM, lane);
  FragReader<T, B_KC, lds_packed(B_L)> rb(wn * kWaveN, lane);
  f32x4 acc[kFragM][kFragN];
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (g.K + KTE - 1) / KTE;
  // prologue: tiles 0 .. kStages - 2 in flight, wait for tiles 0 and 1
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t) {
    da.issue(st[t], t, g.K, wave);
    db.issue(st[t] + kOperandBytes, t, g.K, wave);
  }
  static_assert((kStages - 3) * kLoadsPerTile == 4, "the prologue vmcnt literal assumes kStages - 3 tiles in flight");
  asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
  Frags cur;
#pragma unroll
  for (int mt = 0; mt < kFragM; ++mt) cur.a[mt] = ra.read(st[0], mt);
#pragma unroll
  for (int nt = 0; nt < kFragN; ++nt) cur.b[nt] = rb.read(st[0] + kOperandBytes, nt);
  int kt = 0;
  for (; kt + kStages <= nk; kt += kStages) {
    kstep<T, A_KC, B_KC, 0, A_L, B_L>(st, da, db, ra, rb, acc, cur, kt, g.K, wave);
    kstep<T, A_KC, B_KC, 1, A_L, B_L>(st, da, db, ra, rb, acc, cur, kt + 1, g.K, wave);
    kstep<T, A_KC, B_KC, 2, A_L, B_L>(st, da, db, ra, rb, acc, cur, kt + 2, g.K, wave);
    kstep<T, A_KC, B_KC, 3, A_L, B_L>(st, da, db, ra, rb, acc, cur, kt + 3, g.K, wave);
  }
  // ragged end: the remaining nk - kt < kStages tiles start again at stage 0
  const int rem = nk - kt;
  if (rem > 0) kstep<T, A_KC, B_KC, 0, A_L, B_L>(st, da, db, ra, rb, acc, cur, kt, g.K, wave);
  if (rem > 1) kstep<T, A_KC, B_KC, 1, A_L, B_L>(st, da, db, ra, rb, acc, cur, kt + 1, g.K, wave);
  if (rem > 2) kstep<T, A_KC, B_KC, 2, A_L, B_L>(st, da, db, ra, rb, acc, cur, kt + 2, g.K, wave);
  drain_barrier();  // no direct load may land in the LDS the epilogue reuses

  // ---- epilogue ----
  Epi epi(ep, lane, wm, wn, m0, n0, tn, g.M, g.N);
  float* slab = (float*)(((wave & 3) == 0 ? st0 : (wave & 3) == 1 ? st1 : (wave & 3) == 2 ? st2 : st3) +
                         (wave >> 2) * kEpiSlabBytes);
  const int row_base = m0 + wm * kWaveM;
  const int col = n0 + wn * kWaveN + (lane & 7) * 8;
#pragma unroll
  for (int mt = 0; mt < kFragM; ++mt) {
#pragma unroll
    for (int nt = 0; nt < kFragN; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) slab[(4 * (lane >> 4) + e) * kEpiPitch + nt * 16 + (lane & 15)] = acc[mt][nt][e];
    wave_lds_fence();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int rl = (lane >> 3) + 8 * q;
      const float* src = slab + rl * kEpiPitch + (lane & 7) * 8;
      const f32x4 lo = *(const f32x4*)src, hi = *(const f32x4*)(src + 4);
      float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const int row = row_base + mt * 16 + rl;
      if (row < g.M && col < g.N) epi.apply(mt, q, row, col, v);
    }
    epi.end_slab(mt, row_base + mt * 16);
    wave_lds_fence();  // the slab's reads are done before the next slab overwrites it
  }
  epi.finish();
}

}  // namespace coda
