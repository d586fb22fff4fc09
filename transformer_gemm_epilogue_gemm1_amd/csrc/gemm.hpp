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
// Workgroup: 256 threads = 4 wavefronts (2 x 2), a 256 x 256 output tile,
// each wavefront a 128 x 128 sub-tile held as 8 x 8 MFMA 16x16 accumulators
// (256 fp32 per lane).  Per k-tile (128 bytes of contraction = 64 bf16 or 32
// fp32) both operand tiles are loaded from HBM into registers, written to a
// double-buffered, XOR-swizzled LDS stage ([row][k], contraction contiguous;
// row-contiguous operands are transposed in registers on the way), and read
// back as MFMA fragments:
//   bf16: v_mfma_f32_16x16x32_bf16, one 16-byte fragment per lane per operand
//   fp32: v_mfma_f32_16x16x4_f32, the 4 floats of a fragment feed 4 MFMAs
// Lane l of a 16x16 fragment holds operand row (l % 16) and contraction chunk
// (l / 16); accumulator element e of lane l is output (4*(l/16)+e, l%16).
// The contraction order inside one MFMA is the same for A and B, so the
// product does not depend on how the hardware orders the k values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// ---- operand staging: HBM -> registers -> LDS ---------------------------
// Global reads go through a raw buffer descriptor spanning exactly the
// operand's bytes.  A slot that falls outside the matrix (row >= rows,
// contraction index >= K) gets an offset past the descriptor's extent, for
// which the hardware returns zeros: no load ever leaves the operand and no
// select has to wait for the load to land.
constexpr uint32_t kOutOfRange = 0x80000000u;  // every operand spans < 2 GiB

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t span_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)span_bytes, 0x00020000);
}

template <typename T, bool KC>
struct Stager {
  static constexpr int E = Elem<T>::E;
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[8];  // byte offset of each slot for the k-tile at k0 = 0 (kOutOfRange: row outside)
  int kidx[8];      // contraction index of each slot's first element at k0 = 0
  u32x4 reg[8];

  __device__ __forceinline__ void init(const T* base, uint32_t span_bytes, int64_t ld, int row0, int nrows,
                                       int tid) {
    rsrc = make_rsrc(base, span_bytes);
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int row, c;
        kc_slot(tid, i, &row, &c);
        const int gr = row0 + row;
        kidx[i] = c * E;
        off[i] = gr < nrows ? (uint32_t)(((int64_t)gr * ld + c * E) * (int64_t)sizeof(T)) : kOutOfRange;
      }
    } else {
      constexpr int NB = 8 / E;  // E x E blocks per thread (bf16: 1, fp32: 2)
#pragma unroll
      for (int bi = 0; bi < NB; ++bi) {
        int rb, kb;
        rc_block(tid, bi, E, &rb, &kb);
        const int gr = row0 + rb * E;
#pragma unroll
        for (int j = 0; j < E; ++j) {
          kidx[bi * E + j] = kb * E + j;
          off[bi * E + j] =
              gr < nrows ? (uint32_t)(((int64_t)(kb * E + j) * ld + gr) * (int64_t)sizeof(T)) : kOutOfRange;
        }
      }
    }
  }

  // Loads the k-tile starting at contraction index k0 (a multiple of the
  // k-tile width); k_step_bytes is the byte distance of k0 from k-tile 0.
  __device__ __forceinline__ void load(int k0, uint32_t k_step_bytes, int K) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = (off[i] != kOutOfRange) && (k0 + kidx[i] < K);
      const uint32_t o = ok ? off[i] + k_step_bytes : kOutOfRange;
      reg[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)o, 0, 0);
    }
  }

  __device__ __forceinline__ void store(char* lds, int tid) const {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int row, c;
        kc_slot(tid, i, &row, &c);
        *(u32x4*)(lds + lds_offset(row, c)) = reg[i];
      }
    } else if constexpr (E == 8) {
      // 8 x 8 bf16 transpose: reg[j] holds contraction index j for tile rows
      // rb*8 .. rb*8+7 (two per dword); out[c] gathers tile row c's 8
      // contraction values.
      int rb, kb;
      rc_block(tid, 0, E, &rb, &kb);
      uint32_t in[8][4], out[8][4];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int p = 0; p < 4; ++p) in[j][p] = reg[j][p];
      transpose8x8_b16(in, out);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *(u32x4*)(lds + lds_offset(rb * 8 + c, kb)) = u32x4{out[c][0], out[c][1], out[c][2], out[c][3]};
    } else {
      // 4 x 4 fp32 transpose, two blocks per thread
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        int rb, kb;
        rc_block(tid, bi, E, &rb, &kb);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4 o{reg[bi * 4 + 0][c], reg[bi * 4 + 1][c], reg[bi * 4 + 2][c], reg[bi * 4 + 3][c]};
          *(u32x4*)(lds + lds_offset(rb * 4 + c, kb)) = o;
        }
      }
    }
  }
};

// ---- one k-tile of MFMAs from an LDS stage ------------------------------
template <typename T>
struct Mma;

template <>
struct Mma<uint16_t> {
  __device__ __forceinline__ static void run(const char* As, const char* Bs, f32x4 (&acc)[8][8], int lane,
                                             int wm, int wn) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = ks * 4 + (lane >> 4);
      bf16x8 af[8], bfr[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int ra = wm * 128 + t * 16 + (lane & 15);
        const int rbn = wn * 128 + t * 16 + (lane & 15);
        af[t] = __builtin_bit_cast(bf16x8, *(const u32x4*)(As + lds_offset(ra, ch)));
        bfr[t] = __builtin_bit_cast(bf16x8, *(const u32x4*)(Bs + lds_offset(rbn, ch)));
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bfr[nt], acc[mt][nt], 0, 0, 0);
    }
  }
};

template <>
struct Mma<float> {
  __device__ __forceinline__ static void run(const char* As, const char* Bs, f32x4 (&acc)[8][8], int lane,
                                             int wm, int wn) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = ks * 4 + (lane >> 4);
      f32x4 af[8], bfr[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int ra = wm * 128 + t * 16 + (lane & 15);
        const int rbn = wn * 128 + t * 16 + (lane & 15);
        af[t] = *(const f32x4*)(As + lds_offset(ra, ch));
        bfr[t] = *(const f32x4*)(Bs + lds_offset(rbn, ch));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int nt = 0; nt < 8; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[mt][j], bfr[nt][j], acc[mt][nt], 0, 0, 0);
    }
  }
};

struct GemmArgs {
  int M, N, K;
  int tiles_m, tiles_n, group_m;
  const void* a;
  int64_t lda;
  uint32_t a_span;  // bytes the A operand spans (< 2 GiB)
  const void* b;
  int64_t ldb;
  uint32_t b_span;
};

constexpr int kLdsBytes = 4 * kStageBytes;  // two stages x (A tile + B tile) = 128 KiB

// The epilogue sees the wavefront's accumulators 16 rows at a time, staged
// through LDS so that each lane holds 8 consecutive columns of one row:
// lane l, slot q (0..3) gets row (l/16 + 4q) of the 16-row slab and columns
// [8*(l%16), 8*(l%16)+8) of the wavefront's 128.  Epi provides
//   apply(q, row, col, v[8])   for rows < M and columns < N (col % 8 == 0)
//   end_slab(mt, slab_row0)    after all lanes applied one 16-row slab
template <typename T, bool A_KC, bool B_KC, class Epi>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_kernel(
    GemmArgs g, typename Epi::Params ep) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  constexpr int KT = kRowBytes / sizeof(T);  // contraction elements per k-tile
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  map_tile(blockIdx.x, g.tiles_m, g.tiles_n, g.group_m, &tm, &tn);
  const int m0 = tm * kTileM, n0 = tn * kTileN;

  Stager<T, A_KC> sa;
  Stager<T, B_KC> sb;
  sa.init((const T*)g.a, g.a_span, g.lda, m0, g.M, tid);
  sb.init((const T*)g.b, g.b_span, g.ldb, n0, g.N, tid);
  // byte step per k-tile: along a row (contraction contiguous) or down rows
  const uint32_t a_step = A_KC ? (uint32_t)kRowBytes : (uint32_t)(KT * g.lda * (int64_t)sizeof(T));
  const uint32_t b_step = B_KC ? (uint32_t)kRowBytes : (uint32_t)(KT * g.ldb * (int64_t)sizeof(T));
  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (g.K + KT - 1) / KT;
  sa.load(0, 0, g.K);
  sb.load(0, 0, g.K);
  sa.store(lds, tid);
  sb.store(lds + kStageBytes, tid);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const char* As = lds + (kt & 1) * 2 * kStageBytes;
    const char* Bs = As + kStageBytes;
    const bool more = kt + 1 < nk;
    if (more) {
      sa.load((kt + 1) * KT, (uint32_t)(kt + 1) * a_step, g.K);
      sb.load((kt + 1) * KT, (uint32_t)(kt + 1) * b_step, g.K);
    }
    Mma<T>::run(As, Bs, acc, lane, wm, wn);
    if (more) {
      char* nxt = lds + ((kt + 1) & 1) * 2 * kStageBytes;
      sa.store(nxt, tid);
      sb.store(nxt + kStageBytes, tid);
    }
    __syncthreads();
  }

  // ---- epilogue ----
  Epi epi(ep, lane, wm, wn, m0, n0, tn, g.M, g.N);
  float* slab = (float*)(lds + wave * 16 * kEpiPitch * 4);
  const int row_base = m0 + wm * 128;
  const int col = n0 + wn * 128 + (lane & 15) * 8;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) slab[(4 * (lane >> 4) + e) * kEpiPitch + nt * 16 + (lane & 15)] = acc[mt][nt][e];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rl = (lane >> 4) + 4 * q;
      const float* src = slab + rl * kEpiPitch + (lane & 15) * 8;
      const f32x4 lo = *(const f32x4*)src, hi = *(const f32x4*)(src + 4);
      float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const int row = row_base + mt * 16 + rl;
      if (row < g.M && col < g.N) epi.apply(q, row, col, v);
    }
    epi.end_slab(row_base + mt * 16);
    __syncthreads();
  }
}

}  // namespace coda
