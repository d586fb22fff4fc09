// Epilogues of the chain's GEMMs with fp8 (OCP e4m3) operands.
//
// The operands carry float32 dequantisation scales: A per row (sa), the
// weights per output channel (sw).  A product's accumulator is
// acc = sum_k code(A)_ik code(W)_jk, so the dequantised product is
// acc * sa_i * sw_j; the epilogue applies both scales (vector loads of the
// CODA news article by Synced, section "五种「积木」和一套「乐高语言」")
// before the chain's own epilogue work.
#pragma once

#include "epilogues.hpp"

namespace coda {

// float -> e4m3 with magnitudes clamped to 448 first: the conversion
// instruction rounds to nearest-even but turns values past the largest
// finite code into NaN.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  const float m = 448.f;
  a = fminf(fmaxf(a, -m), m);
  b = fminf(fmaxf(b, -m), m);
  c = fminf(fmaxf(c, -m), m);
  d = fminf(fmaxf(d, -m), m);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Column scales of a lane's 8 columns.
__device__ __forceinline__ void load_col_scales(const float* sw, int col, int N, float out[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = 0.f;
  if (col < N) {
    const f32x4 lo = *(const f32x4*)(sw + col), hi = *(const f32x4*)(sw + col + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[i] = lo[i];
      out[4 + i] = hi[i];
    }
  }
}

// First GEMM, fp8 operands:
//   H   = round_bf16((acc * sa_i) * sw_j + R_ij)                 bf16 [M, D]
//   Hg8 = e4m3(clamp(float(H_ij) * g_j, +-448))                  e4m3 [M, D]
//   partials[t][row] = sum over partial tile t of float(H)^2    (as in EpiResPrms)
struct EpiResPrmsFp8 {
  struct Params {
    const float* sa;    // [M]
    const float* sw;    // [D]
    const uint16_t* R;  // bf16
    int64_t ldr;
    const uint16_t* g;  // bf16 [D]
    uint16_t* H;        // bf16
    int64_t ldh;
    uint8_t* Hg8;       // e4m3
    int64_t ldhg;
    float* partials;    // [T][M]
    int64_t hg_nck;     // > 0: Hg8 is tile-packed (kp_unit) with hg_nck 16-byte chunks per row
  };
  Params p;
  RowChunks<uint16_t> rc;
  RowScalars sa;
  float sw[8], gv[8];
  float ss[2];
  int lane, t, M;

  __device__ __forceinline__ EpiResPrmsFp8(const Params& p_, int lane_, int wm, int wn, int m0, int n0, int tn,
                                           int M_, int N)
      : p(p_), lane(lane_), t(4 * tn + wn), M(M_) {
    const int col = n0 + wn * kWaveN + (lane & 7) * 8;
    rc.prefetch(p.R, p.ldr, m0 + wm * kWaveM, col, lane, M_, N);
    sa.prefetch(p.sa, m0 + wm * kWaveM, lane, M_);
    load_col_scales(p.sw, col, N, sw);
#pragma unroll
    for (int i = 0; i < 8; ++i) gv[i] = 0.f;
    if (col < N) Chunk8<uint16_t>::load(p.g + col, gv);
    ss[0] = ss[1] = 0.f;
  }

  __device__ __forceinline__ void apply(int mt, int q, int row, int col, float v[8]) {
    float rv[8], h[8];
    rc.get(p.R, p.ldr, mt, q, row, col, rv);
    const float s = sa.v[mt][q];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h[i] = Chunk8<uint16_t>::round((v[i] * s) * sw[i] + rv[i]);
      ss[q] += h[i] * h[i];
    }
    Chunk8<uint16_t>::store(p.H + (int64_t)row * p.ldh + col, h);
    const uint32_t lo = pack_e4m3x4(h[0] * gv[0], h[1] * gv[1], h[2] * gv[2], h[3] * gv[3]);
    const uint32_t hi = pack_e4m3x4(h[4] * gv[4], h[5] * gv[5], h[6] * gv[6], h[7] * gv[7]);
    uint8_t* dst = p.hg_nck > 0 ? p.Hg8 + kp_unit(row, col >> 4, p.hg_nck) * 16 + (col & 15)
                                : p.Hg8 + (int64_t)row * p.ldhg + col;
    *(u32x2*)dst = u32x2{lo, hi};
  }

  __device__ __forceinline__ void end_slab(int, int slab_row0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float s = ss[q];
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      const int row = slab_row0 + (lane >> 3) + 8 * q;
      if ((lane & 7) == 0 && row < M) p.partials[(int64_t)t * M + row] = s;
      ss[q] = 0.f;
    }
  }
  __device__ __forceinline__ void finish() {}
};

// Second GEMM, fp8 operands: Y = round_bf16((acc * r_i) * sw_k), r may be
// null (then only the column scales apply).
struct EpiRowScaleFp8 {
  struct Params {
    const float* r;  // [M] or null
    const float* sw;  // [N2]
    uint16_t* Y;      // bf16
    int64_t ldy;
  };
  Params p;
  RowScalars rs;
  float sw[8];
  __device__ __forceinline__ EpiRowScaleFp8(const Params& p_, int lane, int wm, int wn, int m0, int n0, int, int M,
                                            int N)
      : p(p_) {
    if (p.r != nullptr) rs.prefetch(p.r, m0 + wm * kWaveM, lane, M);
    load_col_scales(p.sw, n0 + wn * kWaveN + (lane & 7) * 8, N, sw);
  }
  __device__ __forceinline__ void apply(int mt, int q, int row, int col, float v[8]) {
    const float s = p.r != nullptr ? rs.v[mt][q] : 1.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (v[i] * s) * sw[i];
    Chunk8<uint16_t>::store(p.Y + (int64_t)row * p.ldy + col, v);
  }
  __device__ __forceinline__ void end_slab(int, int) {}
  __device__ __forceinline__ void finish() {}
};

// Dequantisation in front of another epilogue: the accumulator of a product
// of e4m3 operands quantised with row scales sa (A's rows) and sb (B's rows,
// the output columns) is v = (acc * sa[row]) * sb[col]; Inner then sees v as
// if the product had been taken in full precision.
template <class Inner>
struct EpiDequant {
  struct Params {
    const float* sa;  // [M]
    const float* sb;  // [N]
    typename Inner::Params inner;
  };
  Inner in;
  RowScalars rs;
  float sb[8];
  __device__ __forceinline__ EpiDequant(const Params& p, int lane, int wm, int wn, int m0, int n0, int tn, int M,
                                        int N)
      : in(p.inner, lane, wm, wn, m0, n0, tn, M, N) {
    rs.prefetch(p.sa, m0 + wm * kWaveM, lane, M);
    load_col_scales(p.sb, n0 + wn * kWaveN + (lane & 7) * 8, N, sb);
  }
  __device__ __forceinline__ void apply(int mt, int q, int row, int col, float v[8]) {
    const float s = rs.v[mt][q];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (v[i] * s) * sb[i];
    in.apply(mt, q, row, col, v);
  }
  __device__ __forceinline__ void end_slab(int mt, int slab_row0) { in.end_slab(mt, slab_row0); }
  __device__ __forceinline__ void finish() { in.finish(); }
};

}  // namespace coda
