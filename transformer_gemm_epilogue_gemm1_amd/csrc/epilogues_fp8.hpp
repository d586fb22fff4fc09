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

// Block exponent of the OCP microscaling formats for a block whose largest
// magnitude is amax: the smallest integer E with amax <= 448 * 2^E, so that
// amax * 2^-E fits e4m3 without saturating, clamped to the E8M0 range
// [-127, 127]; 0 for an all-zero block.  With amax = m 2^e, m in [0.5, 1),
// and 448 = 0.875 * 2^9: E = e - 9, or e - 8 when m > 0.875.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int e;
  const float m = frexpf(amax, &e);
  const int E = e - 9 + (m > 0.875f ? 1 : 0);
  return E < -127 ? -127 : (E > 127 ? 127 : E);
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
//   x   = float(H_ij) * g_j                                      float32
//   E_ib = mx_exponent(max |x| over block b = columns [32b, 32b + 32) of row i)
//   Hg8 = e4m3(x * 2^-E_ib)                                      e4m3 [M, D]
//   hg_exp[mx_byte(i, b / 2, b % 2, M)] = E_ib + 127            E8M0 bytes
//   partials[t][row] = sum over partial tile t of float(H)^2    (as in EpiResPrms)
// A block's 32 columns are 4 lanes of a row group (lanes l with equal l / 4),
// so the block maximum is two lane exchanges (a tile reduction of the CODA
// news article's building blocks).  apply() keeps x; end_slab(), which
// every lane runs, takes the block maxima and writes codes and exponents.
// Every byte of the exponent array is written: its groups of 4 k-tiles
// cover exactly the 256-column tiles, its row blocks the rows up to M
// rounded up to 128 (whose lanes run end_slab with x = 0), and a block past
// D or a padding row gets exponent 0.  The second GEMM reads whole groups.
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
    uint8_t* hg_exp;    // block exponents (mx_byte layout), 1024 ceil(M / 128) ceil(D / 256) bytes
  };
  Params p;
  RowChunks<uint16_t> rc;
  RowScalars sa;
  float sw[8], gv[8];
  float ss[2];
  float xg[2][8];  // x of the lane's two rows of the current slab (0 where not applied)
  int lane, t, M, N, col;

  __device__ __forceinline__ EpiResPrmsFp8(const Params& p_, int lane_, int wm, int wn, int m0, int n0, int tn,
                                           int M_, int N_)
      : p(p_), lane(lane_), t(4 * tn + wn), M(M_), N(N_) {
    col = n0 + wn * kWaveN + (lane & 7) * 8;
    rc.prefetch(p.R, p.ldr, m0 + wm * kWaveM, col, lane, M_, N_);
    sa.prefetch(p.sa, m0 + wm * kWaveM, lane, M_);
    load_col_scales(p.sw, col, N_, sw);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      gv[i] = 0.f;
      xg[0][i] = xg[1][i] = 0.f;
    }
    if (col < N_) Chunk8<uint16_t>::load(p.g + col, gv);
    ss[0] = ss[1] = 0.f;
  }

  __device__ __forceinline__ void apply(int mt, int q, int row, int col_, float v[8]) {
    float rv[8], h[8];
    rc.get(p.R, p.ldr, mt, q, row, col_, rv);
    const float s = sa.v[mt][q];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h[i] = Chunk8<uint16_t>::round((v[i] * s) * sw[i] + rv[i]);
      ss[q] += h[i] * h[i];
      xg[q][i] = h[i] * gv[i];
    }
    Chunk8<uint16_t>::store(p.H + (int64_t)row * p.ldh + col_, h);
  }

  __device__ __forceinline__ void end_slab(int, int slab_row0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float s = sum8(ss[q]);
      const int row = slab_row0 + (lane >> 3) + 8 * q;
      if ((lane & 7) == 0 && row < M) p.partials[(int64_t)t * M + row] = s;
      ss[q] = 0.f;
      // the block of 32 columns: its maximum over the 4 lanes holding it
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(xg[q][i]));
      a = max4(a);
      const int E = mx_exponent(a);
      if (row < M && col < N) {
        const uint32_t lo = pack_e4m3x4(ldexpf(xg[q][0], -E), ldexpf(xg[q][1], -E), ldexpf(xg[q][2], -E),
                                        ldexpf(xg[q][3], -E));
        const uint32_t hi = pack_e4m3x4(ldexpf(xg[q][4], -E), ldexpf(xg[q][5], -E), ldexpf(xg[q][6], -E),
                                        ldexpf(xg[q][7], -E));
        uint8_t* dst = p.hg_nck > 0 ? p.Hg8 + kp_unit(row, col >> 4, p.hg_nck) * 16 + (col & 15)
                                    : p.Hg8 + (int64_t)row * p.ldhg + col;
        *(u32x2*)dst = u32x2{lo, hi};
      }
      if ((lane & 3) == 0 && row < 128 * mx_row_blocks(M))
        p.hg_exp[mx_byte(row, col >> 6, (col >> 5) & 1, M)] = (uint8_t)(E + 127);
#pragma unroll
      for (int i = 0; i < 8; ++i) xg[q][i] = 0.f;
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

// Backward, first product G = dY W2^T on e4m3 operands (the fp8 backward):
// EpiBwdG's P, row sums and column sums, with X_n leaving as the operand the
// weight gradient dW2 = X_n^T dY reads, instead of as bf16.  X_n is rounded
// to bf16 first (the stored value the recipe quantises) and then coded along
// its columns with MX block exponents, as the MX quantiser codes a matrix's
// columns: per column j and block of 32 rows b, E = mx_exponent(max |X_n|),
// byte E + 127 at mx_byte(j, b / 2, b % 2, D) of exn, and the codes
// e4m3(X_n 2^-E) as the rows of X_n^T [D, M], tile-packed (kp_unit with M / 16
// units per row) in xnt8.  A block is two epilogue slabs: the wavefront keeps
// its 32 x 64 values in LDS, and after the second slab lane l takes column l
// of the wavefront's 64 (one read pass for the maximum, one per 16-row unit
// for the codes).  Values outside X (rows >= M, columns >= D) read as 0, so
// every exponent byte the array holds is written: 127 for padding rows and
// for blocks past M, as the quantiser writes them.
struct EpiBwdGMx : EpiBwdG<uint16_t> {
  using Base = EpiBwdG<uint16_t>;
  struct Params {
    Base::Params b;  // b.Xn is not used
    uint8_t* xnt8;
    uint8_t* exn;
  };
  static constexpr int kLdsBytes = 32 * kWaveN * 4;
  uint8_t* xnt8;
  uint8_t* exn;
  float* xs;  // [32][kWaveN] X_n values of the current block
  int row0, col0;

  __device__ __forceinline__ EpiBwdGMx(const Params& p_, int lane_, int wm, int wn, int m0, int n0, int tn, int M_,
                                       int N_)
      : Base(p_.b, lane_, wm, wn, m0, n0, tn, M_, N_), xnt8(p_.xnt8), exn(p_.exn), xs(nullptr) {
    row0 = m0 + wm * kWaveM;
    col0 = n0 + wn * kWaveN;
  }

  // the lane's own positions of a block: rows 16 s + l / 8 + 8 q, columns
  // 8 (l % 8) .. + 7
  __device__ __forceinline__ void zero_own() {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float* d = xs + (16 * s + (lane >> 3) + 8 * q) * kWaveN + 8 * (lane & 7);
        *(f32x4*)d = f32x4{0.f, 0.f, 0.f, 0.f};
        *(f32x4*)(d + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
  }
  __device__ __forceinline__ void set_lds(char* lds) {
    xs = (float*)lds;
    zero_own();
  }

  __device__ __forceinline__ void apply(int mt, int q, int row, int col_, float v[8]) {
    float xv[8];
    apply_p(mt, q, row, col_, v, xv);
#pragma unroll
    for (int i = 0; i < 8; ++i) xv[i] = Chunk8<uint16_t>::round(xv[i]);
    float* d = xs + (16 * (mt & 1) + (lane >> 3) + 8 * q) * kWaveN + 8 * (lane & 7);
    *(f32x4*)d = f32x4{xv[0], xv[1], xv[2], xv[3]};
    *(f32x4*)(d + 4) = f32x4{xv[4], xv[5], xv[6], xv[7]};
  }

  __device__ __forceinline__ void end_slab(int mt, int slab_row0) {
    Base::end_slab(mt, slab_row0);
    if (mt & 1) {
      const int br = slab_row0 - 16;  // the block's first row
      wave_lds_fence();
      float a = 0.f;
#pragma unroll
      for (int r = 0; r < 32; ++r) a = fmaxf(a, fabsf(xs[r * kWaveN + lane]));
      const int E = mx_exponent(a);
      const int crow = col0 + lane;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (crow < N && br + 16 * h < M) {
          u32x4 o;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float* x = xs + (16 * h + 4 * k) * kWaveN + lane;
            o[k] = pack_e4m3x4(ldexpf(x[0], -E), ldexpf(x[kWaveN], -E), ldexpf(x[2 * kWaveN], -E),
                               ldexpf(x[3 * kWaveN], -E));
          }
          *(u32x4*)(xnt8 + kp_unit(crow, (br >> 4) + h, M >> 4) * 16) = o;
        }
      }
      if (crow < 128 * mx_row_blocks(N)) exn[mx_byte(crow, br >> 6, (br >> 5) & 1, N)] = (uint8_t)(E + 127);
      wave_lds_fence();  // the block's reads are done before the next block's writes
      zero_own();
    }
  }
};

}  // namespace coda
