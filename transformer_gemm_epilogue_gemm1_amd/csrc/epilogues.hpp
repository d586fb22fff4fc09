// Epilogues of the chain's GEMMs, run on the accumulators before write-back.
//
// Building blocks (CODA news article by Synced, section
// "五种「积木」和一套「乐高语言」"): element-wise (residual add), vector load
// (the broadcast RMSNorm weight g, the per-row scale r), tile load/store (R in,
// H out), tile reduction (partial sums of squares per row).
//
// The GEMM kernel hands each lane 8 consecutive columns `col .. col+7` of one
// row through apply(q, row, col, v) (q = which of the lane's 2 rows of the
// current 16-row slab), calls end_slab(slab_row0) on every lane once the
// slab is done, and finish() on every lane after the last slab.  Lanes l and
// l' with l/8 == l'/8 hold the same rows; the 8 lanes of such a group
// together cover the wavefront's 64 columns, and lanes with equal l % 8 hold
// the same 8 columns in every slab.
#pragma once

#include "gemm.hpp"

namespace coda {

// First GEMM of the chain: H = round(acc + R), Hg = round(float(H) * g),
// partials[t][row] = sum over the 64 columns of partial tile t of float(H)^2
// with t = 4 * (column tile) + (column quarter of the workgroup).  The squares
// use the stored (rounded) H so that r computed from them normalises exactly
// the H that is kept for the backward.
template <typename T>
struct EpiResPrms {
  struct Params {
    const T* R;
    int64_t ldr;
    const T* g;  // may be null (then Hg is not written)
    T* H;
    int64_t ldh;
    T* Hg;
    int64_t ldhg;
    float* partials;  // [T][M]
  };
  Params p;
  float gv[8];
  float ss[2];
  int lane, t, M;

  __device__ __forceinline__ EpiResPrms(const Params& p_, int lane_, int wm, int wn, int m0, int n0, int tn,
                                        int M_, int N)
      : p(p_), lane(lane_), t(4 * tn + wn), M(M_) {
    (void)wm;
    (void)m0;
    const int col = n0 + wn * kWaveN + (lane & 7) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) gv[i] = 1.f;
    if (p.g != nullptr && col < N) Chunk8<T>::load(p.g + col, gv);
    ss[0] = ss[1] = 0.f;
  }

  __device__ __forceinline__ void apply(int q, int row, int col, float v[8]) {
    float rv[8], h[8];
    Chunk8<T>::load(p.R + (int64_t)row * p.ldr + col, rv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h[i] = Chunk8<T>::round(v[i] + rv[i]);
      ss[q] += h[i] * h[i];
    }
    Chunk8<T>::store(p.H + (int64_t)row * p.ldh + col, h);
    if (p.Hg != nullptr) {
      float hg[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) hg[i] = h[i] * gv[i];
      Chunk8<T>::store(p.Hg + (int64_t)row * p.ldhg + col, hg);
    }
  }

  __device__ __forceinline__ void end_slab(int slab_row0) {
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

// Second GEMM of the chain: the deferred RMSNorm row scale,
// Y = round(r[row] * acc) (r == null: plain GEMM, Y = round(acc)).
template <typename T>
struct EpiRowScale {
  struct Params {
    const float* r;
    T* Y;
    int64_t ldy;
  };
  Params p;
  __device__ __forceinline__ EpiRowScale(const Params& p_, int, int, int, int, int, int, int, int) : p(p_) {}
  __device__ __forceinline__ void apply(int, int row, int col, float v[8]) {
    const float s = p.r != nullptr ? p.r[row] : 1.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= s;
    Chunk8<T>::store(p.Y + (int64_t)row * p.ldy + col, v);
  }
  __device__ __forceinline__ void end_slab(int) {}
  __device__ __forceinline__ void finish() {}
};

// Plain float32 output of the accumulators (the unfused chain's first GEMM).
struct EpiStoreF32 {
  struct Params {
    float* C;
    int64_t ldc;
  };
  Params p;
  __device__ __forceinline__ EpiStoreF32(const Params& p_, int, int, int, int, int, int, int, int) : p(p_) {}
  __device__ __forceinline__ void apply(int, int row, int col, float v[8]) {
    Chunk8<float>::store(p.C + (int64_t)row * p.ldc + col, v);
  }
  __device__ __forceinline__ void end_slab(int) {}
  __device__ __forceinline__ void finish() {}
};

// Backward, first GEMM G = dY W2^T (columns j = 0..D-1 of the chain's hidden
// width).  With the forward's stored H and r and the weight g:
//   P_ij = round(g_j G_ij)                      written into P (the dR buffer)
//   X_n,ij = round((float(H_ij) r_i) g_j)       the normalised activation
//   srow[t][i] = sum over the 64 columns of partial tile t of g_j G_ij H_ij
//   dgcol[u][j] = sum over the 128 rows of row block u of r_i H_ij G_ij
// with t = 4 * (column tile) + (column quarter of the workgroup) and
// u = 2 * (row tile) + (row half of the workgroup), i.e. u = row / 128.
// The row sums reduce over the 8 lanes of a row group, the column sums over
// the 8 lanes sharing a column chunk, in fixed order.
template <typename T>
struct EpiBwdG {
  struct Params {
    const T* H;
    const T* g;
    const float* r;
    T* P;
    T* Xn;
    int64_t ld;        // leading dimension of H, P and Xn (elements)
    float* srow;       // [num_partials][M]
    float* dgcol;      // [ceil(M / 128)][D]
  };
  Params p;
  float gv[8];
  float colsum[8];
  float ss[2];
  int lane, t, M, N, col, u;
  bool rows_in;  // this wavefront holds at least one row < M

  __device__ __forceinline__ EpiBwdG(const Params& p_, int lane_, int wm, int wn, int m0, int n0, int tn, int M_,
                                     int N_)
      : p(p_), lane(lane_), t(4 * tn + wn), M(M_), N(N_) {
    col = n0 + wn * kWaveN + (lane & 7) * 8;
    u = m0 / kWaveM + wm;
    rows_in = m0 + wm * kWaveM < M_;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      gv[i] = 0.f;
      colsum[i] = 0.f;
    }
    if (col < N_) Chunk8<T>::load(p.g + col, gv);
    ss[0] = ss[1] = 0.f;
  }

  __device__ __forceinline__ void apply(int q, int row, int col_, float v[8]) {
    float hv[8], pv[8], xv[8];
    const int64_t o = (int64_t)row * p.ld + col_;
    Chunk8<T>::load(p.H + o, hv);
    const float rr = p.r[row];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = gv[i] * v[i];
      ss[q] += pv[i] * hv[i];
      colsum[i] += (rr * hv[i]) * v[i];
      xv[i] = (hv[i] * rr) * gv[i];
    }
    Chunk8<T>::store(p.P + o, pv);
    Chunk8<T>::store(p.Xn + o, xv);
  }

  __device__ __forceinline__ void end_slab(int slab_row0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float s = ss[q];
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      const int row = slab_row0 + (lane >> 3) + 8 * q;
      if ((lane & 7) == 0 && row < M) p.srow[(int64_t)t * M + row] = s;
      ss[q] = 0.f;
    }
  }

  __device__ __forceinline__ void finish() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float c = colsum[i];
      c += __shfl_xor(c, 8);
      c += __shfl_xor(c, 16);
      c += __shfl_xor(c, 32);
      colsum[i] = c;
    }
    if (lane < 8 && rows_in && col < N) {
      float* dst = p.dgcol + (int64_t)u * N + col;
      *(f32x4*)dst = f32x4{colsum[0], colsum[1], colsum[2], colsum[3]};
      *(f32x4*)(dst + 4) = f32x4{colsum[4], colsum[5], colsum[6], colsum[7]};
    }
  }
};

}  // namespace coda
