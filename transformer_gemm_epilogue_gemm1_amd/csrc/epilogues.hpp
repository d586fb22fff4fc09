// Epilogues of the chain's GEMMs, run on the accumulators before write-back.
//
// Building blocks (CODA news article by Synced, section
// "五种「积木」和一套「乐高语言」"): element-wise (residual add), vector load
// (the broadcast RMSNorm weight g, the per-row scale r), tile load/store (R in,
// H out), tile reduction (partial sums of squares per row).
//
// The GEMM kernel hands each lane 8 consecutive columns `col .. col+7` of one
// row through apply(q, row, col, v) (q = which of the lane's 2 rows of the
// current 16-row slab), and calls end_slab(slab_row0) on every lane once the
// slab is done.  Lanes l and l' with l/8 == l'/8 hold the same rows; the 8
// lanes of such a group together cover the wavefront's 64 columns.
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
};

}  // namespace coda
