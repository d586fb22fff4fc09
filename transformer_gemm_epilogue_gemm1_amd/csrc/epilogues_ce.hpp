// Epilogue of the LM-head GEMM for the cross-entropy backward.
#pragma once

#include "epilogues.hpp"

namespace coda {

// Gradient of sum_i dloss_i loss_i with respect to the logits, straight from
// the recomputed LM-head accumulators (the backward of the cross-entropy head
// the CODA news article by Synced, epilogue section, says the
// re-parameterisation covers).  With y = r[row] * acc and the forward's lse:
//   dY_row,j = round(dloss[row] * (e^(y - lse[row]) - [j == t_row]))
// A target outside [0, V) gives a NaN row (its loss was NaN).  The row
// values (r, lse, dloss, target) are loaded in the constructor; e^x is the
// hardware exp2 of x log2(e), as in the forward statistics.
template <typename T>
struct EpiCEGrad {
  struct Params {
    const float* r;      // [M] or null
    const int* targets;  // [M]
    const float* lse;    // [M]
    const float* dloss;  // [M]
    T* dY;
    int64_t lddy;
    int V;
  };
  Params p;
  RowScalars rs, ls, dl;
  int tg[kFragM][2];
  __device__ __forceinline__ EpiCEGrad(const Params& p_, int lane, int wm, int, int m0, int, int, int M, int)
      : p(p_) {
    const int row_base = m0 + wm * kWaveM;
    if (p.r != nullptr) rs.prefetch(p.r, row_base, lane, M);
    ls.prefetch(p.lse, row_base, lane, M);
    dl.prefetch(p.dloss, row_base, lane, M);
#pragma unroll
    for (int mt = 0; mt < kFragM; ++mt)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row = epi_row(row_base, mt, q, lane);
        tg[mt][q] = row < M ? p.targets[row] : 0;
      }
  }
  __device__ __forceinline__ void apply(int mt, int q, int row, int col, float v[8]) {
    const float s = p.r != nullptr ? rs.v[mt][q] : 1.f;
    const float l = ls.v[mt][q], d = dl.v[mt][q];
    const int t = tg[mt][q];
    const bool ok = (unsigned)t < (unsigned)p.V;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = __builtin_amdgcn_exp2f((v[i] * s - l) * 1.4426950408889634f);
      const float g = d * (col + i == t ? e - 1.f : e);
      v[i] = ok ? g : __builtin_nanf("");
    }
    Chunk8<T>::store(p.dY + (int64_t)row * p.lddy + col, v);
  }
  __device__ __forceinline__ void end_slab(int, int) {}
  __device__ __forceinline__ void finish() {}
};

}  // namespace coda
