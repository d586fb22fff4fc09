// Epilogue of the chain's second GEMM as the attention QKV projection with
// the rotary position embedding.
#pragma once

#include "epilogues.hpp"

namespace coda {

// Second GEMM as a QKV projection with rotary position embedding in the
// epilogue (CODA news article by Synced: the epilogue section says the
// re-parameterisation carries over to RoPE, the building-block section counts
// RoPE among the element-wise transforms).  Columns [0, n_rot) hold query and
// key heads of d_head columns; the columns after them (values) only get the
// row scale.  With y = r[row] * acc, p = positions[row] and
// (c_i, s_i) = cos_sin[p][i] (the table coda_rope_cache writes), the pair
// (2i, 2i + 1) of a head turns by the angle p theta_i:
//   Y_2i = round(y_2i c_i - y_2i+1 s_i),  Y_2i+1 = round(y_2i s_i + y_2i+1 c_i)
// d_head is a multiple of 8, so a lane's 8 columns are 4 whole pairs of one
// head and its 8 table values are 32 contiguous bytes.  A position outside
// [0, max_pos) is never read: that row's rotated columns become NaN.
//
// Table loads run two slabs ahead of their use (double-buffered by slab
// parity) and are unconditional: a lane past the last row, in a value head
// or with an invalid position reads table row 0 and ignores it.  A load under
// a lane-dependent branch would make the compiler merge its result into the
// buffer at the branch's end, which waits for the load right there.
template <typename T>
struct EpiRowScaleRope {
  struct Params {
    const float* r;        // [M] or null
    const int* positions;  // [M]
    const float* cos_sin;  // [max_pos][d_head / 2][2]
    int max_pos, n_rot, d_head;
    T* Y;
    int64_t ldy;
  };
  Params p;
  RowScalars rs;
  int pos[kFragM][2];
  f32x4 cs[2][2][2];  // [slab parity][q][half]: (c, s) of the lane's 4 pairs
  int row_base, lane, head_col;
  bool rot;

  __device__ __forceinline__ void load_cs(int mt) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int pp = pos[mt][q];
      const int idx = (unsigned)pp < (unsigned)p.max_pos ? pp : 0;
      const float* t = p.cos_sin + (int64_t)idx * p.d_head + head_col;
      cs[mt & 1][q][0] = *(const f32x4*)t;
      cs[mt & 1][q][1] = *(const f32x4*)(t + 4);
    }
  }

  __device__ __forceinline__ EpiRowScaleRope(const Params& p_, int lane_, int wm, int wn, int m0, int n0, int,
                                             int M, int)
      : p(p_), row_base(m0 + wm * kWaveM), lane(lane_) {
    const int col = n0 + wn * kWaveN + (lane & 7) * 8;
    rot = col < p.n_rot;
    head_col = col % p.d_head;
#pragma unroll
    for (int mt = 0; mt < kFragM; ++mt)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row = epi_row(row_base, mt, q, lane);
        pos[mt][q] = (rot && row < M) ? p.positions[row] : 0;
      }
    load_cs(0);
    load_cs(1);
    if (p.r != nullptr) rs.prefetch(p.r, row_base, lane, M);
  }

  __device__ __forceinline__ void apply(int mt, int q, int row, int col, float v[8]) {
    const float sc = p.r != nullptr ? rs.v[mt][q] : 1.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= sc;
    if (rot) {
      const f32x4 a = cs[mt & 1][q][0], b = cs[mt & 1][q][1];
      const float c[4] = {a[0], a[2], b[0], b[2]}, s[4] = {a[1], a[3], b[1], b[3]};
      const bool ok = (unsigned)pos[mt][q] < (unsigned)p.max_pos;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = v[2 * i], o = v[2 * i + 1];
        v[2 * i] = ok ? e * c[i] - o * s[i] : __builtin_nanf("");
        v[2 * i + 1] = ok ? e * s[i] + o * c[i] : __builtin_nanf("");
      }
    }
    Chunk8<T>::store(p.Y + (int64_t)row * p.ldy + col, v);
  }
  __device__ __forceinline__ void end_slab(int mt, int) {
    if (mt + 2 < kFragM) load_cs(mt + 2);
  }
  __device__ __forceinline__ void finish() {}
};

}  // namespace coda
