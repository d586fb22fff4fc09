// Epilogues of the chain's GEMMs, run on the accumulators before write-back.
//
// Building blocks (CODA news article by Synced, section
// "五种「积木」和一套「乐高语言」"): element-wise (residual add), vector load
// (the broadcast RMSNorm weight g, the per-row scale r), tile load/store (R in,
// H out), tile reduction (partial sums of squares per row).
//
// The GEMM kernel hands each lane 8 consecutive columns `col .. col+7` of one
// row through apply(mt, q, row, col, v) (mt = which of the wavefront's eight
// 16-row slabs, q = which of the lane's 2 rows in it), calls
// end_slab(mt, slab_row0) on every lane once slab mt is done, and finish() on
// every lane after the last slab.  Lanes l and l' with l/8 == l'/8 hold the
// same rows; the 8 lanes of such a group together cover the wavefront's 64
// columns, and lanes with equal l % 8 hold the same 8 columns in every slab.
//
// Epilogues that read global memory (R, H, r) issue all of a lane's loads in
// their constructor, before the first slab, so the wavefront waits for one
// memory round trip rather than one per slab (the stores of a slab could
// otherwise alias the next slab's loads, so the compiler keeps them in order).
#pragma once

#include "gemm.hpp"
#include "lanes.hpp"

namespace coda {

// Row of slot (mt, q) of `lane` in the wavefront's epilogue.
__device__ __forceinline__ int epi_row(int row_base, int mt, int q, int lane) {
  return row_base + mt * 16 + (lane >> 3) + 8 * q;
}

// Prefetched 8-column chunks of one operand for a lane's 16 epilogue rows:
// bf16 only (64 registers as stored); for fp32 (128 registers) the loads
// stay in apply().
template <typename T>
struct RowChunks {
  static constexpr bool kPrefetch = sizeof(T) == 2;
  u32x4 raw[kPrefetch ? kFragM : 1][2];
  __device__ __forceinline__ void prefetch(const T* base, int64_t ld, int row_base, int col, int lane, int M, int N) {
    if constexpr (kPrefetch) {
#pragma unroll
      for (int mt = 0; mt < kFragM; ++mt)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int row = epi_row(row_base, mt, q, lane);
          raw[mt][q] = (row < M && col < N) ? Chunk8<T>::load_raw(base + (int64_t)row * ld + col) : u32x4{0, 0, 0, 0};
        }
    }
  }
  __device__ __forceinline__ void get(const T* base, int64_t ld, int mt, int q, int row, int col, float v[8]) const {
    if constexpr (kPrefetch)
      Chunk8<T>::unpack(raw[mt][q], v);
    else
      Chunk8<T>::load(base + (int64_t)row * ld + col, v);
  }
};

// Per-row float values (r) for a lane's 16 epilogue rows.
struct RowScalars {
  float v[kFragM][2];
  __device__ __forceinline__ void prefetch(const float* p, int row_base, int lane, int M) {
#pragma unroll
    for (int mt = 0; mt < kFragM; ++mt)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row = epi_row(row_base, mt, q, lane);
        v[mt][q] = row < M ? p[row] : 0.f;
      }
  }
};

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
    int64_t hg_nck;   // > 0: Hg is tile-packed (kp_unit) with hg_nck chunks per row, bf16 only
  };
  Params p;
  RowChunks<T> rc;
  float gv[8];
  float ss[2];
  int lane, t, M;

  __device__ __forceinline__ EpiResPrms(const Params& p_, int lane_, int wm, int wn, int m0, int n0, int tn,
                                        int M_, int N)
      : p(p_), lane(lane_), t(4 * tn + wn), M(M_) {
    const int col = n0 + wn * kWaveN + (lane & 7) * 8;
    rc.prefetch(p.R, p.ldr, m0 + wm * kWaveM, col, lane, M_, N);
#pragma unroll
    for (int i = 0; i < 8; ++i) gv[i] = 1.f;
    if (p.g != nullptr && col < N) Chunk8<T>::load(p.g + col, gv);
    ss[0] = ss[1] = 0.f;
  }

  __device__ __forceinline__ void apply(int mt, int q, int row, int col, float v[8]) {
    float rv[8], h[8];
    rc.get(p.R, p.ldr, mt, q, row, col, rv);
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
      T* dst = p.Hg + (int64_t)row * p.ldhg + col;
      if constexpr (sizeof(T) == 2)
        if (p.hg_nck > 0) dst = p.Hg + kp_unit(row, col >> 3, p.hg_nck) * 8;
      Chunk8<T>::store(dst, hg);
    }
  }

  __device__ __forceinline__ void end_slab(int, int slab_row0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float s = sum8(ss[q]);
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
  RowScalars rs;
  __device__ __forceinline__ EpiRowScale(const Params& p_, int lane, int wm, int, int m0, int, int, int M, int)
      : p(p_) {
    if (p.r != nullptr) rs.prefetch(p.r, m0 + wm * kWaveM, lane, M);
  }
  __device__ __forceinline__ void apply(int mt, int q, int row, int col, float v[8]) {
    const float s = p.r != nullptr ? rs.v[mt][q] : 1.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= s;
    Chunk8<T>::store(p.Y + (int64_t)row * p.ldy + col, v);
  }
  __device__ __forceinline__ void end_slab(int, int) {}
  __device__ __forceinline__ void finish() {}
};

// Second GEMM with the SwiGLU gate (CODA news article by Synced, epilogue
// section: the re-parameterisation carries over to SwiGLU).  The B operand is
// read in the SwiGLU order (swiglu_col in tile_map.hpp): logical column col
// is a gate or an up column (swiglu_is_up) of output column
// swiglu_out_col(col) + i.  With y = r[row] * acc:
//   Y_row, gate or up column = round(y)           (only when Y is set)
//   Z_row, out = round(silu(y_gate) * y_up),  silu(x) = x / (1 + e^-x)
// Lanes l (gate) and l ^ kSwiGLUPartner (up) hold the same row and output
// columns; the up values cross over with one lane shuffle and the gate lane
// writes Z.  silu uses the hardware exp2 and reciprocal (v_exp_f32,
// v_rcp_f32, about 1 ulp each): the library expf and IEEE division would
// inline tens of instructions per value into an epilogue that runs once per
// tile and is fetched cold.  Large |x| behave: e^-x -> inf gives 0, -> 0
// gives x.
static_assert(kSwiGLUPartner == 4, "the SwiGLU epilogue pairs lanes l and l ^ 4");

template <typename T>
struct EpiSwiGLU {
  struct Params {
    const float* r;  // may be null (no row scale)
    T* Z;
    int64_t ldz;
    T* Y;            // may be null (pre-activation not kept)
    int64_t ldy;
    int F;
  };
  Params p;
  RowScalars rs;
  __device__ __forceinline__ EpiSwiGLU(const Params& p_, int lane, int wm, int, int m0, int, int, int M, int)
      : p(p_) {
    if (p.r != nullptr) rs.prefetch(p.r, m0 + wm * kWaveM, lane, M);
  }
  __device__ __forceinline__ void apply(int mt, int q, int row, int col, float v[8]) {
    const float s = p.r != nullptr ? rs.v[mt][q] : 1.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= s;
    const bool up = swiglu_is_up(col);
    const int oc = swiglu_out_col(col);
    if (p.Y != nullptr) Chunk8<T>::store(p.Y + (int64_t)row * p.ldy + (up ? p.F : 0) + oc, v);
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = lane_xor4(v[i]);  // the partner lane (kSwiGLUPartner = 4)
    if (!up) {
      float z[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float e = __builtin_amdgcn_exp2f(v[i] * -1.4426950408889634f);  // e^-x
        z[i] = v[i] * __builtin_amdgcn_rcpf(1.f + e) * o[i];
      }
      Chunk8<T>::store(p.Z + (int64_t)row * p.ldz + oc, z);
    }
  }
  __device__ __forceinline__ void end_slab(int, int) {}
  __device__ __forceinline__ void finish() {}
};

// (max, sum e^(y - max)) statistics merged: the online-normalisation state.
// An empty side is (-inf, 0); two empty sides stay empty.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;
  s = s * __builtin_amdgcn_exp2f((m - mm) * 1.4426950408889634f) +
      s2 * __builtin_amdgcn_exp2f((m2 - mm) * 1.4426950408889634f);
  m = mm;
}

// The chain's second GEMM as the LM head, ending in the cross-entropy
// statistics instead of the logits (CODA news article by Synced, sections
// "CODA：「尾声」里藏着宝藏" and "五种「积木」和一套「乐高语言」": the tile
// log-sum-exp reduction and the max / sum-exp state of online
// normalisation).  With y = r[row] * acc, never written to memory:
//   pmax[t][row] = max of y over the 64 columns of partial tile t
//   psum[t][row] = sum of e^(y - pmax) over those columns
//   tgt[row]     = y at column targets[row] (by the lane holding it)
// t = 4 * (column tile) + (column quarter), as for the partial RMS; a
// partial tile past the last column gets (-inf, 0).  Lanes reduce their 8
// columns, then the 8 lanes of a row group merge in fixed order.
template <typename T>
struct EpiLSE {
  struct Params {
    const float* r;        // [M] or null
    const int* targets;    // [M]
    float* pmax;           // [T][M]
    float* psum;           // [T][M]
    float* tgt;            // [M]
  };
  Params p;
  RowScalars rs;
  int tg[kFragM][2];
  float mx[2], sm[2];
  int lane, t, M;
  __device__ __forceinline__ EpiLSE(const Params& p_, int lane_, int wm, int wn, int m0, int, int tn, int M_, int)
      : p(p_), lane(lane_), t(4 * tn + wn), M(M_) {
    const int row_base = m0 + wm * kWaveM;
    if (p.r != nullptr) rs.prefetch(p.r, row_base, lane, M_);
#pragma unroll
    for (int mt = 0; mt < kFragM; ++mt)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row = epi_row(row_base, mt, q, lane);
        tg[mt][q] = row < M_ ? p.targets[row] : -1;
      }
    mx[0] = mx[1] = -INFINITY;
    sm[0] = sm[1] = 0.f;
  }
  __device__ __forceinline__ void apply(int mt, int q, int row, int col, float v[8]) {
    const float s = p.r != nullptr ? rs.v[mt][q] : 1.f;
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] *= s;
      m = fmaxf(m, v[i]);
    }
    float e = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) e += __builtin_amdgcn_exp2f((v[i] - m) * 1.4426950408889634f);
    mx[q] = m;
    sm[q] = e;
    const int k = tg[mt][q] - col;
    if (k >= 0 && k < 8) {
      float y = v[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) y = k == i ? v[i] : y;
      p.tgt[row] = y;
    }
  }
  __device__ __forceinline__ void end_slab(int, int slab_row0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float m = mx[q], s = sm[q];
      lse_merge(m, s, lane_xor1(m), lane_xor1(s));
      lse_merge(m, s, lane_xor2(m), lane_xor2(s));
      lse_merge(m, s, lane_xor4(m), lane_xor4(s));
      const int row = slab_row0 + (lane >> 3) + 8 * q;
      if ((lane & 7) == 0 && row < M) {
        p.pmax[(int64_t)t * M + row] = m;
        p.psum[(int64_t)t * M + row] = s;
      }
      mx[q] = -INFINITY;
      sm[q] = 0.f;
    }
  }
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
  __device__ __forceinline__ void apply(int, int, int row, int col, float v[8]) {
    Chunk8<float>::store(p.C + (int64_t)row * p.ldc + col, v);
  }
  __device__ __forceinline__ void end_slab(int, int) {}
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
  RowChunks<T> hc;
  RowScalars rs;
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
    hc.prefetch(p.H, p.ld, m0 + wm * kWaveM, col, lane, M_, N_);
    rs.prefetch(p.r, m0 + wm * kWaveM, lane, M_);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      gv[i] = 0.f;
      colsum[i] = 0.f;
    }
    if (col < N_) Chunk8<T>::load(p.g + col, gv);
    ss[0] = ss[1] = 0.f;
  }

  __device__ __forceinline__ void apply(int mt, int q, int row, int col_, float v[8]) {
    float xv[8];
    apply_p(mt, q, row, col_, v, xv);
    Chunk8<T>::store(p.Xn + (int64_t)row * p.ld + col_, xv);
  }

  // P and the sums; xv gets X_n's 8 values before their rounding to T
  __device__ __forceinline__ void apply_p(int mt, int q, int row, int col_, const float v[8], float xv[8]) {
    float hv[8], pv[8];
    hc.get(p.H, p.ld, mt, q, row, col_, hv);
    const float rr = rs.v[mt][q];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = gv[i] * v[i];
      ss[q] += pv[i] * hv[i];
      colsum[i] += (rr * hv[i]) * v[i];
      xv[i] = (hv[i] * rr) * gv[i];
    }
    Chunk8<T>::store(p.P + (int64_t)row * p.ld + col_, pv);
  }

  __device__ __forceinline__ void end_slab(int, int slab_row0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float s = sum8(ss[q]);
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
