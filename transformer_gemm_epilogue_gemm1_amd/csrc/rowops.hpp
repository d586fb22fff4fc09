// Small row-wise kernels: the combine of the partial sums of squares, the
// unfused chain's residual-add and RMSNorm passes, and the backward's combine
// and dH passes.
#pragma once

#include "gemm.hpp"

namespace coda {

// Fixed-order sum of parts[t * stride + i], t = 0 .. T-1, for the 64
// indices i = i0 .. i0+63 of a 256-thread workgroup: wavefront q sums its
// quarter of t in increasing order, then the quarters are added as
// ((q0 + q1) + q2) + q3.  Lane l of every wavefront gets the sum for i0 + l.
// Each load of a wavefront reads 64 consecutive floats.
__device__ __forceinline__ float quarter_sum(const float* __restrict__ parts, int64_t stride, int T, int i, bool in,
                                             float (*red)[64]) {
  const int q = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tq = (T + 3) / 4;
  const int t0 = q * tq, t1 = t0 + tq < T ? t0 + tq : T;
  float s = 0.f;
  if (in) {
#pragma unroll 8
    for (int t = t0; t < t1; ++t) s += parts[(int64_t)t * stride + i];
  }
  red[q][lane] = s;
  __syncthreads();
  return ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

// r_i = 1/sqrt(mean_j H_ij^2 + eps) from the per-tile partial sums of squares
// (the light auxiliary reduction of the CODA news article by Synced, section
// "CODA：「尾声」里藏着宝藏").  64 rows per 256-thread workgroup, partials
// [T][M] summed in the fixed order of quarter_sum (deterministic); the mean
// and reciprocal square root are taken in double precision and rounded once.
__global__ __launch_bounds__(256) void rms_combine_kernel(const float* __restrict__ partials,
                                                          float* __restrict__ r, int M, int T, int D,
                                                          float eps) {
  __shared__ float red[4][64];
  const int i = blockIdx.x * 64 + (threadIdx.x & 63);
  const float s = quarter_sum(partials, M, T, i, i < M, red);
  if (threadIdx.x < 64 && i < M) r[i] = (float)(1.0 / sqrt((double)s / (double)D + (double)eps));
}

// Unfused chain, step 2: H = round(C + R), elementwise over dense [M, D].
template <typename T>
__global__ __launch_bounds__(256) void residual_add_kernel(const float* __restrict__ C, const T* __restrict__ R,
                                                           T* __restrict__ H, int64_t nchunks) {
  for (int64_t c = blockIdx.x * 256ll + threadIdx.x; c < nchunks; c += (int64_t)gridDim.x * 256) {
    float cv[8], rv[8];
    Chunk8<float>::load(C + c * 8, cv);
    Chunk8<T>::load(R + c * 8, rv);
#pragma unroll
    for (int i = 0; i < 8; ++i) cv[i] = cv[i] + rv[i];
    Chunk8<T>::store(H + c * 8, cv);
  }
}

// Unfused chain, step 3: standalone RMSNorm over dense [M, D], one workgroup
// per row: r = 1/sqrt(mean(H^2) + eps), X_n = round(float(H) * r * g).
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const T* __restrict__ H, const T* __restrict__ g,
                                                           float* __restrict__ r, T* __restrict__ Xn, int D,
                                                           float eps) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const T* h = H + row * D;
  const int nch = D / 8;
  float s = 0.f;
  for (int c = threadIdx.x; c < nch; c += 256) {
    float v[8];
    Chunk8<T>::load(h + c * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[i] * v[i];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float rr = (float)(1.0 / sqrt((double)tot / (double)D + (double)eps));
  if (threadIdx.x == 0) r[row] = rr;
  for (int c = threadIdx.x; c < nch; c += 256) {
    float v[8], gv[8];
    Chunk8<T>::load(h + c * 8, v);
    Chunk8<T>::load(g + c * 8, gv);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (v[i] * rr) * gv[i];
    Chunk8<T>::store(Xn + row * D + c * 8, v);
  }
}

// Backward combine.  Workgroups 0 .. ceil(M/64)-1 take 64 rows each:
//   c_i = r_i^3 * (sum_t srow[t][i]) / D
// (the coefficient of H_i in dH_i; the product in double, rounded once);
// the following ceil(D/64) workgroups take 64 columns each:
//   dg_j = sum_u dgcol[u][j], u = 0 .. U-1.
// Both sums in the fixed order of quarter_sum.
__global__ __launch_bounds__(256) void bwd_combine_kernel(const float* __restrict__ srow,
                                                          const float* __restrict__ dgcol,
                                                          const float* __restrict__ r, float* __restrict__ c,
                                                          float* __restrict__ dg, int M, int T, int D, int U) {
  __shared__ float red[4][64];
  const int row_blocks = (M + 63) / 64;
  const int lane = threadIdx.x & 63;
  if ((int)blockIdx.x < row_blocks) {
    const int i = blockIdx.x * 64 + lane;
    const float s = quarter_sum(srow, M, T, i, i < M, red);
    if (threadIdx.x < 64 && i < M) {
      const double rr = (double)r[i];
      c[i] = (float)(rr * rr * rr * (double)s / (double)D);
    }
  } else {
    const int j = (blockIdx.x - row_blocks) * 64 + lane;
    const float s = quarter_sum(dgcol, D, U, j, j < D, red);
    if (threadIdx.x < 64 && j < D) dg[j] = s;
  }
}

// Backward dH, in place over dense [M, D]: the buffer holds P = round(g G) on
// entry and dH = round(r_i float(P_ij) - c_i float(H_ij)) on exit.
template <typename T>
__global__ __launch_bounds__(256) void dh_finalize_kernel(T* __restrict__ PdH, const T* __restrict__ H,
                                                          const float* __restrict__ r,
                                                          const float* __restrict__ c, int D, int64_t nchunks) {
  const int cpr = D / 8;  // chunks per row
  for (int64_t k = blockIdx.x * 256ll + threadIdx.x; k < nchunks; k += (int64_t)gridDim.x * 256) {
    const int64_t row = k / cpr;
    float pv[8], hv[8];
    Chunk8<T>::load(PdH + k * 8, pv);
    Chunk8<T>::load(H + k * 8, hv);
    const float rr = r[row], cc = c[row];
#pragma unroll
    for (int i = 0; i < 8; ++i) pv[i] = rr * pv[i] - cc * hv[i];
    Chunk8<T>::store(PdH + k * 8, pv);
  }
}

// SwiGLU backward through the gate, elementwise over [M, F]: with
// Z = silu(Y_gate) * Y_up, s = sigmoid(Y_gate),
//   dY_gate = dZ * Y_up * s (1 + Y_gate (1 - s))
//   dY_up   = dZ * Y_gate * s
// One thread per 8-column chunk; dY[:, :F] and dY[:, F:] written side by side
// as the [M, 2F] gradient of the second GEMM's output.
template <typename T>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const T* __restrict__ dZ, int64_t ldz,
                                                         const T* __restrict__ Y, int64_t ldy, T* __restrict__ dY,
                                                         int64_t lddy, int F, int64_t nchunks) {
  const int cpr = F / 8;
  for (int64_t k = blockIdx.x * 256ll + threadIdx.x; k < nchunks; k += (int64_t)gridDim.x * 256) {
    const int64_t row = k / cpr;
    const int col = (int)(k - row * cpr) * 8;
    float dz[8], yg[8], yu[8], dg[8], du[8];
    Chunk8<T>::load(dZ + row * ldz + col, dz);
    Chunk8<T>::load(Y + row * ldy + col, yg);
    Chunk8<T>::load(Y + row * ldy + F + col, yu);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sg = 1.f / (1.f + expf(-yg[i]));
      dg[i] = dz[i] * yu[i] * (sg * (1.f + yg[i] * (1.f - sg)));
      du[i] = dz[i] * (yg[i] * sg);
    }
    Chunk8<T>::store(dY + row * lddy + col, dg);
    Chunk8<T>::store(dY + row * lddy + F + col, du);
  }
}

// Cross-entropy combine, 64 rows per 256-thread workgroup: wavefront q
// merges the (max, sum-exp) statistics of its quarter of the T partial tiles
// in increasing t, then the quarters are merged first to last (fixed order):
//   lse_i  = M_i + log(sum_t psum[t][i] e^(pmax[t][i] - M_i)),  M_i = max_t pmax
//   loss_i = lse_i - tgt[i], or NaN when targets[i] is outside [0, V).
__global__ __launch_bounds__(256) void ce_combine_kernel(const float* __restrict__ pmax,
                                                         const float* __restrict__ psum,
                                                         const float* __restrict__ tgt,
                                                         const int* __restrict__ targets, float* __restrict__ lse,
                                                         float* __restrict__ loss, int M, int T, int V) {
  __shared__ float red_m[4][64], red_s[4][64];
  const int q = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 64 + lane;
  const int tq = (T + 3) / 4;
  const int t0 = q * tq, t1 = t0 + tq < T ? t0 + tq : T;
  float m = -INFINITY, s = 0.f;
  if (i < M) {
    for (int t = t0; t < t1; ++t) {
      const float pm = pmax[(int64_t)t * M + i], ps = psum[(int64_t)t * M + i];
      const float mm = fmaxf(m, pm);
      if (mm != -INFINITY) {
        s = s * expf(m - mm) + ps * expf(pm - mm);
        m = mm;
      }
    }
  }
  red_m[q][lane] = m;
  red_s[q][lane] = s;
  __syncthreads();
  if (q == 0 && i < M) {
    for (int k = 1; k < 4; ++k) {
      const float pm = red_m[k][lane], ps = red_s[k][lane];
      const float mm = fmaxf(m, pm);
      if (mm != -INFINITY) {
        s = s * expf(m - mm) + ps * expf(pm - mm);
        m = mm;
      }
    }
    const float l = m + logf(s);
    lse[i] = l;
    const int ti = targets[i];
    loss[i] = (ti >= 0 && ti < V) ? l - tgt[i] : __builtin_nanf("");
  }
}

// Table of the rotary embedding: cos_sin[p][i] = (cos(p theta_i), sin(p theta_i))
// with theta_i = base^(-2i / d_head), i < half = d_head / 2, evaluated in
// double precision and stored as float.  One thread per entry.
__global__ __launch_bounds__(256) void rope_cache_kernel(float* __restrict__ cs, int64_t n, int half, double base) {
  const int64_t k = blockIdx.x * 256ll + threadIdx.x;
  if (k >= n) return;
  const int64_t p = k / half;
  const int i = (int)(k - p * half);
  const double theta = pow(base, -(double)i / (double)half);
  double sn, cn;
  sincos((double)p * theta, &sn, &cn);
  *(float2*)(cs + 2 * k) = float2{(float)cn, (float)sn};
}

// Gradient through the rotary embedding: the rotation is orthogonal, so the
// gradient of the unrotated values is the incoming gradient turned back,
//   dY_2i = g_2i c_i + g_2i+1 s_i,  dY_2i+1 = -g_2i s_i + g_2i+1 c_i,
// in the rotated columns [0, n_rot) (NaN for a position outside
// [0, max_pos)), copied in the others.  One thread per 8-column chunk.
template <typename T>
__global__ __launch_bounds__(256) void rope_bwd_kernel(const T* __restrict__ dYr, int64_t ldg,
                                                       const int* __restrict__ positions,
                                                       const float* __restrict__ cos_sin, int max_pos, int n_rot,
                                                       int d_head, T* __restrict__ dY, int64_t lddy, int N,
                                                       int64_t nchunks) {
  const int cpr = N / 8;
  for (int64_t k = blockIdx.x * 256ll + threadIdx.x; k < nchunks; k += (int64_t)gridDim.x * 256) {
    const int64_t row = k / cpr;
    const int col = (int)(k - row * cpr) * 8;
    float gv[8];
    Chunk8<T>::load(dYr + row * ldg + col, gv);
    if (col < n_rot) {
      const int pp = positions[row];
      if ((unsigned)pp < (unsigned)max_pos) {
        const float* t = cos_sin + (int64_t)pp * d_head + col % d_head;
        const f32x4 a = *(const f32x4*)t, b = *(const f32x4*)(t + 4);
        const float c[4] = {a[0], a[2], b[0], b[2]}, s[4] = {a[1], a[3], b[1], b[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = gv[2 * i], o = gv[2 * i + 1];
          gv[2 * i] = e * c[i] + o * s[i];
          gv[2 * i + 1] = o * c[i] - e * s[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) gv[i] = __builtin_nanf("");
      }
    }
    Chunk8<T>::store(dY + row * lddy + col, gv);
  }
}

// Y = X^T for X [R, C] (row-major, ldx) into Y [C, R] (ldy), bit-exact,
// through 64 x 64 tiles in LDS.  Thread t loads 8-element chunk t % 8 of tile
// rows t / 8 and t / 8 + 32, and stores the two 8-element chunks of output
// row t / 4 at offsets 16 (t % 4) and 16 (t % 4) + 8.  R % 8 == 0, C % 8 == 0.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ X, int64_t ldx, int R, int C,
                                                        T* __restrict__ Y, int64_t ldy) {
  __shared__ float tile[64][65];
  const int t = threadIdx.x;
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int cc = (t & 7) * 8;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rr = (t >> 3) + 32 * h;
    if (r0 + rr < R && c0 + cc < C) {
      float v[8];
      Chunk8<T>::load(X + (int64_t)(r0 + rr) * ldx + c0 + cc, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) tile[rr][cc + i] = v[i];
    }
  }
  __syncthreads();
  const int j = t >> 2;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i0 = (t & 3) * 16 + 8 * h;
    if (c0 + j < C && r0 + i0 < R) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = tile[i0 + i][j];
      Chunk8<T>::store(Y + (int64_t)(c0 + j) * ldy + r0 + i0, v);
    }
  }
}

}  // namespace coda
