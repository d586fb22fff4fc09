// Quantisation of bf16 operands to e4m3 codes with float32 scales, the
// recipe of the fp8 chain: the largest magnitude of a row (activations) or of
// an output channel (weights, stored transposed) maps to 448,
//   scale = amax / 448 (1 for an all-zero vector),
//   code  = e4m3_rne(clamp(x / scale, +-448)),
// the division correctly rounded in float32.  Inputs are finite.
#pragma once

#include "epilogues_fp8.hpp"

namespace coda {

__device__ __forceinline__ float e4m3_scale(float amax) { return amax > 0.f ? amax / 448.f : 1.f; }

// Largest magnitude over a 256-thread workgroup (wavefront shuffles, then
// the four wavefronts through LDS); every thread gets the result.
__device__ __forceinline__ float block_amax(float v, float* red) {
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) v = fmaxf(v, __shfl_xor(v, x));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return m;
}

// One workgroup per row of X [M, K] (bf16): scales[row] and the row's codes.
// K % 8 == 0; each thread takes 8-element chunks, the second pass reads the
// row again (from cache).
__global__ __launch_bounds__(256) void quantize_rows_e4m3_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                                 int K, uint8_t* __restrict__ X8, int64_t ldx8,
                                                                 float* __restrict__ scales) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const uint16_t* x = X + row * ldx;
  const int nc = K / 8;
  float m = 0.f;
  for (int c = threadIdx.x; c < nc; c += 256) {
    float v[8];
    Chunk8<uint16_t>::load(x + 8 * c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  const float s = e4m3_scale(block_amax(m, red));
  if (threadIdx.x == 0) scales[row] = s;
  uint8_t* y = X8 + row * ldx8;
  for (int c = threadIdx.x; c < nc; c += 256) {
    float v[8];
    Chunk8<uint16_t>::load(x + 8 * c, v);
    const uint32_t lo = pack_e4m3x4(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
    const uint32_t hi = pack_e4m3x4(v[4] / s, v[5] / s, v[6] / s, v[7] / s);
    *(u32x2*)(y + 8 * c) = u32x2{lo, hi};
  }
}

// Column-wise quantisation of W [K, N] (bf16, N contiguous) into the codes
// of W^T, Wt8 [N, K] (K contiguous), one scale per column, in three steps
// that keep every CU busy for tall matrices (activations of 16k rows as
// well as weights):
//   1. colmax_kernel: each workgroup takes a 64-column x 256-row block and
//      folds its column maxima into amax (the scales array, zeroed first) with
//      atomic max on the float bits (non-negative floats order like their
//      bits; the result does not depend on the order);
//   2. quantize_cols_kernel: each workgroup encodes a 64 x 64 block through
//      LDS, transposed, with the scales of its columns;
//   3. amax_to_scale_kernel turns the maxima into the scales in place.
// K % 16 == 0, N % 16 == 0; columns past N and rows past K are neither read
// nor written.
__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, int n, uint32_t v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// Thread t: the 8 columns 8 * (t % 8) .. +7 of the block's rows t / 8 + 32 j.
__global__ __launch_bounds__(256) void colmax_kernel(const uint16_t* __restrict__ W, int64_t ldw, int K, int N,
                                                     uint32_t* __restrict__ amax) {
  __shared__ float part[32][65];
  const int t = threadIdx.x;
  const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 256;
  const int c8 = (t & 7) * 8;
  float m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) m[i] = 0.f;
  if (n0 + c8 < N) {
    const int k1 = k0 + 256 < K ? k0 + 256 : K;
    for (int k = k0 + (t >> 3); k < k1; k += 32) {
      float v[8];
      Chunk8<uint16_t>::load(W + (int64_t)k * ldw + n0 + c8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(v[i]));
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[t >> 3][c8 + i] = m[i];
  __syncthreads();
  if (t < 64 && n0 + t < N) {
    float mx = 0.f;
    for (int j = 0; j < 32; ++j) mx = fmaxf(mx, part[j][t]);
    atomicMax(amax + n0 + t, __float_as_uint(mx));
  }
}

// Thread t reads columns 8 * (t % 8) .. +7 of block rows t / 8 and t / 8 + 32,
// and writes 16 codes of output row t / 4 at k offset 16 * (t % 4).
__global__ __launch_bounds__(256) void quantize_cols_kernel(const uint16_t* __restrict__ W, int64_t ldw, int K,
                                                            int N, const uint32_t* __restrict__ amax,
                                                            uint8_t* __restrict__ Wt8, int64_t ldwt) {
  __shared__ float tile[64][65];
  __shared__ float colscale[64];
  const int t = threadIdx.x;
  const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  if (t < 64) colscale[t] = e4m3_scale(n0 + t < N ? __uint_as_float(amax[n0 + t]) : 0.f);
  __syncthreads();
  const int rc = (t & 7) * 8;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kr = (t >> 3) + 32 * h, k = k0 + kr;
    float v[8];
    if (k < K && n0 + rc < N) {
      Chunk8<uint16_t>::load(W + (int64_t)k * ldw + n0 + rc, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[kr][rc + i] = v[i] / colscale[rc + i];
  }
  __syncthreads();
  const int wr = t >> 2, wk = (t & 3) * 16;
  if (n0 + wr < N && k0 + wk < K) {
    float q[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = tile[wk + i][wr];
    u32x4 out;
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = pack_e4m3x4(q[4 * j], q[4 * j + 1], q[4 * j + 2], q[4 * j + 3]);
    *(u32x4*)(Wt8 + (int64_t)(n0 + wr) * ldwt + k0 + wk) = out;
  }
}

__global__ __launch_bounds__(256) void amax_to_scale_kernel(float* __restrict__ scales, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) scales[i] = e4m3_scale(scales[i]);
}

}  // namespace coda
