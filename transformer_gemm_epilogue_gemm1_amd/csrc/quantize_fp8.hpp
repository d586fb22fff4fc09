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

// x / s correctly rounded wherever that decides the e4m3 code, in five
// instructions instead of a full IEEE division: Markstein's correction
// (q0 = x y, the residual r = x - q0 s exact by fma, q = q0 + r y, with y the
// correctly rounded 1 / s) on x and s rescaled by 2^-e so that s lies in
// [1/2, 1).  The residual can then underflow only where |x / s| < 2^-100,
// whose code is a zero anyway, and the sign comes from x so that -0 stays -0.
// An exhaustive host check over every bf16 x and every scale of a bf16
// maximum finds the quotient correctly rounded wherever |x / s| >= 2^-100
// and each code equal to that of the correctly rounded quotient.
struct E4m3Divider {
  float s1, y1;
  int e;
  __device__ __forceinline__ static E4m3Divider of(float s) {
    E4m3Divider d;
    d.s1 = frexpf(s, &d.e);
    d.y1 = 1.f / d.s1;
    return d;
  }
  __device__ __forceinline__ float operator()(float x) const {
    const float x1 = ldexpf(x, -e);
    const float q0 = x1 * y1;
    const float r = fmaf(-q0, s1, x1);
    return copysignf(fmaf(r, y1, q0), x);
  }
};

// The e4m3 codes of 8 values divided by one scale, and by one scale each.
__device__ __forceinline__ u32x2 encode8(const float v[8], const E4m3Divider& d) {
  return u32x2{pack_e4m3x4(d(v[0]), d(v[1]), d(v[2]), d(v[3])), pack_e4m3x4(d(v[4]), d(v[5]), d(v[6]), d(v[7]))};
}
__device__ __forceinline__ u32x2 encode8(const float v[8], const E4m3Divider (&d)[8]) {
  return u32x2{pack_e4m3x4(d[0](v[0]), d[1](v[1]), d[2](v[2]), d[3](v[3])),
               pack_e4m3x4(d[4](v[4]), d[5](v[5]), d[6](v[6]), d[7](v[7]))};
}

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
// K % 8 == 0.  Rows of up to 2048 CPT elements stay in registers (CPT
// 16-byte chunks per thread, all loads in flight at once), so the row is read
// from memory once.
// Where the 8 row codes of columns col .. col + 7 (col a multiple of 8) of
// row `row` go: row-major with leading dimension ldx8, or, for x8_nck > 0,
// tile-packed with x8_nck 16-code units per row (kp_unit).
__device__ __forceinline__ uint8_t* row_codes(uint8_t* X8, int64_t ldx8, int64_t x8_nck, int64_t row, int col) {
  return x8_nck > 0 ? X8 + kp_unit(row, col >> 4, x8_nck) * 16 + (col & 15) : X8 + row * ldx8 + col;
}

template <int CPT>
__global__ __launch_bounds__(256) void quantize_rows_e4m3_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                                 int K, uint8_t* __restrict__ X8, int64_t ldx8,
                                                                 float* __restrict__ scales, int64_t x8_nck) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const uint16_t* x = X + row * ldx;
  const int nc = K / 8;
  u32x4 raw[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = threadIdx.x + 256 * j;
    raw[j] = c < nc ? Chunk8<uint16_t>::load_raw(x + 8 * c) : u32x4{0, 0, 0, 0};
  }
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    float v[8];
    Chunk8<uint16_t>::unpack(raw[j], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  const float s = e4m3_scale(block_amax(m, red));
  if (threadIdx.x == 0) scales[row] = s;
  const E4m3Divider enc = E4m3Divider::of(s);
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = threadIdx.x + 256 * j;
    if (c < nc) {
      float v[8];
      Chunk8<uint16_t>::unpack(raw[j], v);
      *(u32x2*)row_codes(X8, ldx8, x8_nck, row, 8 * c) = encode8(v, enc);
    }
  }
}

// The row quantisation with the codes tile-packed (kp_unit, nck = K / 16
// units per row), laid out for that layout's stores; the same scales and
// codes as quantize_rows_e4m3_kernel.  In the packed layout the 16-code units
// of one row lie 256 bytes apart and the 16 rows of a unit column are
// contiguous, so a workgroup takes 4 rows: lane l of wavefront w holds row
// 4 blockIdx.x + (l & 3) and its units u = 16 (UPL w + j) + (l >> 2),
// j < UPL (two 16-byte loads of bf16 each, 512 contiguous bytes per row and
// instruction pair).  Each store instruction then writes 4 rows of 16 unit
// columns, 64 contiguous bytes each.  The row maximum reduces over the 16
// lanes of a row, then over the 4 wavefronts through LDS.  K <= 1024 UPL;
// the launcher takes it up to K = 8192 (UPL = 8, 160 VGPRs), longer rows
// take the one-row kernels.
template <int UPL>
__global__ __launch_bounds__(256) void quantize_rows_packed_e4m3_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                                        int M, int K, uint8_t* __restrict__ X8,
                                                                        float* __restrict__ scales, int64_t nck) {
  __shared__ float red[4][4];
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t row = 4 * (int64_t)blockIdx.x + (l & 3);
  const int q = l >> 2, nu = K / 16;
  const bool rin = row < M;
  const uint16_t* x = X + (rin ? row : 0) * ldx;
  u32x4 raw[UPL][2];
#pragma unroll
  for (int j = 0; j < UPL; ++j) {
    const int u = 16 * (UPL * w + j) + q;
    const bool in = rin && u < nu;
#pragma unroll
    for (int h = 0; h < 2; ++h) raw[j][h] = in ? Chunk8<uint16_t>::load_raw(x + 16 * u + 8 * h) : u32x4{0, 0, 0, 0};
  }
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < UPL; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float v[8];
      Chunk8<uint16_t>::unpack(raw[j][h], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    }
#pragma unroll
  for (int d = 4; d < 64; d *= 2) m = fmaxf(m, __shfl_xor(m, d));
  if (q == 0) red[w][l & 3] = m;
  __syncthreads();
  const int r = l & 3;
  const float s = e4m3_scale(fmaxf(fmaxf(red[0][r], red[1][r]), fmaxf(red[2][r], red[3][r])));
  if (w == 0 && q == 0 && rin) scales[row] = s;
  const E4m3Divider enc = E4m3Divider::of(s);
#pragma unroll
  for (int j = 0; j < UPL; ++j) {
    const int u = 16 * (UPL * w + j) + q;
    if (rin && u < nu) {
      float v0[8], v1[8];
      Chunk8<uint16_t>::unpack(raw[j][0], v0);
      Chunk8<uint16_t>::unpack(raw[j][1], v1);
      const u32x2 lo = encode8(v0, enc), hi = encode8(v1, enc);
      *(u32x4*)(X8 + kp_unit(row, u, nck) * 16) = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  }
}

// Rows longer than 32768 elements: the same result in two passes over the
// row, the second from cache.
__global__ __launch_bounds__(256) void quantize_long_rows_e4m3_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                                      int K, uint8_t* __restrict__ X8,
                                                                      int64_t ldx8, float* __restrict__ scales,
                                                                      int64_t x8_nck) {
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
  const E4m3Divider enc = E4m3Divider::of(s);
  for (int c = threadIdx.x; c < nc; c += 256) {
    float v[8];
    Chunk8<uint16_t>::load(x + 8 * c, v);
    *(u32x2*)row_codes(X8, ldx8, x8_nck, row, 8 * c) = encode8(v, enc);
  }
}

// Column-wise quantisation of W [K, N] (bf16, N contiguous) into the codes
// of W^T, Wt8 [N, K] (K contiguous), one scale per column, in three steps
// that keep every CU busy for tall matrices (activations of 16k rows as
// well as weights):
//   1. colmax_kernel (or rowcol_max_kernel, which also takes the row maxima):
//      the block maxima are folded into amax (the scales array, zeroed
//      first) with atomic max on the float bits (non-negative floats order
//      like their bits; the result does not depend on the order);
//   2. quantize_cols_kernel: each workgroup encodes a 128 x 128 block with
//      the scales of its columns and writes the codes transposed (through an
//      LDS byte tile), and optionally the row codes of the same block with
//      the row scales;
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

// Row and column maxima of X [M, N] in one pass (for an activation that is
// quantised both ways): each workgroup takes a 256 x 256 block, thread t the
// 8 columns 8 * (t % 32) .. +7 of rows t / 32 + 8 i, and folds the block's
// row maxima into rmax and its column maxima into cmax (both zeroed first).
__global__ __launch_bounds__(256) void rowcol_max_kernel(const uint16_t* __restrict__ X, int64_t ldx, int M, int N,
                                                         uint32_t* __restrict__ rmax, uint32_t* __restrict__ cmax) {
  __shared__ float rpart[256][33];  // [row of the block][column chunk]
  __shared__ float cpart[8][257];   // [row group][column of the block]
  const int t = threadIdx.x, cc = t & 31, rg = t >> 5;
  const int n0 = blockIdx.x * 256, m0 = blockIdx.y * 256;
  const int col = n0 + 8 * cc;
  float cm[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) cm[e] = 0.f;
  for (int i0 = 0; i0 < 32; i0 += 8) {
    u32x4 raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = m0 + rg + 8 * (i0 + i);
      raw[i] = (col < N && row < M) ? Chunk8<uint16_t>::load_raw(X + (int64_t)row * ldx + col) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v[8];
      Chunk8<uint16_t>::unpack(raw[i], v);
      float rm = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float a = fabsf(v[e]);
        rm = fmaxf(rm, a);
        cm[e] = fmaxf(cm[e], a);
      }
      rpart[rg + 8 * (i0 + i)][cc] = rm;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) cpart[rg][8 * cc + e] = cm[e];
  __syncthreads();
  // thread t: row m0 + t and column n0 + t of the block
  float rmx = 0.f, cmx = 0.f;
  for (int j = 0; j < 32; ++j) rmx = fmaxf(rmx, rpart[t][j]);
  for (int j = 0; j < 8; ++j) cmx = fmaxf(cmx, cpart[j][t]);
  if (m0 + t < M) atomicMax(rmax + m0 + t, __float_as_uint(rmx));
  if (n0 + t < N) atomicMax(cmax + n0 + t, __float_as_uint(cmx));
}

// Codes of one 4 x 4 byte block transposed: w[i] holds row i's codes of 4
// columns; out[j] gets column j's codes of the 4 rows.
__device__ __forceinline__ void transpose4x4_bytes(const uint32_t w[4], uint32_t out[4]) {
  // v_perm_b32 picks bytes of {hi: src0, lo: src1} by the selector's bytes
  const uint32_t x01 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);  // w0.b0 w1.b0 w0.b1 w1.b1
  const uint32_t y01 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);  // w2.b0 w3.b0 w2.b1 w3.b1
  const uint32_t x23 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);  // w0.b2 w1.b2 w0.b3 w1.b3
  const uint32_t y23 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(y01, x01, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(y01, x01, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(y23, x23, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(y23, x23, 0x07060302u);
}

// A 128 x 128 block per workgroup.  Thread t reads columns 8 * (t % 16) .. +7
// of block rows t / 16 + 16 h, writes those rows' codes (when X8 is set) and
// puts the column codes into an LDS byte tile; it then writes output rows
// 4 (t / 8) .. +3, 16 codes each at k offset 16 * (t % 8), transposing 4 x 4
// byte blocks in registers.  Every code row a block writes is one 128-byte
// line.
__global__ __launch_bounds__(256) void quantize_cols_kernel(const uint16_t* __restrict__ W, int64_t ldw, int K,
                                                            int N, const uint32_t* __restrict__ amax,
                                                            uint8_t* __restrict__ Wt8, int64_t ldwt,
                                                            const uint32_t* __restrict__ rmax,
                                                            uint8_t* __restrict__ X8, int64_t ldx8,
                                                            int64_t wt_nck, int64_t x8_nck) {
  constexpr int kPitch = 33;  // words per tile row: 128 codes + 4 bytes of padding
  __shared__ uint32_t tile[128 * kPitch];
  __shared__ E4m3Divider coldiv[128], rowdiv[128];
  const int t = threadIdx.x;
  const int n0 = blockIdx.x * 128, k0 = blockIdx.y * 128;
  if (t < 128)
    coldiv[t] = E4m3Divider::of(e4m3_scale(n0 + t < N ? __uint_as_float(amax[n0 + t]) : 0.f));
  else if (X8 != nullptr)
    rowdiv[t - 128] = E4m3Divider::of(e4m3_scale(k0 + t - 128 < K ? __uint_as_float(rmax[k0 + t - 128]) : 0.f));
  const int rc = (t & 15) * 8;
  const bool cin = n0 + rc < N;
  u32x4 raw[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const int k = k0 + (t >> 4) + 16 * h;
    raw[h] = (k < K && cin) ? Chunk8<uint16_t>::load_raw(W + (int64_t)k * ldw + n0 + rc) : u32x4{0, 0, 0, 0};
  }
  __syncthreads();
  E4m3Divider cd[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) cd[i] = coldiv[rc + i];
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const int kr = (t >> 4) + 16 * h, k = k0 + kr;
    float v[8];
    Chunk8<uint16_t>::unpack(raw[h], v);
    if (X8 != nullptr && k < K && cin) *(u32x2*)row_codes(X8, ldx8, x8_nck, k, n0 + rc) = encode8(v, rowdiv[kr]);
    const u32x2 c = encode8(v, cd);
    tile[kr * kPitch + rc / 4] = c[0];
    tile[kr * kPitch + rc / 4 + 1] = c[1];
  }
  __syncthreads();
  const int cg = t >> 3, kc = (t & 7) * 16;  // output rows 4 cg .. +3, codes kc .. kc + 15
  if (n0 + 4 * cg < N && k0 + kc < K) {
    uint32_t out[4][4];  // [output row][word]
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t w[4], o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = tile[(kc + 4 * g + i) * kPitch + cg];
      transpose4x4_bytes(w, o);
#pragma unroll
      for (int j = 0; j < 4; ++j) out[j][g] = o[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // wt_nck > 0: Wt8 tile-packed (kp_unit), 16 codes = one 16-byte unit
      uint8_t* dst = wt_nck > 0 ? Wt8 + kp_unit(n0 + 4 * cg + j, (k0 + kc) >> 4, wt_nck) * 16
                                : Wt8 + (int64_t)(n0 + 4 * cg + j) * ldwt + k0 + kc;
      *(u32x4*)dst = u32x4{out[j][0], out[j][1], out[j][2], out[j][3]};
    }
  }
}

__global__ __launch_bounds__(256) void amax_to_scale_kernel(float* __restrict__ scales, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) scales[i] = e4m3_scale(scales[i]);
}

// ---- MX quantisation (OCP microscaling: one E8M0 exponent per 32 elements) --
//
// X [M, N] (bf16) quantised along its rows and/or along its columns, each
// 32-element block with its own exponent (mx_exponent of the block's largest
// float32 magnitude, as the first fp8 GEMM's epilogue takes it) and the codes
// e4m3(x 2^-E):
//   ROWS: Xr8 [M, N] tile-packed (kp_unit, N / 16 units per row), exponents
//         Er per row and block of 32 columns (mx_byte layout, rows M, cols N);
//   COLS: the codes of X^T, Xc8 [N, M] tile-packed (M / 16 units per row),
//         exponents Ec per column of X and block of 32 rows (rows N, cols M).
// One read of X serves both.  A workgroup takes 32 rows x 256 columns; thread
// t holds row t / 8's 32 columns 32 (t % 8) .. +31, the block of its row
// codes.  For the column codes the tile goes through LDS, where thread t
// then reads column t: element (r, 32 b + k) sits at word
// r * kMxPitch + 32 b + (k + 4 b) % 32, which spreads both the writes of a
// row's 8 blocks and the reads of 64 consecutive columns over the banks.
// Each workgroup takes kMxHalves such 32-row tiles in turn, with the loads of
// all of them in flight first.  The grid covers 256 ceil(M / 256) rows and
// 256 ceil(N / 256) columns, so
// that every exponent byte of both arrays is written, those of padding rows
// and of blocks past the end as 127 (E = 0, their values read as 0); codes
// are written only inside X.  M % 16 == 0, N % 16 == 0.
constexpr int kMxPitch = 257;

template <bool ROWS, bool COLS>
__device__ __forceinline__ void mx_quantize_tile(const float (&v)[32], int i0, int j0, int M, int N,
                                                 uint8_t* __restrict__ Xr8, uint8_t* __restrict__ Er,
                                                 uint8_t* __restrict__ Xc8, uint8_t* __restrict__ Ec, float* tile) {
  const int t = threadIdx.x;
  const int rr = t >> 3, cb = t & 7;
  const int row = i0 + rr, col = j0 + 32 * cb;
  if constexpr (ROWS) {
    float a = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) a = fmaxf(a, fabsf(v[k]));
    const int E = mx_exponent(a);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (row < M && col + 16 * h < N) {
        const float* x = v + 16 * h;
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = pack_e4m3x4(ldexpf(x[4 * q], -E), ldexpf(x[4 * q + 1], -E), ldexpf(x[4 * q + 2], -E),
                             ldexpf(x[4 * q + 3], -E));
        *(u32x4*)(Xr8 + kp_unit(row, (col >> 4) + h, N >> 4) * 16) = w;
      }
    }
    if (row < 128 * mx_row_blocks(M)) Er[mx_byte(row, col >> 6, (col >> 5) & 1, M)] = (uint8_t)(E + 127);
  }
  if constexpr (COLS) {
    __syncthreads();  // the tile's previous reads are done
#pragma unroll
    for (int k = 0; k < 32; ++k) tile[rr * kMxPitch + 32 * cb + ((k + 4 * cb) & 31)] = v[k];
    __syncthreads();
    const int pc = 32 * (t >> 5) + (((t & 31) + 4 * (t >> 5)) & 31);
    float w[32];
    float a = 0.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      w[r] = tile[r * kMxPitch + pc];
      a = fmaxf(a, fabsf(w[r]));
    }
    const int E = mx_exponent(a);
    const int crow = j0 + t;  // the row of X^T
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (crow < N && i0 + 16 * h < M) {
        const float* x = w + 16 * h;
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o[q] = pack_e4m3x4(ldexpf(x[4 * q], -E), ldexpf(x[4 * q + 1], -E), ldexpf(x[4 * q + 2], -E),
                             ldexpf(x[4 * q + 3], -E));
        *(u32x4*)(Xc8 + kp_unit(crow, (i0 >> 4) + h, M >> 4) * 16) = o;
      }
    }
    if (crow < 128 * mx_row_blocks(N)) Ec[mx_byte(crow, i0 >> 6, (i0 >> 5) & 1, N)] = (uint8_t)(E + 127);
  }
}

// A workgroup takes kMxTileRows = 32 kMxHalves rows as kMxHalves 32-row
// tiles, all of whose loads go out first.
constexpr int kMxHalves = 2, kMxTileRows = 32 * kMxHalves;

template <bool ROWS, bool COLS>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const uint16_t* __restrict__ X, int64_t ldx, int M, int N,
                                                          uint8_t* __restrict__ Xr8, uint8_t* __restrict__ Er,
                                                          uint8_t* __restrict__ Xc8, uint8_t* __restrict__ Ec) {
  __shared__ float tile[COLS ? 32 * kMxPitch : 1];
  const int t = threadIdx.x;
  const int j0 = blockIdx.y * 256;  // row tiles along x: the longer grid dimension
  const int rr = t >> 3, cb = t & 7;
  const int col = j0 + 32 * cb;
  float v[kMxHalves][32];
#pragma unroll
  for (int u = 0; u < kMxHalves; ++u) {
    const int row = blockIdx.x * kMxTileRows + 32 * u + rr;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool in = row < M && col + 8 * c < N;
      const u32x4 raw = in ? Chunk8<uint16_t>::load_raw(X + (int64_t)row * ldx + col + 8 * c) : u32x4{0, 0, 0, 0};
      Chunk8<uint16_t>::unpack(raw, v[u] + 8 * c);
    }
  }
#pragma unroll
  for (int u = 0; u < kMxHalves; ++u)
    mx_quantize_tile<ROWS, COLS>(v[u], blockIdx.x * kMxTileRows + 32 * u, j0, M, N, Xr8, Er, Xc8, Ec, tile);
}

}  // namespace coda
