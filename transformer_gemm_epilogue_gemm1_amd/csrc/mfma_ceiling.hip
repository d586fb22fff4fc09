// Sustained matrix-core throughput of the chip, for the benchmark's roofline.
//
// Not part of the chain and not linked into libcoda: bench.py loads the
// separate libcoda_ceiling.so built from this file.  The nominal dense peak
// assumes every matrix core busy at the top clock; under a long run with
// random operands the chip lowers its clock, so the benchmark also measures
// the throughput of a kernel that does nothing but matrix products, launched
// like the GEMMs (512-thread workgroups, two wavefronts per SIMD, 2048
// workgroups), with the same instruction and the same accumulator count per
// wavefront as the GEMM main loops.  Operands live in registers and are
// refreshed between bursts by XOR with varying masks that flip the sign, the
// mantissa and the low exponent bits (values stay finite), so the matrix
// cores see operands that change as often as in a GEMM.  No memory is
// touched inside the loop.
//
//   bf16: 32 products v_mfma_f32_16x16x32_bf16 per wavefront and iteration
//         (8 x 4 fragments, 128 accumulators per lane), as in gemm.hpp
//   fp8:  16 products v_mfma_f32_32x32x64_f8f6f4 (e4m3) per wavefront and
//         iteration (4 x 2 fragments, two k-halves), as in gemm_fp8.hpp
//
// extern "C" int coda_ceiling_bf16(float* out, int64_t out_elems, int grid,
//                                  int iters, uint32_t seed, hipStream_t s);
// extern "C" int coda_ceiling_fp8(...same...);
//   out: device buffer of at least grid * 512 floats (one sum per thread, so
//   nothing is optimised away).  Flops per launch: grid * 8 * iters * 524288
//   (bf16) or grid * 8 * iters * 2097152 (fp8).  Returns 0, or -1 for bad
//   arguments (nothing launched), or the HIP error code of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {  // 32-bit integer hash
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
// a finite bf16 with biased exponent 120..135 from 16 random bits
__device__ __forceinline__ uint32_t bf16_bits(uint32_t b) {
  return (b & 0x8000u) | ((120u + ((b >> 7) & 15u)) << 7) | (b & 0x7fu);
}
__device__ __forceinline__ uint32_t bf16x2_bits(uint32_t h) { return bf16_bits(h & 0xffffu) | (bf16_bits(h >> 16) << 16); }
// a finite e4m3 with biased exponent 4..11 from 8 random bits
__device__ __forceinline__ uint32_t e4m3_bits(uint32_t b) { return (b & 0x87u) | ((4u + ((b >> 3) & 7u)) << 3); }
__device__ __forceinline__ int e4m3x4_bits(uint32_t h) {
  return (int)(e4m3_bits(h & 255u) | (e4m3_bits((h >> 8) & 255u) << 8) | (e4m3_bits((h >> 16) & 255u) << 16) |
               (e4m3_bits(h >> 24) << 24));
}

// bf16 flip mask: sign, mantissa and the two low exponent bits of both halves
constexpr uint32_t kFlipBf16 = 0x81ff81ffu;
// e4m3 flip mask: sign, mantissa and the low exponent bit of all four bytes
constexpr uint32_t kFlipE4m3 = 0x8f8f8f8fu;

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void ceiling_bf16_kernel(
    float* out, int iters, uint32_t seed) {
  const uint32_t tid = blockIdx.x * 512u + threadIdx.x;
  u32x4 a[8], b[4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) a[i][j] = bf16x2_bits(mix(tid * 64u + i * 4 + j + seed));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) b[i][j] = bf16x2_bits(mix(tid * 64u + 32 + i * 4 + j + seed));
  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mt]),
                                                              __builtin_bit_cast(bf16x8, b[nt]), acc[mt][nt], 0, 0, 0);
    const uint32_t m = mix((uint32_t)it * 2654435761u + seed);
    const u32x4 fa = u32x4{m, m >> 1, m << 1, m ^ 0x5a5a5a5au} & kFlipBf16;
    const u32x4 fb = u32x4{m >> 2, m ^ 0xa5a5a5a5u, m << 2, m >> 3} & kFlipBf16;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] ^= fa;
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] ^= fb;
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
  out[tid] = s;
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void ceiling_fp8_kernel(
    float* out, int iters, uint32_t seed) {
  const uint32_t tid = blockIdx.x * 512u + threadIdx.x;
  i32x8 a[8], b[4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) a[i][j] = e4m3x4_bits(mix(tid * 128u + i * 8 + j + seed));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) b[i][j] = e4m3x4_bits(mix(tid * 128u + 64 + i * 8 + j + seed));
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[2 * mt + h], b[2 * nt + h], acc[mt][nt], 0,
                                                                         0, 0, 0, 0, 0);
    const uint32_t m = mix((uint32_t)it * 2654435761u + seed);
    const int f0 = (int)(m & kFlipE4m3), f1 = (int)((m >> 1) & kFlipE4m3), f2 = (int)((m << 1) & kFlipE4m3),
              f3 = (int)((m ^ 0x5a5a5a5au) & kFlipE4m3);
    const i32x8 fa = i32x8{f0, f1, f2, f3, f1, f0, f3, f2};
    const i32x8 fb = i32x8{f2, f3, f0, f1, f3, f2, f1, f0};
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] ^= fa;
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] ^= fb;
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  out[tid] = s;
}

int check(const float* out, int64_t out_elems, int grid, int iters) {
  if (out == nullptr || grid <= 0 || iters <= 0 || out_elems < (int64_t)grid * 512) return -1;
  return 0;
}

}  // namespace

extern "C" int coda_ceiling_bf16(float* out, int64_t out_elems, int grid, int iters, uint32_t seed, hipStream_t s) {
  if (check(out, out_elems, grid, iters) != 0) return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(ceiling_bf16_kernel, dim3(grid), dim3(512), 0, s, out, iters, seed);
  return (int)hipGetLastError();
}

extern "C" int coda_ceiling_fp8(float* out, int64_t out_elems, int grid, int iters, uint32_t seed, hipStream_t s) {
  if (check(out, out_elems, grid, iters) != 0) return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(ceiling_fp8_kernel, dim3(grid), dim3(512), 0, s, out, iters, seed);
  return (int)hipGetLastError();
}
