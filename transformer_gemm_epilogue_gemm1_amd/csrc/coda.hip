// libcoda C ABI: argument validation and kernel launches.
//
// Every entry point validates all arguments on the host first and returns an
// error without enqueuing anything (and without any HIP call) if one fails.
// See include/coda.h for the contract of each call.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/coda.h"
#include "epilogues.hpp"
#include "epilogues_fp8.hpp"
#include "epilogues_ce.hpp"
#include "epilogues_rope.hpp"
#include "quantize_fp8.hpp"
#include "gemm_fp8.hpp"
#include "rowops.hpp"

using namespace coda;

namespace {

thread_local std::string g_last_error;

coda_status fail(coda_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

coda_status ok() {
  g_last_error.clear();
  return CODA_OK;
}

constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr int64_t kMaxSpan = ((int64_t)1 << 31) - 256;  // 32-bit buffer offsets inside one matrix
constexpr int64_t kMaxColRows = 65535 * 64;  // rows of a column-wise quantisation (grid y of its 64-row blocks)

int elem_size(coda_dtype dt) { return dt == CODA_BF16 ? 2 : 4; }
int elems_per_chunk(coda_dtype dt) { return dt == CODA_BF16 ? 8 : 4; }

struct Mat {
  const void* p;
  int64_t rows, cols, ld;
  int es;  // element size in bytes
  const char* name;
  int64_t span() const { return rows <= 0 ? 0 : ((rows - 1) * ld + cols) * es; }
};

coda_status check_mat(const Mat& m, int E) {
  if (m.p == nullptr) return fail(CODA_ERR_NULL, "%s is NULL", m.name);
  if (m.ld < m.cols) return fail(CODA_ERR_SHAPE, "%s: ld %lld < width %lld", m.name, (long long)m.ld, (long long)m.cols);
  if (m.ld % E != 0) return fail(CODA_ERR_ALIGN, "%s: ld %lld not a multiple of %d elements", m.name, (long long)m.ld, E);
  if (((uintptr_t)m.p & 15) != 0) return fail(CODA_ERR_ALIGN, "%s is not 16-byte aligned", m.name);
  if (m.span() > kMaxSpan) return fail(CODA_ERR_SHAPE, "%s spans %lld bytes (limit 2 GiB)", m.name, (long long)m.span());
  return CODA_OK;
}

bool overlaps(const Mat& a, const Mat& b) {
  if (a.p == nullptr || b.p == nullptr || a.span() == 0 || b.span() == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.span();
  const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + b.span();
  return a0 < b1 && b0 < a1;
}

// Each output against every input and every other output.
coda_status check_alias(const Mat* outs, int nout, const Mat* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlaps(outs[i], ins[j])) return fail(CODA_ERR_ALIAS, "%s overlaps input %s", outs[i].name, ins[j].name);
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(outs[i], outs[j])) return fail(CODA_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  return CODA_OK;
}

coda_status check_dims(coda_dtype dt, int64_t M, std::initializer_list<std::pair<const char*, int64_t>> dims) {
  if (dt != CODA_BF16 && dt != CODA_F32) return fail(CODA_ERR_DTYPE, "unknown dtype %d", (int)dt);
  if (M < 0 || M > kMaxDim) return fail(CODA_ERR_SHAPE, "M = %lld out of range", (long long)M);
  for (auto& d : dims) {
    if (d.second < 1 || d.second > kMaxDim) return fail(CODA_ERR_SHAPE, "%s = %lld out of range", d.first, (long long)d.second);
    if (d.second % 8 != 0) return fail(CODA_ERR_SHAPE, "%s = %lld is not a multiple of 8", d.first, (long long)d.second);
  }
  return CODA_OK;
}

coda_status launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CODA_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return ok();
}

constexpr int kGroupM = 8;

// Bytes spanned by an operand stored as `rows` rows of `cols` elements.
uint32_t span_bytes(int64_t rows, int64_t cols, int64_t ld, int es) {
  return (uint32_t)(rows <= 0 ? 0 : ((rows - 1) * ld + cols) * es);
}

// Bytes of a tile-packed bf16 matrix (kp_unit): rows padded to 16, cols / 8 chunks.
int64_t packed_bytes(int64_t rows, int64_t cols) { return (rows + 15) / 16 * 16 * cols * 2; }

// AL, BL: OpLayout of a contraction-contiguous A or B (kLayPacked: lda / ldb
// count 16-byte chunks per row).
template <typename T, bool AKC, bool BKC, class Epi, int AL = kLayKC, int BL = kLayKC>
coda_status launch_gemm(const char* what, int M, int N, int K, const void* a, int64_t lda, const void* b,
                        int64_t ldb, const typename Epi::Params& ep, hipStream_t s, int b_split = 0) {
  GemmArgs g;
  g.M = M;
  g.N = N;
  g.K = K;
  g.tiles_m = (M + kTileM - 1) / kTileM;
  g.tiles_n = (N + kTileN - 1) / kTileN;
  g.group_m = kGroupM;
  g.a = a;
  g.lda = lda;
  constexpr int al = AKC ? AL : kLayKC, bl = BKC ? BL : kLayKC;
  g.a_span = al == kLayPacked ? (uint32_t)packed_bytes(M, 8 * lda)
                              : AKC ? span_bytes(M, K, lda, sizeof(T)) : span_bytes(K, M, lda, sizeof(T));
  g.b = b;
  g.ldb = ldb;
  g.b_span = bl == kLayPacked ? (uint32_t)packed_bytes(N, 8 * ldb)
                              : BKC ? span_bytes(N, K, ldb, sizeof(T)) : span_bytes(K, N, ldb, sizeof(T));
  g.b_split = b_split;
  const int nblocks = g.tiles_m * g.tiles_n;
  hipLaunchKernelGGL((gemm_kernel<T, AKC, BKC, Epi, al, bl>), dim3(nblocks), dim3(kThreads), 0, s, g, ep);
  return launch_status(what);
}

// Bytes of a tile-packed e4m3 matrix (kp_unit): rows padded to 16, cols / 16 chunks.
int64_t packed_bytes_e4m3(int64_t rows, int64_t cols) { return (rows + 15) / 16 * 16 * cols; }

// Bytes of a block-exponent array (mx_byte layout) for `rows` rows and
// `cols` contraction columns: 1 KiB per 128-row block and group of 4 k-tiles.
int64_t mx_exp_bytes(int64_t rows, int64_t cols) { return 1024 * mx_row_blocks(rows) * ((cols + 255) / 256); }

// L: OpLayout of both operands (kLayPacked: lda / ldb counting 16-byte chunks
// per row).  MX: a mask of kMxA (a_exp holds the block exponents of A,
// mx_byte layout, mx_exp_bytes(M, K) bytes) and kMxB (b_exp those of B,
// mx_exp_bytes(N, K) bytes).
template <class Epi, int L = kLayKC, int MX = 0>
coda_status launch_gemm_fp8(const char* what, int M, int N, int K, const void* a, int64_t lda, const void* b,
                            int64_t ldb, const typename Epi::Params& ep, hipStream_t s,
                            const void* a_exp = nullptr, const void* b_exp = nullptr) {
  GemmArgs g;
  g.M = M;
  g.N = N;
  g.K = K;
  g.tiles_m = (M + kTileM - 1) / kTileM;
  g.tiles_n = (N + kTileN - 1) / kTileN;
  g.group_m = kGroupM;
  g.a = a;
  g.lda = lda;
  g.a_span = L == kLayPacked ? (uint32_t)packed_bytes_e4m3(M, 16 * lda) : span_bytes(M, K, lda, 1);
  g.b = b;
  g.ldb = ldb;
  g.b_span = L == kLayPacked ? (uint32_t)packed_bytes_e4m3(N, 16 * ldb) : span_bytes(N, K, ldb, 1);
  g.b_split = 0;
  const MxArgs mxa{(const uint8_t*)a_exp, M, (uint32_t)mx_exp_bytes(M, K)};
  const MxArgs mxb{(const uint8_t*)b_exp, N, (uint32_t)mx_exp_bytes(N, K)};
  hipLaunchKernelGGL((gemm_fp8_kernel<Epi, L, MX>), dim3(g.tiles_m * g.tiles_n), dim3(kThreads), 0, s, g, ep, mxa,
                     mxb);
  return launch_status(what);
}

// fp8 operands come in 16-element (16-byte) chunks: contraction lengths and
// widths are multiples of 16.
coda_status check_dims_fp8(int64_t M, std::initializer_list<std::pair<const char*, int64_t>> dims) {
  if (M < 0 || M > kMaxDim) return fail(CODA_ERR_SHAPE, "M = %lld out of range", (long long)M);
  for (auto& d : dims) {
    if (d.second < 1 || d.second > kMaxDim) return fail(CODA_ERR_SHAPE, "%s = %lld out of range", d.first, (long long)d.second);
    if (d.second % 16 != 0) return fail(CODA_ERR_SHAPE, "%s = %lld is not a multiple of 16", d.first, (long long)d.second);
  }
  return CODA_OK;
}

coda_status check_vec(const float* p, int64_t n, int align, const char* name) {
  if (p == nullptr) return fail(CODA_ERR_NULL, "%s is NULL", name);
  if (((uintptr_t)p & (align - 1)) != 0) return fail(CODA_ERR_ALIGN, "%s is not %d-byte aligned", name, align);
  if (n * 4 > kMaxSpan) return fail(CODA_ERR_SHAPE, "%s too long", name);
  return CODA_OK;
}

int64_t num_partials(int64_t D) { return (kTileN / kPartialCols) * ((D + kTileN - 1) / kTileN); }

template <typename T>
coda_status gemm_res_prms_impl(int M, int K, int D, const void* A, int64_t lda, const void* W1, int64_t ldw1,
                               const void* R, int64_t ldr, const void* g, void* H, int64_t ldh, void* Hg,
                               int64_t ldhg, float* partials, hipStream_t s) {
  typename EpiResPrms<T>::Params ep{(const T*)R, ldr, (const T*)g, (T*)H, ldh, (T*)Hg, ldhg, partials};
  return launch_gemm<T, true, false, EpiResPrms<T>>("coda_gemm_res_prms", M, D, K, A, lda, W1, ldw1, ep, s);
}

template <typename T>
coda_status gemm_rowscale_impl(int M, int D, int N2, const void* X, int64_t ldx, const void* W2, int64_t ldw2,
                               const float* r, void* Y, int64_t ldy, hipStream_t s) {
  typename EpiRowScale<T>::Params ep{r, (T*)Y, ldy};
  return launch_gemm<T, true, false, EpiRowScale<T>>("coda_gemm_rowscale", M, N2, D, X, ldx, W2, ldw2, ep, s);
}

// The forward pair with the Hg intermediate tile-packed (bf16): the first
// GEMM's epilogue stores Hg in the order the second GEMM's fragment reads use.
coda_status gemm_res_prms_packed_impl(int M, int K, int D, const void* A, int64_t lda, const void* W1, int64_t ldw1,
                                      const void* R, int64_t ldr, const void* g, void* H, int64_t ldh, void* Hgp,
                                      float* partials, hipStream_t s) {
  typename EpiResPrms<uint16_t>::Params ep{(const uint16_t*)R, ldr, (const uint16_t*)g, (uint16_t*)H, ldh,
                                           (uint16_t*)Hgp, 0, partials, D / 8};
  return launch_gemm<uint16_t, true, false, EpiResPrms<uint16_t>>("coda_gemm_res_prms_packed", M, D, K, A, lda, W1,
                                                                  ldw1, ep, s);
}

coda_status gemm_rowscale_packed_impl(int M, int D, int N2, const void* Xp, const void* W2, int64_t ldw2,
                                      const float* r, void* Y, int64_t ldy, hipStream_t s) {
  typename EpiRowScale<uint16_t>::Params ep{r, (uint16_t*)Y, ldy};
  return launch_gemm<uint16_t, true, false, EpiRowScale<uint16_t>, kLayPacked>("coda_gemm_rowscale_packed", M, N2, D, Xp,
                                                                         D / 8, W2, ldw2, ep, s);
}

template <typename T>
coda_status gemm_rowscale_swiglu_impl(int M, int D, int F, const void* X, int64_t ldx, const void* W2,
                                      int64_t ldw2, const float* r, void* Z, int64_t ldz, void* Y, int64_t ldy,
                                      hipStream_t s) {
  typename EpiSwiGLU<T>::Params ep{r, (T*)Z, ldz, (T*)Y, ldy, F};
  return launch_gemm<T, true, false, EpiSwiGLU<T>>("coda_gemm_rowscale_swiglu", M, 2 * F, D, X, ldx, W2, ldw2, ep,
                                                   s, F);
}

coda_status gemm_rowscale_swiglu_packed_impl(int M, int D, int F, const void* Xp, const void* W2, int64_t ldw2,
                                             const float* r, void* Z, int64_t ldz, void* Y, int64_t ldy,
                                             hipStream_t s) {
  typename EpiSwiGLU<uint16_t>::Params ep{r, (uint16_t*)Z, ldz, (uint16_t*)Y, ldy, F};
  return launch_gemm<uint16_t, true, false, EpiSwiGLU<uint16_t>, kLayPacked>("coda_gemm_rowscale_swiglu_packed", M, 2 * F,
                                                                       D, Xp, D / 8, W2, ldw2, ep, s, F);
}

coda_status combine_impl(int M, int D, int T, float eps, const float* partials, float* r, hipStream_t s) {
  hipLaunchKernelGGL(rms_combine_kernel, dim3((M + 63) / 64), dim3(256), 0, s, partials, r, M, T, D, eps);
  return launch_status("coda_rms_combine");
}

// ---- backward ------------------------------------------------------------
constexpr size_t kWsAlign = 256;
size_t align_up(size_t x) { return (x + kWsAlign - 1) & ~(kWsAlign - 1); }

// Workspace of the backward, in this order, each part 256-byte aligned: X_n,
// the row and column partial sums, c, and the transposed weights W2^T [N2, D]
// and W1^T [D, K] (K = N2 = 0: none), so that G = dY W2^T and dA = dH W1^T
// read their weight row-contiguously.  (Read in place, both operands of those
// products are contraction-contiguous; measured 1% slower for the whole
// backward at 7B than transposing first.)
struct BwdWs {
  size_t xn, srow, dgcol, c, w2t, w1t, total;
  // with_xn false: no room for X_n (the fp8 backward codes it in G's epilogue)
  BwdWs(int64_t M, int64_t K, int64_t D, int64_t N2, int es, bool with_xn = true) {
    const int64_t T = num_partials(D), U = (M + kWaveM - 1) / kWaveM;
    xn = 0;
    srow = align_up(xn + (with_xn ? (size_t)M * D * es : 0));
    dgcol = align_up(srow + (size_t)T * M * 4);
    c = align_up(dgcol + (size_t)U * D * 4);
    w2t = align_up(c + (size_t)M * 4);
    w1t = align_up(w2t + (size_t)N2 * D * es);
    total = align_up(w1t + (size_t)D * K * es);
    if (total < kWsAlign) total = kWsAlign;  // never empty: a zero-byte workspace would come as NULL
  }
};

// IN_PLACE: G and dA read W2 and W1 where they lie, as contraction-contiguous
// B operands, and the workspace holds no transposed weights (BwdWs with
// K = N2 = 0).  The products see the same fragments either way, so the
// results are bit-identical; the transposes make the whole backward about 1%
// faster at 7B.
template <typename T, bool IN_PLACE = false>
coda_status chain_bwd_impl(int M, int K, int D, int N2, const void* dY, const void* A, const void* W1,
                           const void* g, const void* W2, const void* H, const float* r, void* dA, void* dR,
                           void* dW1, void* dW2, float* dg, char* ws, hipStream_t s) {
  const BwdWs L(M, IN_PLACE ? 0 : K, D, IN_PLACE ? 0 : N2, sizeof(T));
  T* Xn = (T*)(ws + L.xn);
  float* srow = (float*)(ws + L.srow);
  float* dgcol = (float*)(ws + L.dgcol);
  float* c = (float*)(ws + L.c);
  T* W2t = (T*)(ws + L.w2t);
  T* W1t = (T*)(ws + L.w1t);
  const int Tn = (int)num_partials(D), U = (M + kWaveM - 1) / kWaveM;
  coda_status st;
  if (M > 0) {
    typename EpiBwdG<T>::Params ep{(const T*)H, (const T*)g, r, (T*)dR, Xn, D, srow, dgcol};
    if constexpr (IN_PLACE) {
      // 1. G = dY W2^T with the P / X_n / partial-sum epilogue, W2 [D, N2] in place
      if ((st = launch_gemm<T, true, true, EpiBwdG<T>>("coda_chain_bwd G", M, D, N2, dY, N2, W2, N2, ep, s)) !=
          CODA_OK)
        return st;
    } else {
      // 0. W2^T and W1^T: the contraction of G and dA then runs across their
      // rows (transposing LDS reads, no bank conflicts) instead of along them
      hipLaunchKernelGGL(transpose_kernel<T>, dim3((unsigned)((N2 + 63) / 64), (unsigned)((D + 63) / 64)), dim3(256),
                         0, s, (const T*)W2, N2, D, N2, W2t, D);
      hipLaunchKernelGGL(transpose_kernel<T>, dim3((unsigned)((D + 63) / 64), (unsigned)((K + 63) / 64)), dim3(256),
                         0, s, (const T*)W1, D, K, D, W1t, K);
      if ((st = launch_status("coda_chain_bwd transpose")) != CODA_OK) return st;
      // 1. G = dY W2^T with the P / X_n / partial-sum epilogue
      if ((st = launch_gemm<T, true, false, EpiBwdG<T>>("coda_chain_bwd G", M, D, N2, dY, N2, W2t, D, ep, s)) !=
          CODA_OK)
        return st;
    }
  }
  // 2. c and dg (with M = 0 only the columns: dg = 0)
  hipLaunchKernelGGL(bwd_combine_kernel, dim3((unsigned)((M + 63) / 64 + (D + 63) / 64)), dim3(256), 0, s, srow,
                     dgcol, r, c, dg, M, Tn, D, U);
  if ((st = launch_status("coda_chain_bwd combine")) != CODA_OK) return st;
  if (M > 0) {
    // 3. dH in place in dR
    const int64_t nchunks = (int64_t)M * D / 8;
    const int blocks = (int)((nchunks + 255) / 256 < 16384 ? (nchunks + 255) / 256 : 16384);
    hipLaunchKernelGGL(dh_finalize_kernel<T>, dim3(blocks), dim3(256), 0, s, (T*)dR, (const T*)H, r, c, D, nchunks);
    if ((st = launch_status("coda_chain_bwd dH")) != CODA_OK) return st;
    // 4. dA = dH W1^T  (W1^T [D, K] read row-contiguously, or W1 [K, D] in place)
    const typename EpiRowScale<T>::Params epa{nullptr, (T*)dA, K};
    if constexpr (IN_PLACE)
      st = launch_gemm<T, true, true, EpiRowScale<T>>("coda_chain_bwd dA", M, K, D, dR, D, W1, D, epa, s);
    else
      st = launch_gemm<T, true, false, EpiRowScale<T>>("coda_chain_bwd dA", M, K, D, dR, D, W1t, K, epa, s);
    if (st != CODA_OK) return st;
  }
  // 5. dW1 = A^T dH  and  6. dW2 = X_n^T dY: contraction over the M rows.
  // With M = 0 the main loop runs no k-tile and writes zeros; the M-row
  // operands (possibly NULL then) are replaced by W1 with an empty span, so
  // no load is ever made from them.
  const void* a5 = M > 0 ? A : W1;
  const void* b5 = M > 0 ? (const void*)dR : W1;
  const void* b6 = M > 0 ? dY : W1;
  if ((st = launch_gemm<T, false, false, EpiRowScale<T>>("coda_chain_bwd dW1", K, D, M, a5, K, b5, D,
                                                         typename EpiRowScale<T>::Params{nullptr, (T*)dW1, D}, s)) !=
      CODA_OK)
    return st;
  return launch_gemm<T, false, false, EpiRowScale<T>>("coda_chain_bwd dW2", D, N2, M, Xn, D, b6, N2,
                                                      typename EpiRowScale<T>::Params{nullptr, (T*)dW2, N2}, s);
}

// Workspace of the fp8 backward: the bf16 backward's partial sums and c (no
// X_n: G's epilogue writes its codes) followed by the e4m3 operands of the
// four products (tile-packed codes) and their block exponents (mx_byte
// layout).
struct Bwd8Ws {
  BwdWs b;
  size_t dy8, edy, dyt8, edyt, w2q, ew2, w1q, ew1, dh8, edh, dht8, edht, xnt8, exn, at8, eat, total;
  Bwd8Ws(int64_t M, int64_t K, int64_t D, int64_t N2) : b(M, 0, D, 0, 2, false) {
    size_t o = b.total;
    auto take = [&o](int64_t bytes) {
      const size_t at = o;
      o = align_up(o + (size_t)bytes);
      return at;
    };
    dy8 = take(M * N2);                  // dY, rows (G's A)
    edy = take(mx_exp_bytes(M, N2));
    dyt8 = take(N2 * M);                 // dY^T (dW2's B)
    edyt = take(mx_exp_bytes(N2, M));
    w2q = take(D * N2);                  // W2 [D, N2], rows (G's B)
    ew2 = take(mx_exp_bytes(D, N2));
    w1q = take(K * D);                   // W1 [K, D], rows (dA's B)
    ew1 = take(mx_exp_bytes(K, D));
    dh8 = take(M * D);                   // dH, rows (dA's A)
    edh = take(mx_exp_bytes(M, D));
    dht8 = take(D * M);                  // dH^T (dW1's B)
    edht = take(mx_exp_bytes(D, M));
    xnt8 = take(D * M);                  // X_n^T (dW2's A)
    exn = take(mx_exp_bytes(D, M));
    at8 = take(K * M);                   // A^T (dW1's A)
    eat = take(mx_exp_bytes(K, M));
    total = o;
  }
};

// Unchecked launches of the quantisers (shapes validated by the caller).
// A nonzero *_nck writes that code array tile-packed (kp_unit) with that many
// 16-code units per row instead of row-major.
void q_rows(const void* X, int64_t ldx, int M, int K, void* X8, int64_t ldx8, float* sc, hipStream_t s,
            int64_t x8_nck = 0) {
  const dim3 grid((unsigned)M), block(256);
  const uint16_t* x = (const uint16_t*)X;
  uint8_t* x8 = (uint8_t*)X8;
  const int chunks = (K / 8 + 255) / 256;  // 16-byte chunks per thread
  if (x8_nck > 0 && K <= 8 * 1024) {
    // tile-packed codes: 4 rows per workgroup, up to UPL units per lane
    const dim3 g4((unsigned)((M + 3) / 4));
    const int upl = (K / 16 + 63) / 64;
    if (upl <= 1)
      hipLaunchKernelGGL(quantize_rows_packed_e4m3_kernel<1>, g4, block, 0, s, x, ldx, M, K, x8, sc, x8_nck);
    else if (upl <= 2)
      hipLaunchKernelGGL(quantize_rows_packed_e4m3_kernel<2>, g4, block, 0, s, x, ldx, M, K, x8, sc, x8_nck);
    else if (upl <= 4)
      hipLaunchKernelGGL(quantize_rows_packed_e4m3_kernel<4>, g4, block, 0, s, x, ldx, M, K, x8, sc, x8_nck);
    else
      hipLaunchKernelGGL(quantize_rows_packed_e4m3_kernel<8>, g4, block, 0, s, x, ldx, M, K, x8, sc, x8_nck);
    return;
  }
  if (chunks <= 1)
    hipLaunchKernelGGL(quantize_rows_e4m3_kernel<1>, grid, block, 0, s, x, ldx, K, x8, ldx8, sc, x8_nck);
  else if (chunks <= 2)
    hipLaunchKernelGGL(quantize_rows_e4m3_kernel<2>, grid, block, 0, s, x, ldx, K, x8, ldx8, sc, x8_nck);
  else if (chunks <= 4)
    hipLaunchKernelGGL(quantize_rows_e4m3_kernel<4>, grid, block, 0, s, x, ldx, K, x8, ldx8, sc, x8_nck);
  else if (chunks <= 8)
    hipLaunchKernelGGL(quantize_rows_e4m3_kernel<8>, grid, block, 0, s, x, ldx, K, x8, ldx8, sc, x8_nck);
  else if (chunks <= 16)
    hipLaunchKernelGGL(quantize_rows_e4m3_kernel<16>, grid, block, 0, s, x, ldx, K, x8, ldx8, sc, x8_nck);
  else
    hipLaunchKernelGGL(quantize_long_rows_e4m3_kernel, grid, block, 0, s, x, ldx, K, x8, ldx8, sc, x8_nck);
}
// wt_nck > 0: Wt8 written tile-packed with wt_nck chunks per row (K / 16).
void q_cols(const void* W, int64_t ldw, int K, int N, void* Wt8, int64_t ldwt, float* sc, hipStream_t s,
            int64_t wt_nck = 0) {
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, (uint32_t*)sc, N, 0u);
  hipLaunchKernelGGL(colmax_kernel, dim3((unsigned)((N + 63) / 64), (unsigned)((K + 255) / 256)), dim3(256), 0, s,
                     (const uint16_t*)W, ldw, K, N, (uint32_t*)sc);
  hipLaunchKernelGGL(quantize_cols_kernel, dim3((unsigned)((N + 127) / 128), (unsigned)((K + 127) / 128)), dim3(256),
                     0, s, (const uint16_t*)W, ldw, K, N, (const uint32_t*)sc, (uint8_t*)Wt8, ldwt,
                     (const uint32_t*)nullptr, (uint8_t*)nullptr, (int64_t)0, wt_nck, (int64_t)0);
  hipLaunchKernelGGL(amax_to_scale_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, sc, N);
}
// Both quantisations of an activation X [M, N]: row codes X8 [M, N] with
// scales sr [M] (as q_rows) and column codes Xt8 [N, M] with scales sc [N]
// (as q_cols), from one pass for the maxima and one for the codes.
void q_rows_cols(const void* X, int64_t ldx, int M, int N, void* X8, int64_t ldx8, float* sr, void* Xt8,
                 int64_t ldxt, float* sc, hipStream_t s, int64_t x8_nck = 0, int64_t xt_nck = 0) {
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, (uint32_t*)sr, M, 0u);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, (uint32_t*)sc, N, 0u);
  hipLaunchKernelGGL(rowcol_max_kernel, dim3((unsigned)((N + 255) / 256), (unsigned)((M + 255) / 256)), dim3(256), 0,
                     s, (const uint16_t*)X, ldx, M, N, (uint32_t*)sr, (uint32_t*)sc);
  hipLaunchKernelGGL(quantize_cols_kernel, dim3((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128)), dim3(256),
                     0, s, (const uint16_t*)X, ldx, M, N, (const uint32_t*)sc, (uint8_t*)Xt8, ldxt,
                     (const uint32_t*)sr, (uint8_t*)X8, ldx8, xt_nck, x8_nck);
  hipLaunchKernelGGL(amax_to_scale_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, sr, M);
  hipLaunchKernelGGL(amax_to_scale_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, sc, N);
}

// MX quantisation of X [M, N] (bf16) along its rows (Xr8, Er) and/or along
// its columns (Xc8 = the codes of X^T, Ec), tile-packed; a pair left null is
// not produced.  M % 16 == 0, N % 16 == 0, ceil(N / 256) <= 65535.
void q_mx(const void* X, int64_t ldx, int M, int N, void* Xr8, void* Er, void* Xc8, void* Ec, hipStream_t s) {
  const dim3 grid((unsigned)((256 / kMxTileRows) * ((M + 255) / 256)), (unsigned)((N + 255) / 256)), block(256);
  const uint16_t* x = (const uint16_t*)X;
  uint8_t *r8 = (uint8_t*)Xr8, *er = (uint8_t*)Er, *c8 = (uint8_t*)Xc8, *ec = (uint8_t*)Ec;
  if (Xr8 != nullptr && Xc8 != nullptr)
    hipLaunchKernelGGL((mx_quantize_kernel<true, true>), grid, block, 0, s, x, ldx, M, N, r8, er, c8, ec);
  else if (Xr8 != nullptr)
    hipLaunchKernelGGL((mx_quantize_kernel<true, false>), grid, block, 0, s, x, ldx, M, N, r8, er, c8, ec);
  else
    hipLaunchKernelGGL((mx_quantize_kernel<false, true>), grid, block, 0, s, x, ldx, M, N, r8, er, c8, ec);
}

// The chain's backward with every product on e4m3 operands with MX block
// exponents along its contraction (bf16 tensors in and out); the products
// apply the exponents of both operands, and the per-element steps are the
// bf16 backward's.  M > 0, all sizes multiples of 16.  Every code array is
// written tile-packed (no padding rows, since all row counts are multiples of
// 16), so all four products read both operands in the packed layout.
coda_status chain_bwd_fp8_impl(int M, int K, int D, int N2, const void* dY, const void* A, const void* W1,
                               const void* g, const void* W2, const void* H, const float* r, void* dA, void* dR,
                               void* dW1, void* dW2, float* dg, char* ws, hipStream_t s) {
  const Bwd8Ws L(M, K, D, N2);
  float* srow = (float*)(ws + L.b.srow);
  float* dgcol = (float*)(ws + L.b.dgcol);
  float* c = (float*)(ws + L.b.c);
  const int Tn = (int)num_partials(D), U = (M + kWaveM - 1) / kWaveM;
  coda_status st;
  char* const w = ws;
  // operands of G = dY W2^T (rows) and dW2 = X_n^T dY (dY's columns)
  q_mx(dY, N2, M, N2, w + L.dy8, w + L.edy, w + L.dyt8, w + L.edyt, s);
  q_mx(W2, N2, D, N2, w + L.w2q, w + L.ew2, nullptr, nullptr, s);
  q_mx(W1, D, K, D, w + L.w1q, w + L.ew1, nullptr, nullptr, s);
  if ((st = launch_status("coda_chain_bwd_fp8 quantise dY, W1, W2")) != CODA_OK) return st;
  // 1. G with the P / partial-sum epilogue, X_n leaving as dW2's operand (its
  // column codes and exponents)
  using EpiG = EpiBwdGMx;
  const typename EpiG::Params eg{{(const uint16_t*)H, (const uint16_t*)g, r, (uint16_t*)dR, nullptr, D, srow, dgcol},
                                 (uint8_t*)(w + L.xnt8), (uint8_t*)(w + L.exn)};
  if ((st = launch_gemm_fp8<EpiG, kLayPacked, kMxA | kMxB>("coda_chain_bwd_fp8 G", M, D, N2, w + L.dy8, N2 / 16,
                                                           w + L.w2q, N2 / 16, eg, s, w + L.edy, w + L.ew2)) !=
      CODA_OK)
    return st;
  // 2. c and dg;  3. dH in place in dR
  hipLaunchKernelGGL(bwd_combine_kernel, dim3((unsigned)((M + 63) / 64 + (D + 63) / 64)), dim3(256), 0, s, srow,
                     dgcol, r, c, dg, M, Tn, D, U);
  const int64_t nchunks = (int64_t)M * D / 8;
  const int blocks = (int)((nchunks + 255) / 256 < 16384 ? (nchunks + 255) / 256 : 16384);
  hipLaunchKernelGGL(dh_finalize_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, (uint16_t*)dR, (const uint16_t*)H,
                     r, c, D, nchunks);
  // operands of dA = dH W1^T (dH rows) and dW1 = A^T dH (columns)
  q_mx(dR, D, M, D, w + L.dh8, w + L.edh, w + L.dht8, w + L.edht, s);
  q_mx(A, K, M, K, nullptr, nullptr, w + L.at8, w + L.eat, s);
  if ((st = launch_status("coda_chain_bwd_fp8 combine, dH, quantise")) != CODA_OK) return st;
  using EpiO = EpiRowScale<uint16_t>;
  // 4. dA = dH W1^T
  if ((st = launch_gemm_fp8<EpiO, kLayPacked, kMxA | kMxB>("coda_chain_bwd_fp8 dA", M, K, D, w + L.dh8, D / 16,
                                                           w + L.w1q, D / 16, typename EpiO::Params{nullptr, (uint16_t*)dA, K},
                                                           s, w + L.edh, w + L.ew1)) != CODA_OK)
    return st;
  // 5. dW1 = A^T dH;  6. dW2 = X_n^T dY  (contraction over the M rows)
  if ((st = launch_gemm_fp8<EpiO, kLayPacked, kMxA | kMxB>("coda_chain_bwd_fp8 dW1", K, D, M, w + L.at8, M / 16,
                                                           w + L.dht8, M / 16, typename EpiO::Params{nullptr, (uint16_t*)dW1, D},
                                                           s, w + L.eat, w + L.edht)) != CODA_OK)
    return st;
  return launch_gemm_fp8<EpiO, kLayPacked, kMxA | kMxB>("coda_chain_bwd_fp8 dW2", D, N2, M, w + L.xnt8, M / 16,
                                                        w + L.dyt8, M / 16, typename EpiO::Params{nullptr, (uint16_t*)dW2, N2},
                                                        s, w + L.exn, w + L.edyt);
}

// Shared checks of the RoPE entry points: head layout, positions, table.
coda_status check_rope(int64_t M, int64_t N, const int32_t* positions, const float* cos_sin, int64_t max_pos,
                       int64_t n_q, int64_t n_k, int64_t d_head, Mat* mpos, Mat* mcs) {
  if (d_head < 8 || d_head > 4096 || d_head % 8 != 0)
    return fail(CODA_ERR_SHAPE, "d_head = %lld is not a multiple of 8 in [8, 4096]", (long long)d_head);
  if (n_q < 0 || n_k < 0 || n_q % d_head != 0 || n_k % d_head != 0)
    return fail(CODA_ERR_SHAPE, "n_q = %lld and n_k = %lld must be whole heads of %lld", (long long)n_q,
                (long long)n_k, (long long)d_head);
  if (n_q + n_k > N) return fail(CODA_ERR_SHAPE, "n_q + n_k = %lld exceeds the width %lld", (long long)(n_q + n_k),
                                 (long long)N);
  if (max_pos < 1 || max_pos > kMaxDim) return fail(CODA_ERR_SHAPE, "max_pos = %lld out of range", (long long)max_pos);
  if (M == 0) return CODA_OK;  // nothing is read
  if (positions == nullptr || cos_sin == nullptr) return fail(CODA_ERR_NULL, "positions and cos_sin must be set");
  if (((uintptr_t)positions & 3) != 0) return fail(CODA_ERR_ALIGN, "positions is not 4-byte aligned");
  if (((uintptr_t)cos_sin & 15) != 0) return fail(CODA_ERR_ALIGN, "cos_sin is not 16-byte aligned");
  *mpos = Mat{positions, 1, M, M, 4, "positions"};
  *mcs = Mat{cos_sin, max_pos, d_head, d_head, 4, "cos_sin"};
  if (mcs->span() > kMaxSpan) return fail(CODA_ERR_SHAPE, "cos_sin spans more than 2 GiB");
  return CODA_OK;
}

// Argument checks of the backward shared by coda_chain_bwd and
// coda_chain_bwd_noalloc (all but the workspace).  Matrices with M rows are
// checked only when M > 0 (they may be NULL then).
coda_status check_bwd_args(coda_dtype dt, int64_t M, int64_t K, int64_t D, int64_t N2, const void* dY,
                           const void* A, const void* W1, const void* g, const void* W2, const void* H,
                           const float* r, void* dA, void* dR, void* dW1, void* dW2, float* dg) {
  coda_status st = check_dims(dt, M, {{"K", K}, {"D", D}, {"N2", N2}});
  if (st != CODA_OK) return st;
  const int es = elem_size(dt), E = elems_per_chunk(dt);
  const Mat mdY{dY, M, N2, N2, es, "dY"}, mA{A, M, K, K, es, "A"}, mH{H, M, D, D, es, "H"};
  const Mat mdA{dA, M, K, K, es, "dA"}, mdR{dR, M, D, D, es, "dR"};
  const Mat mW1{W1, K, D, D, es, "W1"}, mg{g, 1, D, D, es, "g"}, mW2{W2, D, N2, N2, es, "W2"};
  const Mat mdW1{dW1, K, D, D, es, "dW1"}, mdW2{dW2, D, N2, N2, es, "dW2"};
  for (const Mat* m : {&mW1, &mg, &mW2, &mdW1, &mdW2})
    if ((st = check_mat(*m, E)) != CODA_OK) return st;
  if (M > 0) {
    for (const Mat* m : {&mdY, &mA, &mH, &mdA, &mdR})
      if ((st = check_mat(*m, E)) != CODA_OK) return st;
    if (r == nullptr) return fail(CODA_ERR_NULL, "r is NULL");
    if (((uintptr_t)r & 3) != 0) return fail(CODA_ERR_ALIGN, "r is not 4-byte aligned");
  }
  if (dg == nullptr) return fail(CODA_ERR_NULL, "dg is NULL");
  if (((uintptr_t)dg & 3) != 0) return fail(CODA_ERR_ALIGN, "dg is not 4-byte aligned");
  return CODA_OK;
}

// Outputs (and the workspace, when ws names one) against the inputs and
// each other.
coda_status check_bwd_alias(coda_dtype dt, int64_t M, int64_t K, int64_t D, int64_t N2, const void* dY,
                            const void* A, const void* W1, const void* g, const void* W2, const void* H,
                            const float* r, void* dA, void* dR, void* dW1, void* dW2, float* dg, const Mat& ws) {
  const int es = elem_size(dt);
  const Mat mdY{dY, M, N2, N2, es, "dY"}, mA{A, M, K, K, es, "A"}, mH{H, M, D, D, es, "H"};
  const Mat mdA{dA, M, K, K, es, "dA"}, mdR{dR, M, D, D, es, "dR"};
  const Mat mW1{W1, K, D, D, es, "W1"}, mg{g, 1, D, D, es, "g"}, mW2{W2, D, N2, N2, es, "W2"};
  const Mat mdW1{dW1, K, D, D, es, "dW1"}, mdW2{dW2, D, N2, N2, es, "dW2"};
  const Mat mr{r, 1, M, M, 4, "r"}, mdg{dg, 1, D, D, 4, "dg"};
  const Mat none{nullptr, 0, 0, 0, es, ""};
  const Mat outs[6] = {M > 0 ? mdA : none, M > 0 ? mdR : none, mdW1, mdW2, mdg, ws};
  const Mat ins[7] = {M > 0 ? mdY : none, M > 0 ? mA : none, mW1, mg, mW2, M > 0 ? mH : none, M > 0 ? mr : none};
  return check_alias(outs, 6, ins, 7);
}

// ---- scratch of coda_chain_bwd_noalloc ----------------------------------
// A file-scope device array: every GPU the library runs on holds its own
// copy from the time the library's code is loaded on it until the process
// ends.  Host code never passes the array's name to a kernel or a copy (on
// the host it is only a stand-in for the symbol): the device address comes
// from hipGetSymbolAddress, taken once per device with that device current,
// on the first call of coda_chain_bwd_noalloc there.
constexpr size_t kNoAllocScratchBytes = CODA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::vector<char*> g_scratch_ptr;  // per device ordinal, nullptr until looked up

coda_status noalloc_scratch(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CODA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(CODA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = (char*)p;
  }
  *out = g_scratch_ptr[dev];
  return CODA_OK;
}

}  // namespace

extern "C" {

int64_t coda_prms_num_partials(coda_dtype dt, int64_t D) {
  if (dt != CODA_BF16 && dt != CODA_F32) return -1;
  if (D < 1 || D > kMaxDim) return -1;
  return num_partials(D);
}

coda_status coda_gemm_res_prms(coda_dtype dt, int64_t M, int64_t K, int64_t D, const void* A, int64_t lda,
                               const void* W1, int64_t ldw1, const void* R, int64_t ldr, const void* g, void* H,
                               int64_t ldh, void* Hg, int64_t ldhg, float* partials, void* stream) {
  coda_status st = check_dims(dt, M, {{"K", K}, {"D", D}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  const int es = elem_size(dt), E = elems_per_chunk(dt);
  const int64_t T = num_partials(D);
  if ((g == nullptr) != (Hg == nullptr)) return fail(CODA_ERR_NULL, "g and Hg must be both NULL or both set");
  const Mat mA{A, M, K, lda, es, "A"}, mW1{W1, K, D, ldw1, es, "W1"}, mR{R, M, D, ldr, es, "R"};
  const Mat mg{g, 1, D, D, es, "g"}, mH{H, M, D, ldh, es, "H"}, mHg{Hg, M, D, ldhg, es, "Hg"};
  const Mat mP{partials, T, M, M, 4, "partials"};
  for (const Mat* m : {&mA, &mW1, &mR, &mH})
    if ((st = check_mat(*m, E)) != CODA_OK) return st;
  if (g != nullptr) {
    if ((st = check_mat(mg, E)) != CODA_OK) return st;
    if ((st = check_mat(mHg, E)) != CODA_OK) return st;
  }
  if (partials == nullptr) return fail(CODA_ERR_NULL, "partials is NULL");
  if (((uintptr_t)partials & 3) != 0) return fail(CODA_ERR_ALIGN, "partials is not 4-byte aligned");
  if (mP.span() > kMaxSpan) return fail(CODA_ERR_SHAPE, "partials span too large");
  const Mat outs[3] = {mH, g ? mHg : Mat{nullptr, 0, 0, 0, es, "Hg"}, mP};
  const Mat ins[4] = {mA, mW1, mR, g ? mg : Mat{nullptr, 0, 0, 0, es, "g"}};
  if ((st = check_alias(outs, 3, ins, 4)) != CODA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (dt == CODA_BF16)
    return gemm_res_prms_impl<uint16_t>((int)M, (int)K, (int)D, A, lda, W1, ldw1, R, ldr, g, H, ldh, Hg, ldhg,
                                        partials, s);
  return gemm_res_prms_impl<float>((int)M, (int)K, (int)D, A, lda, W1, ldw1, R, ldr, g, H, ldh, Hg, ldhg, partials,
                                   s);
}

coda_status coda_rms_combine(int64_t M, int64_t D, int64_t T, float eps, const float* partials, float* r,
                             void* stream) {
  if (M < 0 || M > kMaxDim) return fail(CODA_ERR_SHAPE, "M = %lld out of range", (long long)M);
  if (D < 1 || D > kMaxDim) return fail(CODA_ERR_SHAPE, "D = %lld out of range", (long long)D);
  if (T < 1 || T > 65536) return fail(CODA_ERR_SHAPE, "T = %lld out of range", (long long)T);
  if (!(eps >= 0.f) || isinf(eps)) return fail(CODA_ERR_SHAPE, "eps must be finite and >= 0");
  if (M == 0) return ok();
  if (partials == nullptr || r == nullptr) return fail(CODA_ERR_NULL, "partials and r must be set");
  if ((((uintptr_t)partials | (uintptr_t)r) & 3) != 0) return fail(CODA_ERR_ALIGN, "partials / r not 4-byte aligned");
  const Mat mP{partials, T, M, M, 4, "partials"}, mr{r, 1, M, M, 4, "r"};
  if (mP.span() > kMaxSpan) return fail(CODA_ERR_SHAPE, "partials span too large");
  if (overlaps(mP, mr)) return fail(CODA_ERR_ALIAS, "r overlaps partials");
  return combine_impl((int)M, (int)D, (int)T, eps, partials, r, (hipStream_t)stream);
}

coda_status coda_gemm_rowscale(coda_dtype dt, int64_t M, int64_t D, int64_t N2, const void* X, int64_t ldx,
                               const void* W2, int64_t ldw2, const float* r, void* Y, int64_t ldy, void* stream) {
  coda_status st = check_dims(dt, M, {{"D", D}, {"N2", N2}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  const int es = elem_size(dt), E = elems_per_chunk(dt);
  const Mat mX{X, M, D, ldx, es, "X"}, mW2{W2, D, N2, ldw2, es, "W2"}, mY{Y, M, N2, ldy, es, "Y"};
  const Mat mr{r, 1, M, M, 4, "r"};
  for (const Mat* m : {&mX, &mW2, &mY})
    if ((st = check_mat(*m, E)) != CODA_OK) return st;
  if (r != nullptr && ((uintptr_t)r & 3) != 0) return fail(CODA_ERR_ALIGN, "r is not 4-byte aligned");
  const Mat ins[3] = {mX, mW2, r ? mr : Mat{nullptr, 0, 0, 0, 4, "r"}};
  if ((st = check_alias(&mY, 1, ins, 3)) != CODA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (dt == CODA_BF16) return gemm_rowscale_impl<uint16_t>((int)M, (int)D, (int)N2, X, ldx, W2, ldw2, r, Y, ldy, s);
  return gemm_rowscale_impl<float>((int)M, (int)D, (int)N2, X, ldx, W2, ldw2, r, Y, ldy, s);
}

int64_t coda_packed_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || rows > kMaxDim || cols < 1 || cols > kMaxDim || cols % 8 != 0) return -1;
  return packed_bytes(rows, cols);
}

coda_status coda_gemm_res_prms_packed(int64_t M, int64_t K, int64_t D, const void* A, int64_t lda, const void* W1,
                                      int64_t ldw1, const void* R, int64_t ldr, const void* g, void* H, int64_t ldh,
                                      void* Hgp, float* partials, void* stream) {
  coda_status st = check_dims(CODA_BF16, M, {{"K", K}, {"D", D}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  const int es = 2, E = 8;
  const int64_t T = num_partials(D);
  if (g == nullptr || Hgp == nullptr) return fail(CODA_ERR_NULL, "g and Hg must be set");
  const Mat mA{A, M, K, lda, es, "A"}, mW1{W1, K, D, ldw1, es, "W1"}, mR{R, M, D, ldr, es, "R"};
  const Mat mg{g, 1, D, D, es, "g"}, mH{H, M, D, ldh, es, "H"};
  const int64_t hg_elems = packed_bytes(M, D) / 2;
  const Mat mHg{Hgp, 1, hg_elems, hg_elems, es, "Hg"};  // the packed matrix as one flat row
  const Mat mP{partials, T, M, M, 4, "partials"};
  for (const Mat* m : {&mA, &mW1, &mR, &mH, &mg, &mHg})
    if ((st = check_mat(*m, E)) != CODA_OK) return st;
  if (partials == nullptr) return fail(CODA_ERR_NULL, "partials is NULL");
  if (((uintptr_t)partials & 3) != 0) return fail(CODA_ERR_ALIGN, "partials is not 4-byte aligned");
  if (mP.span() > kMaxSpan) return fail(CODA_ERR_SHAPE, "partials span too large");
  const Mat outs[3] = {mH, mHg, mP};
  const Mat ins[4] = {mA, mW1, mR, mg};
  if ((st = check_alias(outs, 3, ins, 4)) != CODA_OK) return st;
  return gemm_res_prms_packed_impl((int)M, (int)K, (int)D, A, lda, W1, ldw1, R, ldr, g, H, ldh, Hgp, partials,
                                   (hipStream_t)stream);
}

coda_status coda_gemm_rowscale_packed(int64_t M, int64_t D, int64_t N2, const void* Xp, const void* W2, int64_t ldw2,
                                      const float* r, void* Y, int64_t ldy, void* stream) {
  coda_status st = check_dims(CODA_BF16, M, {{"D", D}, {"N2", N2}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  const int es = 2, E = 8;
  const int64_t x_elems = packed_bytes(M, D) / 2;
  const Mat mX{Xp, 1, x_elems, x_elems, es, "X"}, mW2{W2, D, N2, ldw2, es, "W2"}, mY{Y, M, N2, ldy, es, "Y"};
  const Mat mr{r, 1, M, M, 4, "r"};
  for (const Mat* m : {&mX, &mW2, &mY})
    if ((st = check_mat(*m, E)) != CODA_OK) return st;
  if (r != nullptr && ((uintptr_t)r & 3) != 0) return fail(CODA_ERR_ALIGN, "r is not 4-byte aligned");
  const Mat ins[3] = {mX, mW2, r ? mr : Mat{nullptr, 0, 0, 0, 4, "r"}};
  if ((st = check_alias(&mY, 1, ins, 3)) != CODA_OK) return st;
  return gemm_rowscale_packed_impl((int)M, (int)D, (int)N2, Xp, W2, ldw2, r, Y, ldy, (hipStream_t)stream);
}

coda_status coda_gemm_rowscale_swiglu(coda_dtype dt, int64_t M, int64_t D, int64_t F, const void* X, int64_t ldx,
                                      const void* W2, int64_t ldw2, const float* r, void* Z, int64_t ldz, void* Y,
                                      int64_t ldy, void* stream) {
  coda_status st = check_dims(dt, M, {{"D", D}, {"F", F}});
  if (st != CODA_OK) return st;
  if (2 * F > kMaxDim) return fail(CODA_ERR_SHAPE, "2F = %lld out of range", (long long)(2 * F));
  if (F % kSwiGLURun != 0) return fail(CODA_ERR_SHAPE, "F = %lld is not a multiple of %d", (long long)F, kSwiGLURun);
  if (M == 0) return ok();
  const int es = elem_size(dt), E = elems_per_chunk(dt);
  const Mat mX{X, M, D, ldx, es, "X"}, mW2{W2, D, 2 * F, ldw2, es, "W2"}, mZ{Z, M, F, ldz, es, "Z"};
  const Mat mY{Y, M, 2 * F, ldy, es, "Y"}, mr{r, 1, M, M, 4, "r"};
  for (const Mat* m : {&mX, &mW2, &mZ})
    if ((st = check_mat(*m, E)) != CODA_OK) return st;
  if (Y != nullptr && (st = check_mat(mY, E)) != CODA_OK) return st;
  if (r != nullptr && ((uintptr_t)r & 3) != 0) return fail(CODA_ERR_ALIGN, "r is not 4-byte aligned");
  const Mat none{nullptr, 0, 0, 0, es, ""};
  const Mat outs[2] = {mZ, Y ? mY : none};
  const Mat ins[3] = {mX, mW2, r ? mr : none};
  if ((st = check_alias(outs, 2, ins, 3)) != CODA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (dt == CODA_BF16)
    return gemm_rowscale_swiglu_impl<uint16_t>((int)M, (int)D, (int)F, X, ldx, W2, ldw2, r, Z, ldz, Y, ldy, s);
  return gemm_rowscale_swiglu_impl<float>((int)M, (int)D, (int)F, X, ldx, W2, ldw2, r, Z, ldz, Y, ldy, s);
}

coda_status coda_gemm_rowscale_swiglu_packed(int64_t M, int64_t D, int64_t F, const void* Xp, const void* W2,
                                             int64_t ldw2, const float* r, void* Z, int64_t ldz, void* Y,
                                             int64_t ldy, void* stream) {
  coda_status st = check_dims(CODA_BF16, M, {{"D", D}, {"F", F}});
  if (st != CODA_OK) return st;
  if (2 * F > kMaxDim) return fail(CODA_ERR_SHAPE, "2F = %lld out of range", (long long)(2 * F));
  if (F % kSwiGLURun != 0) return fail(CODA_ERR_SHAPE, "F = %lld is not a multiple of %d", (long long)F, kSwiGLURun);
  if (M == 0) return ok();
  const int es = 2, E = 8;
  const int64_t x_elems = packed_bytes(M, D) / 2;
  const Mat mX{Xp, 1, x_elems, x_elems, es, "X"}, mW2{W2, D, 2 * F, ldw2, es, "W2"}, mZ{Z, M, F, ldz, es, "Z"};
  const Mat mY{Y, M, 2 * F, ldy, es, "Y"}, mr{r, 1, M, M, 4, "r"};
  for (const Mat* m : {&mX, &mW2, &mZ})
    if ((st = check_mat(*m, E)) != CODA_OK) return st;
  if (Y != nullptr && (st = check_mat(mY, E)) != CODA_OK) return st;
  if (r != nullptr && ((uintptr_t)r & 3) != 0) return fail(CODA_ERR_ALIGN, "r is not 4-byte aligned");
  const Mat none{nullptr, 0, 0, 0, es, ""};
  const Mat outs[2] = {mZ, Y ? mY : none};
  const Mat ins[3] = {mX, mW2, r ? mr : none};
  if ((st = check_alias(outs, 2, ins, 3)) != CODA_OK) return st;
  return gemm_rowscale_swiglu_packed_impl((int)M, (int)D, (int)F, Xp, W2, ldw2, r, Z, ldz, Y, ldy,
                                          (hipStream_t)stream);
}

coda_status coda_swiglu_bwd(coda_dtype dt, int64_t M, int64_t F, const void* dZ, int64_t ldz, const void* Y,
                            int64_t ldy, void* dY, int64_t lddy, void* stream) {
  coda_status st = check_dims(dt, M, {{"F", F}});
  if (st != CODA_OK) return st;
  if (2 * F > kMaxDim) return fail(CODA_ERR_SHAPE, "2F = %lld out of range", (long long)(2 * F));
  if (M == 0) return ok();
  const int es = elem_size(dt), E = elems_per_chunk(dt);
  const Mat mdZ{dZ, M, F, ldz, es, "dZ"}, mY{Y, M, 2 * F, ldy, es, "Y"}, mdY{dY, M, 2 * F, lddy, es, "dY"};
  for (const Mat* m : {&mdZ, &mY, &mdY})
    if ((st = check_mat(*m, E)) != CODA_OK) return st;
  const Mat ins[2] = {mdZ, mY};
  if ((st = check_alias(&mdY, 1, ins, 2)) != CODA_OK) return st;
  const int64_t nchunks = M * F / 8;
  const int blocks = (int)((nchunks + 255) / 256 < 16384 ? (nchunks + 255) / 256 : 16384);
  hipStream_t s = (hipStream_t)stream;
  if (dt == CODA_BF16)
    hipLaunchKernelGGL(swiglu_bwd_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, (const uint16_t*)dZ, ldz,
                       (const uint16_t*)Y, ldy, (uint16_t*)dY, lddy, (int)F, nchunks);
  else
    hipLaunchKernelGGL(swiglu_bwd_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)dZ, ldz,
                       (const float*)Y, ldy, (float*)dY, lddy, (int)F, nchunks);
  return launch_status("coda_swiglu_bwd");
}

coda_status coda_rope_cache(float* cos_sin, int64_t max_pos, int64_t d_head, double base, void* stream) {
  if (d_head < 2 || d_head > 4096 || d_head % 2 != 0)
    return fail(CODA_ERR_SHAPE, "d_head = %lld is not even in [2, 4096]", (long long)d_head);
  if (max_pos < 1 || max_pos > kMaxDim) return fail(CODA_ERR_SHAPE, "max_pos = %lld out of range", (long long)max_pos);
  if (!(base > 0.0) || isinf(base)) return fail(CODA_ERR_SHAPE, "base must be finite and > 0");
  if (cos_sin == nullptr) return fail(CODA_ERR_NULL, "cos_sin is NULL");
  if (((uintptr_t)cos_sin & 7) != 0) return fail(CODA_ERR_ALIGN, "cos_sin is not 8-byte aligned");
  if (max_pos * d_head * 4 > kMaxSpan) return fail(CODA_ERR_SHAPE, "cos_sin spans more than 2 GiB");
  const int64_t n = max_pos * (d_head / 2);
  hipLaunchKernelGGL(rope_cache_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, cos_sin,
                     n, (int)(d_head / 2), base);
  return launch_status("coda_rope_cache");
}

coda_status coda_gemm_rowscale_rope(coda_dtype dt, int64_t M, int64_t D, int64_t N2, const void* X, int64_t ldx,
                                    const void* W2, int64_t ldw2, const float* r, const int32_t* positions,
                                    const float* cos_sin, int64_t max_pos, int64_t n_q, int64_t n_k, int64_t d_head,
                                    void* Y, int64_t ldy, void* stream) {
  coda_status st = check_dims(dt, M, {{"D", D}, {"N2", N2}});
  if (st != CODA_OK) return st;
  Mat mpos, mcs;
  if ((st = check_rope(M, N2, positions, cos_sin, max_pos, n_q, n_k, d_head, &mpos, &mcs)) != CODA_OK) return st;
  if (M == 0) return ok();
  const int es = elem_size(dt), E = elems_per_chunk(dt);
  const Mat mX{X, M, D, ldx, es, "X"}, mW2{W2, D, N2, ldw2, es, "W2"}, mY{Y, M, N2, ldy, es, "Y"};
  const Mat mr{r, 1, M, M, 4, "r"};
  for (const Mat* m : {&mX, &mW2, &mY})
    if ((st = check_mat(*m, E)) != CODA_OK) return st;
  if (r != nullptr && ((uintptr_t)r & 3) != 0) return fail(CODA_ERR_ALIGN, "r is not 4-byte aligned");
  const Mat ins[5] = {mX, mW2, r ? mr : Mat{nullptr, 0, 0, 0, 4, "r"}, mpos, mcs};
  if ((st = check_alias(&mY, 1, ins, 5)) != CODA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const int nrot = (int)(n_q + n_k), mp = (int)max_pos, dh = (int)d_head;
  if (dt == CODA_BF16) {
    typename EpiRowScaleRope<uint16_t>::Params ep{r, positions, cos_sin, mp, nrot, dh, (uint16_t*)Y, ldy};
    return launch_gemm<uint16_t, true, false, EpiRowScaleRope<uint16_t>>("coda_gemm_rowscale_rope", (int)M, (int)N2,
                                                                         (int)D, X, ldx, W2, ldw2, ep, s);
  }
  typename EpiRowScaleRope<float>::Params ep{r, positions, cos_sin, mp, nrot, dh, (float*)Y, ldy};
  return launch_gemm<float, true, false, EpiRowScaleRope<float>>("coda_gemm_rowscale_rope", (int)M, (int)N2, (int)D,
                                                                 X, ldx, W2, ldw2, ep, s);
}

coda_status coda_rope_bwd(coda_dtype dt, int64_t M, int64_t N2, const void* dYr, int64_t ldg,
                          const int32_t* positions, const float* cos_sin, int64_t max_pos, int64_t n_q, int64_t n_k,
                          int64_t d_head, void* dY, int64_t lddy, void* stream) {
  coda_status st = check_dims(dt, M, {{"N2", N2}});
  if (st != CODA_OK) return st;
  Mat mpos, mcs;
  if ((st = check_rope(M, N2, positions, cos_sin, max_pos, n_q, n_k, d_head, &mpos, &mcs)) != CODA_OK) return st;
  if (M == 0) return ok();
  const int es = elem_size(dt), E = elems_per_chunk(dt);
  const Mat mG{dYr, M, N2, ldg, es, "dYr"}, mdY{dY, M, N2, lddy, es, "dY"};
  for (const Mat* m : {&mG, &mdY})
    if ((st = check_mat(*m, E)) != CODA_OK) return st;
  const Mat ins[3] = {mG, mpos, mcs};
  if ((st = check_alias(&mdY, 1, ins, 3)) != CODA_OK) return st;
  const int64_t nchunks = M * N2 / 8;
  const int blocks = (int)((nchunks + 255) / 256 < 16384 ? (nchunks + 255) / 256 : 16384);
  hipStream_t s = (hipStream_t)stream;
  const int nrot = (int)(n_q + n_k), mp = (int)max_pos, dh = (int)d_head;
  if (dt == CODA_BF16)
    hipLaunchKernelGGL(rope_bwd_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, (const uint16_t*)dYr, ldg, positions,
                       cos_sin, mp, nrot, dh, (uint16_t*)dY, lddy, (int)N2, nchunks);
  else
    hipLaunchKernelGGL(rope_bwd_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)dYr, ldg, positions,
                       cos_sin, mp, nrot, dh, (float*)dY, lddy, (int)N2, nchunks);
  return launch_status("coda_rope_bwd");
}

coda_status coda_gemm_res_prms_fp8(int64_t M, int64_t K, int64_t D, const void* A8, int64_t lda, const float* sa,
                                   const void* W1t8, int64_t ldw1t, const float* sw1, const void* R, int64_t ldr,
                                   const void* g, void* H, int64_t ldh, void* Hg8, int64_t ldhg, void* hg_exp,
                                   float* partials, void* stream) {
  coda_status st = check_dims_fp8(M, {{"K", K}, {"D", D}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  const int64_t T = num_partials(D);
  const int64_t eb = mx_exp_bytes(M, D);
  const Mat mA{A8, M, K, lda, 1, "A8"}, mW{W1t8, D, K, ldw1t, 1, "W1t8"}, mR{R, M, D, ldr, 2, "R"};
  const Mat mg{g, 1, D, D, 2, "g"}, mH{H, M, D, ldh, 2, "H"}, mHg{Hg8, M, D, ldhg, 1, "Hg8"};
  const Mat mP{partials, T, M, M, 4, "partials"}, msa{sa, 1, M, M, 4, "sa"}, msw{sw1, 1, D, D, 4, "sw1"};
  const Mat mE{hg_exp, 1, eb, eb, 1, "hg_exp"};
  for (const Mat* m : {&mA, &mW, &mHg})
    if ((st = check_mat(*m, 16)) != CODA_OK) return st;
  for (const Mat* m : {&mR, &mg, &mH})
    if ((st = check_mat(*m, 8)) != CODA_OK) return st;
  if ((st = check_mat(mE, 4)) != CODA_OK) return st;
  if ((st = check_vec(sa, M, 4, "sa")) != CODA_OK || (st = check_vec(sw1, D, 16, "sw1")) != CODA_OK) return st;
  if (partials == nullptr) return fail(CODA_ERR_NULL, "partials is NULL");
  if (((uintptr_t)partials & 3) != 0) return fail(CODA_ERR_ALIGN, "partials is not 4-byte aligned");
  if (mP.span() > kMaxSpan) return fail(CODA_ERR_SHAPE, "partials span too large");
  const Mat outs[4] = {mH, mHg, mP, mE};
  const Mat ins[6] = {mA, mW, mR, mg, msa, msw};
  if ((st = check_alias(outs, 4, ins, 6)) != CODA_OK) return st;
  EpiResPrmsFp8::Params ep{sa, sw1, (const uint16_t*)R, ldr, (const uint16_t*)g, (uint16_t*)H, ldh,
                           (uint8_t*)Hg8, ldhg, partials, 0, (uint8_t*)hg_exp};
  return launch_gemm_fp8<EpiResPrmsFp8>("coda_gemm_res_prms_fp8", (int)M, (int)D, (int)K, A8, lda, W1t8, ldw1t,
                                        ep, (hipStream_t)stream);
}

coda_status coda_quantize_rows_e4m3(int64_t M, int64_t K, const void* X, int64_t ldx, void* X8, int64_t ldx8,
                                    float* scales, void* stream) {
  coda_status st = check_dims_fp8(M, {{"K", K}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  const Mat mX{X, M, K, ldx, 2, "X"}, mX8{X8, M, K, ldx8, 1, "X8"}, ms{scales, 1, M, M, 4, "scales"};
  if ((st = check_mat(mX, 8)) != CODA_OK || (st = check_mat(mX8, 16)) != CODA_OK) return st;
  if (scales == nullptr) return fail(CODA_ERR_NULL, "scales is NULL");
  if (((uintptr_t)scales & 3) != 0) return fail(CODA_ERR_ALIGN, "scales is not 4-byte aligned");
  const Mat outs[2] = {mX8, ms};
  if ((st = check_alias(outs, 2, &mX, 1)) != CODA_OK) return st;
  q_rows(X, ldx, (int)M, (int)K, X8, ldx8, scales, (hipStream_t)stream);
  return launch_status("coda_quantize_rows_e4m3");
}

coda_status coda_quantize_cols_e4m3(int64_t K, int64_t N, const void* W, int64_t ldw, void* Wt8, int64_t ldwt,
                                    float* scales, void* stream) {
  coda_status st = check_dims_fp8(N, {{"K", K}});
  if (st != CODA_OK) return st;
  if (N == 0) return ok();
  if (N % 16 != 0) return fail(CODA_ERR_SHAPE, "N = %lld is not a multiple of 16", (long long)N);
  if (K > kMaxColRows) return fail(CODA_ERR_SHAPE, "K = %lld exceeds %lld rows", (long long)K, (long long)kMaxColRows);
  const Mat mW{W, K, N, ldw, 2, "W"}, mWt{Wt8, N, K, ldwt, 1, "Wt8"}, ms{scales, 1, N, N, 4, "scales"};
  if ((st = check_mat(mW, 8)) != CODA_OK || (st = check_mat(mWt, 16)) != CODA_OK) return st;
  if (scales == nullptr) return fail(CODA_ERR_NULL, "scales is NULL");
  if (((uintptr_t)scales & 3) != 0) return fail(CODA_ERR_ALIGN, "scales is not 4-byte aligned");
  const Mat outs[2] = {mWt, ms};
  if ((st = check_alias(outs, 2, &mW, 1)) != CODA_OK) return st;
  q_cols(W, ldw, (int)K, (int)N, Wt8, ldwt, scales, (hipStream_t)stream);
  return launch_status("coda_quantize_cols_e4m3");
}

coda_status coda_quantize_rows_cols_e4m3(int64_t M, int64_t N, const void* X, int64_t ldx, void* X8, int64_t ldx8,
                                         float* row_scales, void* Xt8, int64_t ldxt, float* col_scales,
                                         void* stream) {
  coda_status st = check_dims_fp8(M, {{"N", N}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  if (M % 16 != 0) return fail(CODA_ERR_SHAPE, "M = %lld is not a multiple of 16", (long long)M);
  if (M > kMaxColRows) return fail(CODA_ERR_SHAPE, "M = %lld exceeds %lld rows", (long long)M, (long long)kMaxColRows);
  const Mat mX{X, M, N, ldx, 2, "X"}, mX8{X8, M, N, ldx8, 1, "X8"}, mXt{Xt8, N, M, ldxt, 1, "Xt8"};
  const Mat msr{row_scales, 1, M, M, 4, "row_scales"}, msc{col_scales, 1, N, N, 4, "col_scales"};
  if ((st = check_mat(mX, 8)) != CODA_OK || (st = check_mat(mX8, 16)) != CODA_OK ||
      (st = check_mat(mXt, 16)) != CODA_OK)
    return st;
  if (row_scales == nullptr || col_scales == nullptr) return fail(CODA_ERR_NULL, "row_scales and col_scales must be set");
  if ((((uintptr_t)row_scales | (uintptr_t)col_scales) & 3) != 0)
    return fail(CODA_ERR_ALIGN, "row_scales / col_scales not 4-byte aligned");
  const Mat outs[4] = {mX8, msr, mXt, msc};
  if ((st = check_alias(outs, 4, &mX, 1)) != CODA_OK) return st;
  q_rows_cols(X, ldx, (int)M, (int)N, X8, ldx8, row_scales, Xt8, ldxt, col_scales, (hipStream_t)stream);
  return launch_status("coda_quantize_rows_cols_e4m3");
}

coda_status coda_gemm_rowscale_fp8(int64_t M, int64_t D, int64_t N2, const void* X8, int64_t ldx,
                                   const void* x_exp, const void* W2t8, int64_t ldw2t, const float* sw2,
                                   const float* r, void* Y, int64_t ldy, void* stream) {
  coda_status st = check_dims_fp8(M, {{"D", D}, {"N2", N2}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  const int64_t eb = mx_exp_bytes(M, D);
  const Mat mX{X8, M, D, ldx, 1, "X8"}, mW{W2t8, N2, D, ldw2t, 1, "W2t8"}, mY{Y, M, N2, ldy, 2, "Y"};
  const Mat mr{r, 1, M, M, 4, "r"}, msw{sw2, 1, N2, N2, 4, "sw2"}, mE{x_exp, 1, eb, eb, 1, "x_exp"};
  for (const Mat* m : {&mX, &mW})
    if ((st = check_mat(*m, 16)) != CODA_OK) return st;
  if ((st = check_mat(mY, 8)) != CODA_OK) return st;
  if (x_exp != nullptr && (st = check_mat(mE, 4)) != CODA_OK) return st;
  if ((st = check_vec(sw2, N2, 16, "sw2")) != CODA_OK) return st;
  if (r != nullptr && ((uintptr_t)r & 3) != 0) return fail(CODA_ERR_ALIGN, "r is not 4-byte aligned");
  const Mat none{nullptr, 0, 0, 0, 4, ""};
  const Mat ins[5] = {mX, mW, msw, r ? mr : none, x_exp ? mE : none};
  if ((st = check_alias(&mY, 1, ins, 5)) != CODA_OK) return st;
  EpiRowScaleFp8::Params ep{r, sw2, (uint16_t*)Y, ldy};
  if (x_exp != nullptr)
    return launch_gemm_fp8<EpiRowScaleFp8, kLayKC, kMxA>("coda_gemm_rowscale_fp8", (int)M, (int)N2, (int)D, X8, ldx,
                                                         W2t8, ldw2t, ep, (hipStream_t)stream, x_exp);
  return launch_gemm_fp8<EpiRowScaleFp8>("coda_gemm_rowscale_fp8", (int)M, (int)N2, (int)D, X8, ldx, W2t8, ldw2t,
                                         ep, (hipStream_t)stream);
}

int64_t coda_packed_bytes_e4m3(int64_t rows, int64_t cols) {
  if (rows < 0 || rows > kMaxDim || cols < 1 || cols > kMaxDim || cols % 16 != 0) return -1;
  return packed_bytes_e4m3(rows, cols);
}

coda_status coda_quantize_cols_e4m3_packed(int64_t K, int64_t N, const void* W, int64_t ldw, void* Wt8p,
                                           float* scales, void* stream) {
  coda_status st = check_dims_fp8(N, {{"K", K}});
  if (st != CODA_OK) return st;
  if (N == 0) return ok();
  if (N % 16 != 0) return fail(CODA_ERR_SHAPE, "N = %lld is not a multiple of 16", (long long)N);
  if (K > kMaxColRows) return fail(CODA_ERR_SHAPE, "K = %lld exceeds %lld rows", (long long)K, (long long)kMaxColRows);
  const int64_t wt_bytes = packed_bytes_e4m3(N, K);
  const Mat mW{W, K, N, ldw, 2, "W"}, mWt{Wt8p, 1, wt_bytes, wt_bytes, 1, "Wt8"}, ms{scales, 1, N, N, 4, "scales"};
  if ((st = check_mat(mW, 8)) != CODA_OK || (st = check_mat(mWt, 16)) != CODA_OK) return st;
  if (scales == nullptr) return fail(CODA_ERR_NULL, "scales is NULL");
  if (((uintptr_t)scales & 3) != 0) return fail(CODA_ERR_ALIGN, "scales is not 4-byte aligned");
  const Mat outs[2] = {mWt, ms};
  if ((st = check_alias(outs, 2, &mW, 1)) != CODA_OK) return st;
  q_cols(W, ldw, (int)K, (int)N, Wt8p, K, scales, (hipStream_t)stream, K / 16);
  return launch_status("coda_quantize_cols_e4m3_packed");
}

coda_status coda_quantize_rows_e4m3_packed(int64_t M, int64_t K, const void* X, int64_t ldx, void* X8p,
                                           float* scales, void* stream) {
  coda_status st = check_dims_fp8(M, {{"K", K}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  const int64_t x8_bytes = packed_bytes_e4m3(M, K);
  const Mat mX{X, M, K, ldx, 2, "X"}, mX8{X8p, 1, x8_bytes, x8_bytes, 1, "X8"}, ms{scales, 1, M, M, 4, "scales"};
  if ((st = check_mat(mX, 8)) != CODA_OK || (st = check_mat(mX8, 16)) != CODA_OK) return st;
  if (scales == nullptr) return fail(CODA_ERR_NULL, "scales is NULL");
  if (((uintptr_t)scales & 3) != 0) return fail(CODA_ERR_ALIGN, "scales is not 4-byte aligned");
  const Mat outs[2] = {mX8, ms};
  if ((st = check_alias(outs, 2, &mX, 1)) != CODA_OK) return st;
  q_rows(X, ldx, (int)M, (int)K, X8p, K, scales, (hipStream_t)stream, K / 16);
  return launch_status("coda_quantize_rows_e4m3_packed");
}

coda_status coda_quantize_rows_cols_e4m3_packed(int64_t M, int64_t N, const void* X, int64_t ldx, void* X8p,
                                                float* row_scales, void* Xt8p, float* col_scales, void* stream) {
  coda_status st = check_dims_fp8(M, {{"N", N}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  if (M % 16 != 0) return fail(CODA_ERR_SHAPE, "M = %lld is not a multiple of 16", (long long)M);
  if (M > kMaxColRows) return fail(CODA_ERR_SHAPE, "M = %lld exceeds %lld rows", (long long)M, (long long)kMaxColRows);
  const int64_t x8_bytes = packed_bytes_e4m3(M, N), xt_bytes = packed_bytes_e4m3(N, M);
  const Mat mX{X, M, N, ldx, 2, "X"}, mX8{X8p, 1, x8_bytes, x8_bytes, 1, "X8"}, mXt{Xt8p, 1, xt_bytes, xt_bytes, 1, "Xt8"};
  const Mat msr{row_scales, 1, M, M, 4, "row_scales"}, msc{col_scales, 1, N, N, 4, "col_scales"};
  if ((st = check_mat(mX, 8)) != CODA_OK || (st = check_mat(mX8, 16)) != CODA_OK ||
      (st = check_mat(mXt, 16)) != CODA_OK)
    return st;
  if (row_scales == nullptr || col_scales == nullptr) return fail(CODA_ERR_NULL, "row_scales and col_scales must be set");
  if ((((uintptr_t)row_scales | (uintptr_t)col_scales) & 3) != 0)
    return fail(CODA_ERR_ALIGN, "row_scales / col_scales not 4-byte aligned");
  const Mat outs[4] = {mX8, msr, mXt, msc};
  if ((st = check_alias(outs, 4, &mX, 1)) != CODA_OK) return st;
  q_rows_cols(X, ldx, (int)M, (int)N, X8p, N, row_scales, Xt8p, M, col_scales, (hipStream_t)stream, N / 16, M / 16);
  return launch_status("coda_quantize_rows_cols_e4m3_packed");
}

coda_status coda_quantize_mx_e4m3_packed(int64_t M, int64_t N, const void* X, int64_t ldx, void* Xr8p, void* Er,
                                         void* Xc8p, void* Ec, void* stream) {
  coda_status st = check_dims_fp8(M, {{"N", N}});
  if (st != CODA_OK) return st;
  if (M % 16 != 0) return fail(CODA_ERR_SHAPE, "M = %lld is not a multiple of 16", (long long)M);
  if ((N + 255) / 256 > 65535) return fail(CODA_ERR_SHAPE, "N = %lld exceeds %d columns", (long long)N, 65535 * 256);
  if ((Xr8p == nullptr) != (Er == nullptr) || (Xc8p == nullptr) != (Ec == nullptr))
    return fail(CODA_ERR_NULL, "codes and exponents come in pairs: Xr8p with Er, Xc8p with Ec");
  if (Xr8p == nullptr && Xc8p == nullptr) return fail(CODA_ERR_NULL, "no output: set Xr8p / Er or Xc8p / Ec");
  if (M == 0) return ok();
  const int64_t cb = packed_bytes_e4m3(M, N), erb = mx_exp_bytes(M, N), ecb = mx_exp_bytes(N, M);
  const Mat mX{X, M, N, ldx, 2, "X"};
  const Mat mr{Xr8p, 1, cb, cb, 1, "Xr8p"}, mer{Er, 1, erb, erb, 1, "Er"};
  const Mat mc{Xc8p, 1, cb, cb, 1, "Xc8p"}, mec{Ec, 1, ecb, ecb, 1, "Ec"};
  if ((st = check_mat(mX, 8)) != CODA_OK) return st;
  const Mat none{nullptr, 0, 0, 0, 1, ""};
  Mat outs[4] = {none, none, none, none};
  if (Xr8p != nullptr) {
    if ((st = check_mat(mr, 16)) != CODA_OK || (st = check_mat(mer, 16)) != CODA_OK) return st;
    outs[0] = mr;
    outs[1] = mer;
  }
  if (Xc8p != nullptr) {
    if ((st = check_mat(mc, 16)) != CODA_OK || (st = check_mat(mec, 16)) != CODA_OK) return st;
    outs[2] = mc;
    outs[3] = mec;
  }
  if ((st = check_alias(outs, 4, &mX, 1)) != CODA_OK) return st;
  q_mx(X, ldx, (int)M, (int)N, Xr8p, Er, Xc8p, Ec, (hipStream_t)stream);
  return launch_status("coda_quantize_mx_e4m3_packed");
}

coda_status coda_gemm_res_prms_fp8_packed(int64_t M, int64_t K, int64_t D, const void* A8, int64_t lda,
                                          const float* sa, const void* W1t8, int64_t ldw1t, const float* sw1,
                                          const void* R, int64_t ldr, const void* g, void* H, int64_t ldh,
                                          void* Hg8p, void* hg_exp, float* partials, void* stream) {
  coda_status st = check_dims_fp8(M, {{"K", K}, {"D", D}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  const int64_t T = num_partials(D);
  const int64_t hg_bytes = packed_bytes_e4m3(M, D), eb = mx_exp_bytes(M, D);
  const Mat mA{A8, M, K, lda, 1, "A8"}, mW{W1t8, D, K, ldw1t, 1, "W1t8"}, mR{R, M, D, ldr, 2, "R"};
  const Mat mg{g, 1, D, D, 2, "g"}, mH{H, M, D, ldh, 2, "H"}, mHg{Hg8p, 1, hg_bytes, hg_bytes, 1, "Hg8"};
  const Mat mP{partials, T, M, M, 4, "partials"}, msa{sa, 1, M, M, 4, "sa"}, msw{sw1, 1, D, D, 4, "sw1"};
  const Mat mE{hg_exp, 1, eb, eb, 1, "hg_exp"};
  for (const Mat* m : {&mA, &mW, &mHg})
    if ((st = check_mat(*m, 16)) != CODA_OK) return st;
  for (const Mat* m : {&mR, &mg, &mH})
    if ((st = check_mat(*m, 8)) != CODA_OK) return st;
  if ((st = check_mat(mE, 4)) != CODA_OK) return st;
  if ((st = check_vec(sa, M, 4, "sa")) != CODA_OK || (st = check_vec(sw1, D, 16, "sw1")) != CODA_OK) return st;
  if (partials == nullptr) return fail(CODA_ERR_NULL, "partials is NULL");
  if (((uintptr_t)partials & 3) != 0) return fail(CODA_ERR_ALIGN, "partials is not 4-byte aligned");
  if (mP.span() > kMaxSpan) return fail(CODA_ERR_SHAPE, "partials span too large");
  const Mat outs[4] = {mH, mHg, mP, mE};
  const Mat ins[6] = {mA, mW, mR, mg, msa, msw};
  if ((st = check_alias(outs, 4, ins, 6)) != CODA_OK) return st;
  EpiResPrmsFp8::Params ep{sa, sw1, (const uint16_t*)R, ldr, (const uint16_t*)g, (uint16_t*)H, ldh,
                           (uint8_t*)Hg8p, 0, partials, D / 16, (uint8_t*)hg_exp};
  return launch_gemm_fp8<EpiResPrmsFp8>("coda_gemm_res_prms_fp8_packed", (int)M, (int)D, (int)K, A8, lda, W1t8,
                                        ldw1t, ep, (hipStream_t)stream);
}

coda_status coda_gemm_res_prms_fp8_all_packed(int64_t M, int64_t K, int64_t D, const void* A8p, const float* sa,
                                              const void* W1t8p, const float* sw1, const void* R, int64_t ldr,
                                              const void* g, void* H, int64_t ldh, void* Hg8p, void* hg_exp,
                                              float* partials, void* stream) {
  coda_status st = check_dims_fp8(M, {{"K", K}, {"D", D}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  const int64_t T = num_partials(D);
  const int64_t a_bytes = packed_bytes_e4m3(M, K), w_bytes = packed_bytes_e4m3(D, K);
  const int64_t hg_bytes = packed_bytes_e4m3(M, D), eb = mx_exp_bytes(M, D);
  const Mat mA{A8p, 1, a_bytes, a_bytes, 1, "A8p"}, mW{W1t8p, 1, w_bytes, w_bytes, 1, "W1t8p"};
  const Mat mR{R, M, D, ldr, 2, "R"}, mg{g, 1, D, D, 2, "g"}, mH{H, M, D, ldh, 2, "H"};
  const Mat mHg{Hg8p, 1, hg_bytes, hg_bytes, 1, "Hg8"}, mE{hg_exp, 1, eb, eb, 1, "hg_exp"};
  const Mat mP{partials, T, M, M, 4, "partials"}, msa{sa, 1, M, M, 4, "sa"}, msw{sw1, 1, D, D, 4, "sw1"};
  for (const Mat* m : {&mA, &mW, &mHg})
    if ((st = check_mat(*m, 16)) != CODA_OK) return st;
  for (const Mat* m : {&mR, &mg, &mH})
    if ((st = check_mat(*m, 8)) != CODA_OK) return st;
  if ((st = check_mat(mE, 4)) != CODA_OK) return st;
  if ((st = check_vec(sa, M, 4, "sa")) != CODA_OK || (st = check_vec(sw1, D, 16, "sw1")) != CODA_OK) return st;
  if (partials == nullptr) return fail(CODA_ERR_NULL, "partials is NULL");
  if (((uintptr_t)partials & 3) != 0) return fail(CODA_ERR_ALIGN, "partials is not 4-byte aligned");
  if (mP.span() > kMaxSpan) return fail(CODA_ERR_SHAPE, "partials span too large");
  const Mat outs[4] = {mH, mHg, mP, mE};
  const Mat ins[6] = {mA, mW, mR, mg, msa, msw};
  if ((st = check_alias(outs, 4, ins, 6)) != CODA_OK) return st;
  EpiResPrmsFp8::Params ep{sa, sw1, (const uint16_t*)R, ldr, (const uint16_t*)g, (uint16_t*)H, ldh,
                           (uint8_t*)Hg8p, 0, partials, D / 16, (uint8_t*)hg_exp};
  return launch_gemm_fp8<EpiResPrmsFp8, kLayPacked>("coda_gemm_res_prms_fp8_all_packed", (int)M, (int)D, (int)K,
                                                    A8p, K / 16, W1t8p, K / 16, ep, (hipStream_t)stream);
}

coda_status coda_gemm_rowscale_fp8_packed(int64_t M, int64_t D, int64_t N2, const void* X8p, const void* x_exp,
                                          const void* W2t8p, const float* sw2, const float* r, void* Y, int64_t ldy,
                                          void* stream) {
  coda_status st = check_dims_fp8(M, {{"D", D}, {"N2", N2}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  const int64_t x_bytes = packed_bytes_e4m3(M, D), w_bytes = packed_bytes_e4m3(N2, D), eb = mx_exp_bytes(M, D);
  const Mat mX{X8p, 1, x_bytes, x_bytes, 1, "X8"}, mW{W2t8p, 1, w_bytes, w_bytes, 1, "W2t8"};
  const Mat mY{Y, M, N2, ldy, 2, "Y"}, mr{r, 1, M, M, 4, "r"}, msw{sw2, 1, N2, N2, 4, "sw2"};
  const Mat mE{x_exp, 1, eb, eb, 1, "x_exp"};
  for (const Mat* m : {&mX, &mW})
    if ((st = check_mat(*m, 16)) != CODA_OK) return st;
  if ((st = check_mat(mY, 8)) != CODA_OK) return st;
  if (x_exp != nullptr && (st = check_mat(mE, 4)) != CODA_OK) return st;
  if ((st = check_vec(sw2, N2, 16, "sw2")) != CODA_OK) return st;
  if (r != nullptr && ((uintptr_t)r & 3) != 0) return fail(CODA_ERR_ALIGN, "r is not 4-byte aligned");
  const Mat none{nullptr, 0, 0, 0, 4, ""};
  const Mat ins[5] = {mX, mW, msw, r ? mr : none, x_exp ? mE : none};
  if ((st = check_alias(&mY, 1, ins, 5)) != CODA_OK) return st;
  EpiRowScaleFp8::Params ep{r, sw2, (uint16_t*)Y, ldy};
  if (x_exp != nullptr)
    return launch_gemm_fp8<EpiRowScaleFp8, kLayPacked, kMxA>("coda_gemm_rowscale_fp8_packed", (int)M, (int)N2,
                                                             (int)D, X8p, D / 16, W2t8p, D / 16, ep,
                                                             (hipStream_t)stream, x_exp);
  return launch_gemm_fp8<EpiRowScaleFp8, kLayPacked>("coda_gemm_rowscale_fp8_packed", (int)M, (int)N2, (int)D, X8p,
                                                     D / 16, W2t8p, D / 16, ep, (hipStream_t)stream);
}

int64_t coda_mx_exp_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || rows > kMaxDim || cols < 1 || cols > kMaxDim) return -1;
  return mx_exp_bytes(rows, cols);
}

coda_status coda_gemm_rowscale_lse(coda_dtype dt, int64_t M, int64_t D, int64_t V, const void* X, int64_t ldx,
                                   const void* Wv, int64_t ldw, const float* r, const int32_t* targets, float* pmax,
                                   float* psum, float* tgt, void* stream) {
  coda_status st = check_dims(dt, M, {{"D", D}, {"V", V}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  const int es = elem_size(dt), E = elems_per_chunk(dt);
  const int64_t T = num_partials(V);
  const Mat mX{X, M, D, ldx, es, "X"}, mW{Wv, D, V, ldw, es, "Wv"};
  for (const Mat* m : {&mX, &mW})
    if ((st = check_mat(*m, E)) != CODA_OK) return st;
  if (targets == nullptr || pmax == nullptr || psum == nullptr || tgt == nullptr)
    return fail(CODA_ERR_NULL, "targets, pmax, psum and tgt must be set");
  if ((((uintptr_t)targets | (uintptr_t)pmax | (uintptr_t)psum | (uintptr_t)tgt) & 3) != 0 ||
      (r != nullptr && ((uintptr_t)r & 3) != 0))
    return fail(CODA_ERR_ALIGN, "r, targets, pmax, psum and tgt must be 4-byte aligned");
  const Mat mpm{pmax, T, M, M, 4, "pmax"}, mps{psum, T, M, M, 4, "psum"}, mtg{tgt, 1, M, M, 4, "tgt"};
  const Mat mt{targets, 1, M, M, 4, "targets"}, mr{r, 1, M, M, 4, "r"};
  if (mpm.span() > kMaxSpan) return fail(CODA_ERR_SHAPE, "pmax span too large");
  const Mat none{nullptr, 0, 0, 0, 4, ""};
  const Mat outs[3] = {mpm, mps, mtg};
  const Mat ins[4] = {mX, mW, mt, r ? mr : none};
  if ((st = check_alias(outs, 3, ins, 4)) != CODA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (dt == CODA_BF16) {
    typename EpiLSE<uint16_t>::Params ep{r, targets, pmax, psum, tgt};
    return launch_gemm<uint16_t, true, false, EpiLSE<uint16_t>>("coda_gemm_rowscale_lse", (int)M, (int)V, (int)D,
                                                                X, ldx, Wv, ldw, ep, s);
  }
  typename EpiLSE<float>::Params ep{r, targets, pmax, psum, tgt};
  return launch_gemm<float, true, false, EpiLSE<float>>("coda_gemm_rowscale_lse", (int)M, (int)V, (int)D, X, ldx,
                                                        Wv, ldw, ep, s);
}

coda_status coda_gemm_rowscale_ce_bwd(coda_dtype dt, int64_t M, int64_t D, int64_t V, const void* X, int64_t ldx,
                                      const void* Wv, int64_t ldw, const float* r, const int32_t* targets,
                                      const float* lse, const float* dloss, void* dY, int64_t lddy, void* stream) {
  coda_status st = check_dims(dt, M, {{"D", D}, {"V", V}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  const int es = elem_size(dt), E = elems_per_chunk(dt);
  const Mat mX{X, M, D, ldx, es, "X"}, mW{Wv, D, V, ldw, es, "Wv"}, mdY{dY, M, V, lddy, es, "dY"};
  for (const Mat* m : {&mX, &mW, &mdY})
    if ((st = check_mat(*m, E)) != CODA_OK) return st;
  if (targets == nullptr || lse == nullptr || dloss == nullptr)
    return fail(CODA_ERR_NULL, "targets, lse and dloss must be set");
  if ((((uintptr_t)targets | (uintptr_t)lse | (uintptr_t)dloss) & 3) != 0 || (r != nullptr && ((uintptr_t)r & 3) != 0))
    return fail(CODA_ERR_ALIGN, "r, targets, lse and dloss must be 4-byte aligned");
  const Mat mt{targets, 1, M, M, 4, "targets"}, ml{lse, 1, M, M, 4, "lse"}, md{dloss, 1, M, M, 4, "dloss"};
  const Mat mr{r, 1, M, M, 4, "r"};
  const Mat ins[6] = {mX, mW, mt, ml, md, r ? mr : Mat{nullptr, 0, 0, 0, 4, "r"}};
  if ((st = check_alias(&mdY, 1, ins, 6)) != CODA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (dt == CODA_BF16) {
    typename EpiCEGrad<uint16_t>::Params ep{r, targets, lse, dloss, (uint16_t*)dY, lddy, (int)V};
    return launch_gemm<uint16_t, true, false, EpiCEGrad<uint16_t>>("coda_gemm_rowscale_ce_bwd", (int)M, (int)V,
                                                                   (int)D, X, ldx, Wv, ldw, ep, s);
  }
  typename EpiCEGrad<float>::Params ep{r, targets, lse, dloss, (float*)dY, lddy, (int)V};
  return launch_gemm<float, true, false, EpiCEGrad<float>>("coda_gemm_rowscale_ce_bwd", (int)M, (int)V, (int)D, X,
                                                           ldx, Wv, ldw, ep, s);
}

coda_status coda_gemm_rowscale_rope_packed(int64_t M, int64_t D, int64_t N2, const void* Xp, const void* W2,
                                           int64_t ldw2, const float* r, const int32_t* positions,
                                           const float* cos_sin, int64_t max_pos, int64_t n_q, int64_t n_k,
                                           int64_t d_head, void* Y, int64_t ldy, void* stream) {
  coda_status st = check_dims(CODA_BF16, M, {{"D", D}, {"N2", N2}});
  if (st != CODA_OK) return st;
  Mat mpos, mcs;
  if ((st = check_rope(M, N2, positions, cos_sin, max_pos, n_q, n_k, d_head, &mpos, &mcs)) != CODA_OK) return st;
  if (M == 0) return ok();
  const int es = 2, E = 8;
  const int64_t x_elems = packed_bytes(M, D) / 2;
  const Mat mX{Xp, 1, x_elems, x_elems, es, "X"}, mW2{W2, D, N2, ldw2, es, "W2"}, mY{Y, M, N2, ldy, es, "Y"};
  const Mat mr{r, 1, M, M, 4, "r"};
  for (const Mat* m : {&mX, &mW2, &mY})
    if ((st = check_mat(*m, E)) != CODA_OK) return st;
  if (r != nullptr && ((uintptr_t)r & 3) != 0) return fail(CODA_ERR_ALIGN, "r is not 4-byte aligned");
  const Mat ins[5] = {mX, mW2, r ? mr : Mat{nullptr, 0, 0, 0, 4, "r"}, mpos, mcs};
  if ((st = check_alias(&mY, 1, ins, 5)) != CODA_OK) return st;
  typename EpiRowScaleRope<uint16_t>::Params ep{r, positions, cos_sin, (int)max_pos, (int)(n_q + n_k), (int)d_head,
                                                (uint16_t*)Y, ldy};
  return launch_gemm<uint16_t, true, false, EpiRowScaleRope<uint16_t>, kLayPacked>(
      "coda_gemm_rowscale_rope_packed", (int)M, (int)N2, (int)D, Xp, D / 8, W2, ldw2, ep, (hipStream_t)stream);
}

coda_status coda_gemm_rowscale_lse_packed(int64_t M, int64_t D, int64_t V, const void* Xp, const void* Wv,
                                          int64_t ldw, const float* r, const int32_t* targets, float* pmax,
                                          float* psum, float* tgt, void* stream) {
  coda_status st = check_dims(CODA_BF16, M, {{"D", D}, {"V", V}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  const int es = 2, E = 8;
  const int64_t T = num_partials(V), x_elems = packed_bytes(M, D) / 2;
  const Mat mX{Xp, 1, x_elems, x_elems, es, "X"}, mW{Wv, D, V, ldw, es, "Wv"};
  for (const Mat* m : {&mX, &mW})
    if ((st = check_mat(*m, E)) != CODA_OK) return st;
  if (targets == nullptr || pmax == nullptr || psum == nullptr || tgt == nullptr)
    return fail(CODA_ERR_NULL, "targets, pmax, psum and tgt must be set");
  if ((((uintptr_t)targets | (uintptr_t)pmax | (uintptr_t)psum | (uintptr_t)tgt) & 3) != 0 ||
      (r != nullptr && ((uintptr_t)r & 3) != 0))
    return fail(CODA_ERR_ALIGN, "r, targets, pmax, psum and tgt must be 4-byte aligned");
  const Mat mpm{pmax, T, M, M, 4, "pmax"}, mps{psum, T, M, M, 4, "psum"}, mtg{tgt, 1, M, M, 4, "tgt"};
  const Mat mt{targets, 1, M, M, 4, "targets"}, mr{r, 1, M, M, 4, "r"};
  if (mpm.span() > kMaxSpan) return fail(CODA_ERR_SHAPE, "pmax span too large");
  const Mat none{nullptr, 0, 0, 0, 4, ""};
  const Mat outs[3] = {mpm, mps, mtg};
  const Mat ins[4] = {mX, mW, mt, r ? mr : none};
  if ((st = check_alias(outs, 3, ins, 4)) != CODA_OK) return st;
  typename EpiLSE<uint16_t>::Params ep{r, targets, pmax, psum, tgt};
  return launch_gemm<uint16_t, true, false, EpiLSE<uint16_t>, kLayPacked>("coda_gemm_rowscale_lse_packed", (int)M, (int)V,
                                                                    (int)D, Xp, D / 8, Wv, ldw, ep,
                                                                    (hipStream_t)stream);
}

coda_status coda_gemm_rowscale_ce_bwd_packed(int64_t M, int64_t D, int64_t V, const void* Xp, const void* Wv,
                                             int64_t ldw, const float* r, const int32_t* targets, const float* lse,
                                             const float* dloss, void* dY, int64_t lddy, void* stream) {
  coda_status st = check_dims(CODA_BF16, M, {{"D", D}, {"V", V}});
  if (st != CODA_OK) return st;
  if (M == 0) return ok();
  const int es = 2, E = 8;
  const int64_t x_elems = packed_bytes(M, D) / 2;
  const Mat mX{Xp, 1, x_elems, x_elems, es, "X"}, mW{Wv, D, V, ldw, es, "Wv"}, mdY{dY, M, V, lddy, es, "dY"};
  for (const Mat* m : {&mX, &mW, &mdY})
    if ((st = check_mat(*m, E)) != CODA_OK) return st;
  if (targets == nullptr || lse == nullptr || dloss == nullptr)
    return fail(CODA_ERR_NULL, "targets, lse and dloss must be set");
  if ((((uintptr_t)targets | (uintptr_t)lse | (uintptr_t)dloss) & 3) != 0 || (r != nullptr && ((uintptr_t)r & 3) != 0))
    return fail(CODA_ERR_ALIGN, "r, targets, lse and dloss must be 4-byte aligned");
  const Mat mt{targets, 1, M, M, 4, "targets"}, ml{lse, 1, M, M, 4, "lse"}, md{dloss, 1, M, M, 4, "dloss"};
  const Mat mr{r, 1, M, M, 4, "r"};
  const Mat ins[6] = {mX, mW, mt, ml, md, r ? mr : Mat{nullptr, 0, 0, 0, 4, "r"}};
  if ((st = check_alias(&mdY, 1, ins, 6)) != CODA_OK) return st;
  typename EpiCEGrad<uint16_t>::Params ep{r, targets, lse, dloss, (uint16_t*)dY, lddy, (int)V};
  return launch_gemm<uint16_t, true, false, EpiCEGrad<uint16_t>, kLayPacked>("coda_gemm_rowscale_ce_bwd_packed", (int)M,
                                                                       (int)V, (int)D, Xp, D / 8, Wv, ldw, ep,
                                                                       (hipStream_t)stream);
}

coda_status coda_ce_combine(int64_t M, int64_t V, int64_t T, const float* pmax, const float* psum, const float* tgt,
                            const int32_t* targets, float* lse, float* loss, void* stream) {
  if (M < 0 || M > kMaxDim) return fail(CODA_ERR_SHAPE, "M = %lld out of range", (long long)M);
  if (V < 1 || V > kMaxDim) return fail(CODA_ERR_SHAPE, "V = %lld out of range", (long long)V);
  if (T < 1 || T > 65536) return fail(CODA_ERR_SHAPE, "T = %lld out of range", (long long)T);
  if (M == 0) return ok();
  if (!pmax || !psum || !tgt || !targets || !lse || !loss) return fail(CODA_ERR_NULL, "a pointer is NULL");
  if ((((uintptr_t)pmax | (uintptr_t)psum | (uintptr_t)tgt | (uintptr_t)targets | (uintptr_t)lse |
        (uintptr_t)loss) & 3) != 0)
    return fail(CODA_ERR_ALIGN, "arrays must be 4-byte aligned");
  const Mat mpm{pmax, T, M, M, 4, "pmax"}, mps{psum, T, M, M, 4, "psum"}, mtg{tgt, 1, M, M, 4, "tgt"};
  const Mat mt{targets, 1, M, M, 4, "targets"}, ml{lse, 1, M, M, 4, "lse"}, mlo{loss, 1, M, M, 4, "loss"};
  if (mpm.span() > kMaxSpan) return fail(CODA_ERR_SHAPE, "pmax span too large");
  const Mat outs[2] = {ml, mlo};
  const Mat ins[4] = {mpm, mps, mtg, mt};
  coda_status st;
  if ((st = check_alias(outs, 2, ins, 4)) != CODA_OK) return st;
  hipLaunchKernelGGL(ce_combine_kernel, dim3((unsigned)((M + 63) / 64)), dim3(256), 0, (hipStream_t)stream, pmax, psum,
                     tgt, targets, lse, loss, (int)M, (int)T, (int)V);
  return launch_status("coda_ce_combine");
}

size_t coda_ref_chain_workspace_bytes(coda_dtype dt, int64_t M, int64_t D) {
  if ((dt != CODA_BF16 && dt != CODA_F32) || M < 0 || D < 1) return 0;
  const size_t c = (size_t)M * D * 4;
  const size_t c_aligned = (c + 255) & ~(size_t)255;
  return c_aligned + (size_t)M * D * elem_size(dt);
}

coda_status coda_ref_chain(coda_dtype dt, int64_t M, int64_t K, int64_t D, int64_t N2, float eps, const void* A,
                           const void* W1, const void* R, const void* g, const void* W2, void* H, float* r, void* Y,
                           void* ws, size_t ws_bytes, void* stream) {
  coda_status st = check_dims(dt, M, {{"K", K}, {"D", D}, {"N2", N2}});
  if (st != CODA_OK) return st;
  if (!(eps >= 0.f) || isinf(eps)) return fail(CODA_ERR_SHAPE, "eps must be finite and >= 0");
  if (M == 0) return ok();
  const int es = elem_size(dt), E = elems_per_chunk(dt);
  const Mat mA{A, M, K, K, es, "A"}, mW1{W1, K, D, D, es, "W1"}, mR{R, M, D, D, es, "R"}, mg{g, 1, D, D, es, "g"};
  const Mat mW2{W2, D, N2, N2, es, "W2"}, mH{H, M, D, D, es, "H"}, mY{Y, M, N2, N2, es, "Y"};
  const Mat mr{r, 1, M, M, 4, "r"};
  for (const Mat* m : {&mA, &mW1, &mR, &mg, &mW2, &mH, &mY})
    if ((st = check_mat(*m, E)) != CODA_OK) return st;
  if (r == nullptr) return fail(CODA_ERR_NULL, "r is NULL");
  if (((uintptr_t)r & 3) != 0) return fail(CODA_ERR_ALIGN, "r is not 4-byte aligned");
  const size_t need = coda_ref_chain_workspace_bytes(dt, M, D);
  if (ws == nullptr || ws_bytes < need)
    return fail(CODA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  if (((uintptr_t)ws & 255) != 0) return fail(CODA_ERR_ALIGN, "workspace must be 256-byte aligned");
  const size_t c_aligned = ((size_t)M * D * 4 + 255) & ~(size_t)255;
  float* C = (float*)ws;
  void* Xn = (char*)ws + c_aligned;
  const Mat mC{C, M, D, D, 4, "workspace C"}, mXn{Xn, M, D, D, es, "workspace Xn"};
  if (mC.span() > kMaxSpan) return fail(CODA_ERR_SHAPE, "workspace C spans more than 2 GiB");
  const Mat outs[5] = {mH, mr, mY, mC, mXn};
  const Mat ins[5] = {mA, mW1, mR, mg, mW2};
  if ((st = check_alias(outs, 5, ins, 5)) != CODA_OK) return st;

  hipStream_t s = (hipStream_t)stream;
  const int64_t nchunks = M * D / 8;
  const int ew_blocks = (int)((nchunks + 255) / 256 < 16384 ? (nchunks + 255) / 256 : 16384);
  if (dt == CODA_BF16) {
    typedef uint16_t T;
    if ((st = launch_gemm<T, true, false, EpiStoreF32>("coda_ref_chain gemm1", (int)M, (int)D, (int)K, A, K, W1, D,
                                                        EpiStoreF32::Params{C, D}, s)) != CODA_OK)
      return st;
    hipLaunchKernelGGL(residual_add_kernel<T>, dim3(ew_blocks), dim3(256), 0, s, C, (const T*)R, (T*)H, nchunks);
    if ((st = launch_status("coda_ref_chain residual")) != CODA_OK) return st;
    hipLaunchKernelGGL(rmsnorm_rows_kernel<T>, dim3((unsigned)M), dim3(256), 0, s, (const T*)H, (const T*)g, r,
                       (T*)Xn, (int)D, eps);
    if ((st = launch_status("coda_ref_chain rmsnorm")) != CODA_OK) return st;
    return gemm_rowscale_impl<T>((int)M, (int)D, (int)N2, Xn, D, W2, N2, nullptr, Y, N2, s);
  } else {
    typedef float T;
    if ((st = launch_gemm<T, true, false, EpiStoreF32>("coda_ref_chain gemm1", (int)M, (int)D, (int)K, A, K, W1, D,
                                                        EpiStoreF32::Params{C, D}, s)) != CODA_OK)
      return st;
    hipLaunchKernelGGL(residual_add_kernel<T>, dim3(ew_blocks), dim3(256), 0, s, C, (const T*)R, (T*)H, nchunks);
    if ((st = launch_status("coda_ref_chain residual")) != CODA_OK) return st;
    hipLaunchKernelGGL(rmsnorm_rows_kernel<T>, dim3((unsigned)M), dim3(256), 0, s, (const T*)H, (const T*)g, r,
                       (T*)Xn, (int)D, eps);
    if ((st = launch_status("coda_ref_chain rmsnorm")) != CODA_OK) return st;
    return gemm_rowscale_impl<T>((int)M, (int)D, (int)N2, Xn, D, W2, N2, nullptr, Y, N2, s);
  }
}

size_t coda_chain_bwd_workspace_bytes(coda_dtype dt, int64_t M, int64_t K, int64_t D, int64_t N2) {
  if (dt != CODA_BF16 && dt != CODA_F32) return 0;
  if (M < 0 || M > kMaxDim || K < 1 || K > kMaxDim || D < 1 || D > kMaxDim || N2 < 1 || N2 > kMaxDim) return 0;
  return BwdWs(M, K, D, N2, elem_size(dt)).total;
}

coda_status coda_chain_bwd(coda_dtype dt, int64_t M, int64_t K, int64_t D, int64_t N2, const void* dY,
                           const void* A, const void* W1, const void* g, const void* W2, const void* H,
                           const float* r, void* dA, void* dR, void* dW1, void* dW2, float* dg, void* ws,
                           size_t ws_bytes, void* stream) {
  coda_status st = check_bwd_args(dt, M, K, D, N2, dY, A, W1, g, W2, H, r, dA, dR, dW1, dW2, dg);
  if (st != CODA_OK) return st;
  const int es = elem_size(dt);
  const BwdWs L(M, K, D, N2, es);
  if (ws == nullptr || ws_bytes < L.total)
    return fail(CODA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, ws ? ws_bytes : (size_t)0);
  if (((uintptr_t)ws & (kWsAlign - 1)) != 0) return fail(CODA_ERR_ALIGN, "workspace must be 256-byte aligned");
  const Mat mws{ws, 1, (int64_t)L.total, (int64_t)L.total, 1, "workspace"};
  const Mat mXn{(char*)ws + L.xn, M, D, D, es, "workspace X_n"};
  if (mXn.span() > kMaxSpan) return fail(CODA_ERR_SHAPE, "workspace X_n spans more than 2 GiB");
  if ((st = check_bwd_alias(dt, M, K, D, N2, dY, A, W1, g, W2, H, r, dA, dR, dW1, dW2, dg, mws)) != CODA_OK)
    return st;
  hipStream_t s = (hipStream_t)stream;
  if (dt == CODA_BF16)
    return chain_bwd_impl<uint16_t>((int)M, (int)K, (int)D, (int)N2, dY, A, W1, g, W2, H, r, dA, dR, dW1, dW2, dg,
                                    (char*)ws, s);
  return chain_bwd_impl<float>((int)M, (int)K, (int)D, (int)N2, dY, A, W1, g, W2, H, r, dA, dR, dW1, dW2, dg,
                               (char*)ws, s);
}

coda_status coda_chain_bwd_noalloc(coda_dtype dt, int64_t M, int64_t K, int64_t D, int64_t N2, const void* dY,
                                   const void* A, const void* W1, const void* g, const void* W2, const void* H,
                                   const float* r, void* dA, void* dR, void* dW1, void* dW2, float* dg,
                                   void* stream) {
  coda_status st = check_bwd_args(dt, M, K, D, N2, dY, A, W1, g, W2, H, r, dA, dR, dW1, dW2, dg);
  if (st != CODA_OK) return st;
  const size_t need = BwdWs(M, 0, D, 0, elem_size(dt)).total;
  if (need > kNoAllocScratchBytes)
    return fail(CODA_ERR_WORKSPACE, "this shape needs %zu bytes of scratch; the static scratch holds %zu "
                "(M * D elements of X_n dominate): use coda_chain_bwd with a workspace",
                need, kNoAllocScratchBytes);
  const Mat none{nullptr, 0, 0, 0, 1, ""};
  if ((st = check_bwd_alias(dt, M, K, D, N2, dY, A, W1, g, W2, H, r, dA, dR, dW1, dW2, dg, none)) != CODA_OK)
    return st;
  char* ws = nullptr;
  if ((st = noalloc_scratch(&ws)) != CODA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (dt == CODA_BF16)
    return chain_bwd_impl<uint16_t, true>((int)M, (int)K, (int)D, (int)N2, dY, A, W1, g, W2, H, r, dA, dR, dW1,
                                          dW2, dg, ws, s);
  return chain_bwd_impl<float, true>((int)M, (int)K, (int)D, (int)N2, dY, A, W1, g, W2, H, r, dA, dR, dW1, dW2, dg,
                                     ws, s);
}

size_t coda_chain_bwd_fp8_workspace_bytes(int64_t M, int64_t K, int64_t D, int64_t N2) {
  if (M < 0 || K < 1 || D < 1 || N2 < 1) return 0;
  return Bwd8Ws(M, K, D, N2).total;
}

coda_status coda_chain_bwd_fp8(int64_t M, int64_t K, int64_t D, int64_t N2, const void* dY, const void* A,
                               const void* W1, const void* g, const void* W2, const void* H, const float* r,
                               void* dA, void* dR, void* dW1, void* dW2, float* dg, void* ws, size_t ws_bytes,
                               void* stream) {
  coda_status st = check_dims_fp8(M, {{"K", K}, {"D", D}, {"N2", N2}});
  if (st != CODA_OK) return st;
  if (M % 16 != 0) return fail(CODA_ERR_SHAPE, "M = %lld is not a multiple of 16", (long long)M);
  if (M > kMaxColRows) return fail(CODA_ERR_SHAPE, "M = %lld exceeds %lld rows", (long long)M, (long long)kMaxColRows);
  for (const auto& d : {std::make_pair("K", K), std::make_pair("D", D), std::make_pair("N2", N2)})
    if ((d.second + 255) / 256 > 65535)  // the MX quantiser's grid of 256-column tiles
      return fail(CODA_ERR_SHAPE, "%s = %lld exceeds %d", d.first, (long long)d.second, 65535 * 256);
  const Mat mdY{dY, M, N2, N2, 2, "dY"}, mA{A, M, K, K, 2, "A"}, mH{H, M, D, D, 2, "H"};
  const Mat mdA{dA, M, K, K, 2, "dA"}, mdR{dR, M, D, D, 2, "dR"};
  const Mat mW1{W1, K, D, D, 2, "W1"}, mg{g, 1, D, D, 2, "g"}, mW2{W2, D, N2, N2, 2, "W2"};
  const Mat mdW1{dW1, K, D, D, 2, "dW1"}, mdW2{dW2, D, N2, N2, 2, "dW2"};
  const Mat mr{r, 1, M, M, 4, "r"}, mdg{dg, 1, D, D, 4, "dg"};
  for (const Mat* m : {&mW1, &mg, &mW2, &mdW1, &mdW2})
    if ((st = check_mat(*m, 8)) != CODA_OK) return st;
  if (M > 0) {
    for (const Mat* m : {&mdY, &mA, &mH, &mdA, &mdR})
      if ((st = check_mat(*m, 8)) != CODA_OK) return st;
    if (r == nullptr) return fail(CODA_ERR_NULL, "r is NULL");
    if (((uintptr_t)r & 3) != 0) return fail(CODA_ERR_ALIGN, "r is not 4-byte aligned");
  }
  if (dg == nullptr) return fail(CODA_ERR_NULL, "dg is NULL");
  if (((uintptr_t)dg & 3) != 0) return fail(CODA_ERR_ALIGN, "dg is not 4-byte aligned");
  const Bwd8Ws L(M, K, D, N2);
  if (ws == nullptr || ws_bytes < L.total)
    return fail(CODA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, ws ? ws_bytes : (size_t)0);
  if (((uintptr_t)ws & (kWsAlign - 1)) != 0) return fail(CODA_ERR_ALIGN, "workspace must be 256-byte aligned");
  for (int64_t bytes : {M * N2, N2 * M, D * N2, K * D, M * D, K * M})
    if (bytes > kMaxSpan) return fail(CODA_ERR_SHAPE, "an e4m3 workspace operand spans more than 2 GiB");
  const Mat mws{ws, 1, (int64_t)L.total, (int64_t)L.total, 1, "workspace"};
  const Mat none{nullptr, 0, 0, 0, 2, ""};
  const Mat outs[6] = {M > 0 ? mdA : none, M > 0 ? mdR : none, mdW1, mdW2, mdg, mws};
  const Mat ins[7] = {M > 0 ? mdY : none, M > 0 ? mA : none, mW1, mg, mW2, M > 0 ? mH : none, M > 0 ? mr : none};
  if ((st = check_alias(outs, 6, ins, 7)) != CODA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (M == 0)  // no rows: zero weight gradients and dg, as the bf16 backward writes them
    return chain_bwd_impl<uint16_t>(0, (int)K, (int)D, (int)N2, dY, A, W1, g, W2, H, r, dA, dR, dW1, dW2, dg,
                                    (char*)ws, s);
  return chain_bwd_fp8_impl((int)M, (int)K, (int)D, (int)N2, dY, A, W1, g, W2, H, r, dA, dR, dW1, dW2, dg,
                            (char*)ws, s);
}

const char* coda_status_string(coda_status s) {
  switch (s) {
    case CODA_OK: return "CODA_OK";
    case CODA_ERR_NULL: return "CODA_ERR_NULL";
    case CODA_ERR_SHAPE: return "CODA_ERR_SHAPE";
    case CODA_ERR_ALIGN: return "CODA_ERR_ALIGN";
    case CODA_ERR_DTYPE: return "CODA_ERR_DTYPE";
    case CODA_ERR_ALIAS: return "CODA_ERR_ALIAS";
    case CODA_ERR_WORKSPACE: return "CODA_ERR_WORKSPACE";
    case CODA_ERR_HIP: return "CODA_ERR_HIP";
  }
  return "CODA_ERR_UNKNOWN";
}

const char* coda_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
