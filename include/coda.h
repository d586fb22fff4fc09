/*
 * libcoda - the fused GEMM-Residual-PartialRMS-GEMM chain on one AMD Instinct
 * MI355X (CDNA4, gfx950).
 *
 * The chain (CODA news article by Synced / 机器之心, mirrored by KuCoin News,
 * section "CODA：「尾声」里藏着宝藏", the GEMM-RMSNorm-GEMM example):
 *
 *     H = A W1 + R                      residual stream after a projection
 *     Y = RMSNorm(H; g) W2              r_i = 1 / sqrt(mean_j H_ij^2 + eps)
 *                                       RMSNorm(H; g)_ij = r_i H_ij g_j
 *
 * The per-row scale r commutes with the second GEMM, so it is applied in that
 * GEMM's epilogue; the first GEMM's epilogue only emits per-tile partial sums
 * of squares, and a small combine kernel merges them into r.  No standalone
 * RMSNorm pass over H remains.  The epilogue building blocks used (section
 * "五种「积木」和一套「乐高语言」") are: element-wise (residual add), vector
 * load (broadcast of the RMSNorm weight g), tile store (H, kept for the
 * backward) and tile reduction (the partial RMS).
 *
 * Conventions shared by every entry point
 *   - Matrices are row-major with an explicit leading dimension `ld*`, counted
 *     in elements.  Shapes use the article's orientation: A[M,K], W1[K,D],
 *     R/H/Hg[M,D], W2[D,N2], Y[M,N2].
 *   - Every data pointer is a device pointer on the current HIP device.  The
 *     caller owns all memory; the library never allocates or frees.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream): they validate, enqueue kernels and return.  No host sync.
 *   - Validation happens before anything is enqueued.  On error the status is
 *     returned, nothing is enqueued, and coda_last_error() describes it.
 *     CODA_ERR_HIP means a launch failed (hipGetLastError reported it).
 *   - Requirements (CODA_ERR_SHAPE / CODA_ERR_ALIGN otherwise): M >= 0 (M = 0
 *     is a no-op, except where stated); K, D, N2 >= 1 and multiples of 8;
 *     ld >= row width and a multiple of 8 (bf16) or 4 (f32) elements; base
 *     pointers 16-byte aligned; each matrix spans less than 2 GiB.
 *   - Outputs must not overlap inputs (CODA_ERR_ALIAS), except where stated.
 *   - Deterministic: the same inputs give the same bits on every call.  Every
 *     sum runs in a fixed order; the only atomics are the fp8 quantisers'
 *     row and column maxima (an atomic max on the float bits, whose result
 *     does not depend on the order).  Thread-safe: the mutable global state
 *     is the per-thread last-error string and, for coda_chain_bwd_noalloc,
 *     a per-device table of its scratch address (filled once, under a
 *     lock) and the scratch array itself (see that call).
 *   - K, D, N2 multiples of 8 (16 for fp8) is a deliberate narrowing: the
 *     kernels move 16-byte pieces of 8 bf16 (4 f32, 16 e4m3) along every
 *     dimension except M, which may be any size.  LLaMA-shaped layers
 *     satisfy it; other sizes return CODA_ERR_SHAPE.
 *   - Rounding: every float32 -> bfloat16 conversion is round-to-nearest-even.
 */
#ifndef CODA_H
#define CODA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CODA_OK = 0,
  CODA_ERR_NULL = 1,      /* a required pointer is NULL                        */
  CODA_ERR_SHAPE = 2,     /* a size or leading dimension is out of range       */
  CODA_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned                  */
  CODA_ERR_DTYPE = 4,     /* unknown dtype code                                */
  CODA_ERR_ALIAS = 5,     /* an output overlaps an input or another output     */
  CODA_ERR_WORKSPACE = 6, /* workspace missing or smaller than required        */
  CODA_ERR_HIP = 7        /* a HIP launch failed                               */
} coda_status;

typedef enum {
  CODA_BF16 = 0, /* A, W1, R, g, H, Hg, W2, Y stored as bfloat16, fp32 accumulation */
  CODA_F32 = 1   /* everything stored and computed in float32                        */
} coda_dtype;

/* Number of partial-sum rows T that coda_gemm_res_prms writes for width D.
 * The caller allocates partials as float[T * M].  Returns -1 for bad args. */
int64_t coda_prms_num_partials(coda_dtype dt, int64_t D);

/* First GEMM with the residual / partial-RMS epilogue.
 *   H      = round(A W1 + R)                      [M,D]  (stored dtype)
 *   Hg     = round(float(H) * g)                  [M,D]  (only if g != NULL)
 *   partials[t*M + i] = sum over the columns j of tile t of float(H_ij)^2
 * for t in [0, T), T = coda_prms_num_partials(dt, D).  Tile t covers columns
 * [t*64, t*64+64) (clipped to D; an empty tile writes 0).  g and Hg are
 * both NULL or both non-NULL; with g == NULL the caller folds g into W2
 * itself.  A: lda >= K; W1: ldw1 >= D; R: ldr >= D; H, Hg: ldh, ldhg >= D. */
coda_status coda_gemm_res_prms(coda_dtype dt, int64_t M, int64_t K, int64_t D,
                               const void* A, int64_t lda,
                               const void* W1, int64_t ldw1,
                               const void* R, int64_t ldr,
                               const void* g,
                               void* H, int64_t ldh,
                               void* Hg, int64_t ldhg,
                               float* partials, void* stream);

/* Combine: r_i = 1 / sqrt((sum_{t<T} partials[t*M + i]) / D + eps).  The sum
 * runs in a fixed order (four consecutive quarters of t, each in increasing
 * t, then added first to last), so the result is deterministic; the mean and
 * square root are taken in double and rounded once to float.
 * partials: float[T*M] as written above; r: float[M]. T >= 1, D >= 1,
 * eps >= 0. */
coda_status coda_rms_combine(int64_t M, int64_t D, int64_t T, float eps,
                             const float* partials, float* r, void* stream);

/* Second GEMM with the deferred row-scale epilogue:
 *   Y_ik = round(r_i * sum_j X_ij W2_jk)          [M,N2]
 * X is Hg = H diag(g) (or H when g was folded into W2).  r may be NULL
 * (then r_i = 1, a plain GEMM).  X: ldx >= D; W2: ldw2 >= N2; Y: ldy >= N2. */
coda_status coda_gemm_rowscale(coda_dtype dt, int64_t M, int64_t D, int64_t N2,
                               const void* X, int64_t ldx,
                               const void* W2, int64_t ldw2,
                               const float* r,
                               void* Y, int64_t ldy, void* stream);

/* The forward pair with the Hg intermediate tile-packed (bfloat16 only).
 * The article's epilogue section has the first GEMM's epilogue write what the
 * second GEMM consumes; here it also writes it in the order the second GEMM's
 * MFMA fragment reads take it.  Tile-packed layout of an [M,D] matrix (D a
 * multiple of 8, rows padded to a multiple of 16): element (i, 8c + e) lies
 * at bfloat16 index ((i/16 * D/8 + c) * 16 + i%16) * 8 + e, i.e. for each
 * 16-row block and each run of 8 columns, the 16 rows' 16-byte pieces are
 * contiguous.  Padding rows are never written nor read.  Values, H,
 * partials, r and Y are bit-identical to coda_gemm_res_prms +
 * coda_gemm_rowscale; only where Hg lives differs. */

/* Bytes of a tile-packed bfloat16 matrix of `rows` rows and `cols` columns
 * (cols a multiple of 8): 2 * cols * (rows rounded up to 16).  -1 for bad
 * arguments. */
int64_t coda_packed_bytes(int64_t rows, int64_t cols);

/* coda_gemm_res_prms (bfloat16) with Hg tile-packed: Hgp holds
 * coda_packed_bytes(M, D) bytes, 16-byte aligned; g and Hgp must be set.
 * The other arguments and outputs are those of coda_gemm_res_prms. */
coda_status coda_gemm_res_prms_packed(int64_t M, int64_t K, int64_t D,
                                      const void* A, int64_t lda,
                                      const void* W1, int64_t ldw1,
                                      const void* R, int64_t ldr,
                                      const void* g,
                                      void* H, int64_t ldh,
                                      void* Hgp, float* partials, void* stream);

/* coda_gemm_rowscale (bfloat16) reading X = Hg tile-packed (Xp, as written
 * by coda_gemm_res_prms_packed for the same M and D):
 *   Y_ik = round(r_i * sum_j X_ij W2_jk)          [M,N2]
 * r may be NULL (plain GEMM).  W2: ldw2 >= N2; Y: ldy >= N2. */
coda_status coda_gemm_rowscale_packed(int64_t M, int64_t D, int64_t N2,
                                      const void* Xp,
                                      const void* W2, int64_t ldw2,
                                      const float* r,
                                      void* Y, int64_t ldy, void* stream);

/* Second GEMM with the deferred row scale and a SwiGLU gate in the epilogue.
 * The article (section "CODA：「尾声」里藏着宝藏") says the re-parameterisation
 * applies to SwiGLU as well, and its results section measures SwiGLU epilogue
 * compositions; it does not write SwiGLU out.  Reading taken (the LLaMA gate):
 * W2 = [W_gate | W_up], columns [0, F) and [F, 2F), and with
 * y = r_i * (X W2)_ik (fp32 accumulation):
 *   Z_ij = round(silu(y_ij) * y_i,F+j)    [M,F],  silu(x) = x / (1 + e^-x)
 *   Y_ik = round(y_ik)                    [M,2F], only if Y != NULL (the
 *                                          pre-activation kept for a backward)
 * Z (and Y) are written straight from the accumulators: the [M,2F]
 * pre-activation never goes through HBM unless asked for.
 *   X: [M,D] (ldx); W2: [D,2F] (ldw2 >= 2F); r: float[M] or NULL (no row
 *   scale); Z: [M,F] (ldz); Y: [M,2F] (ldy) or NULL.
 * F >= 1, a multiple of 32 (the gate and up halves are read in interleaved
 * 32-column runs).  Z and Y must not overlap X, W2, r or each other. */
coda_status coda_gemm_rowscale_swiglu(coda_dtype dt, int64_t M, int64_t D, int64_t F,
                                      const void* X, int64_t ldx,
                                      const void* W2, int64_t ldw2,
                                      const float* r,
                                      void* Z, int64_t ldz,
                                      void* Y, int64_t ldy, void* stream);

/* coda_gemm_rowscale_swiglu (bfloat16) reading X = Hg tile-packed (Xp, as
 * written by coda_gemm_res_prms_packed for the same M and D).  Z and Y are
 * bit-identical to coda_gemm_rowscale_swiglu's. */
coda_status coda_gemm_rowscale_swiglu_packed(int64_t M, int64_t D, int64_t F,
                                             const void* Xp,
                                             const void* W2, int64_t ldw2,
                                             const float* r,
                                             void* Z, int64_t ldz,
                                             void* Y, int64_t ldy, void* stream);

/* Backward through the SwiGLU gate (the article's results section measures
 * the SwiGLU backward; the formula is the derivative of the reading above):
 * with s = sigmoid(Y_gate),
 *   dY_ij     = round(dZ_ij * Y_i,F+j * s (1 + Y_ij (1 - s)))   j < F (gate)
 *   dY_i,F+j  = round(dZ_ij * Y_ij * s)                          (up)
 * elementwise, fp32 arithmetic.  dZ: [M,F] (ldz); Y: the kept pre-activation
 * [M,2F] (ldy); dY: [M,2F] (lddy), the dY that coda_chain_bwd takes.
 * F >= 1, a multiple of 8.  dY must not overlap dZ or Y. */
coda_status coda_swiglu_bwd(coda_dtype dt, int64_t M, int64_t F,
                            const void* dZ, int64_t ldz, const void* Y, int64_t ldy,
                            void* dY, int64_t lddy, void* stream);

/* ---- cross-entropy head --------------------------------------------------
 * The article says the re-parameterisation covers the cross-entropy loss
 * (section "CODA：「尾声」里藏着宝藏") and lists the tile log-sum-exp and the
 * max / sum-exp state of online normalisation among the epilogue building
 * blocks (section "五种「积木」和一套「乐高语言」").  Reading taken: the chain's
 * second GEMM is the LM head (W2 = W_vocab [D,V]) and the loss is the
 * per-token cross-entropy loss_i = lse_i - Y_i,t_i, lse_i = log sum_j e^Y_ij.
 * The [M,V] logits are never written. */

/* LM-head GEMM with the cross-entropy statistics in the epilogue.  With
 * y = r_i * (X W_v)_ij in fp32 (never stored) and T = coda_prms_num_partials(dt, V)
 * partial tiles of 64 columns:
 *   pmax[t*M + i] = max of y over partial tile t;  psum[t*M + i] = sum of
 *   e^(y - pmax) over it ((-inf, 0) for a tile past the last column);
 *   tgt[i] = y at column targets[i] (not written if the target is outside
 *   [0, V)).
 * X: [M,D] (ldx, e.g. Hg); Wv: [D,V] (ldw); r: float[M] or NULL; targets:
 * int32[M]; pmax, psum: float[T*M]; tgt: float[M].  V a multiple of 8. */
coda_status coda_gemm_rowscale_lse(coda_dtype dt, int64_t M, int64_t D, int64_t V,
                                   const void* X, int64_t ldx, const void* Wv, int64_t ldw,
                                   const float* r, const int32_t* targets,
                                   float* pmax, float* psum, float* tgt, void* stream);

/* coda_gemm_rowscale_lse (bfloat16) reading X = Hg tile-packed (Xp, as
 * written by coda_gemm_res_prms_packed for the same M and D).  pmax, psum and
 * tgt are bit-identical to coda_gemm_rowscale_lse's. */
coda_status coda_gemm_rowscale_lse_packed(int64_t M, int64_t D, int64_t V,
                                          const void* Xp, const void* Wv, int64_t ldw,
                                          const float* r, const int32_t* targets,
                                          float* pmax, float* psum, float* tgt, void* stream);

/* Cross-entropy combine: lse_i = M_i + log(sum_t psum[t*M+i] e^(pmax[t*M+i] - M_i))
 * with M_i = max_t pmax, merged in a fixed order (four quarters of t, each in
 * increasing t, then first to last); loss_i = lse_i - tgt[i], or NaN when
 * targets[i] is outside [0, V).  All arrays float[M] / float[T*M] / int32[M]. */
coda_status coda_ce_combine(int64_t M, int64_t V, int64_t T, const float* pmax, const float* psum,
                            const float* tgt, const int32_t* targets, float* lse, float* loss,
                            void* stream);

/* ---- QKV projection with RoPE -------------------------------------------
 * The article says the re-parameterisation covers RoPE (section
 * "CODA：「尾声」里藏着宝藏") and counts RoPE among the element-wise epilogue
 * transforms (section "五种「积木」和一套「乐高语言」"); it does not write RoPE
 * out.  Reading taken (the rotary embedding in its interleaved form): the
 * chain's second GEMM is the attention QKV projection, its output columns
 * [Q | K | V] with n_q and n_k columns of heads of d_head columns; inside a
 * Q or K head the pair (2i, 2i+1), i < d_head/2, of row m turns by the angle
 * p_m theta_i, theta_i = base^(-2i/d_head), p_m the row's position:
 *   Y_m,2i = y_2i cos - y_2i+1 sin,   Y_m,2i+1 = y_2i sin + y_2i+1 cos.
 * V columns are not rotated.  The unrotated [M,N2] projection is never
 * written. */

/* Rotary table: cos_sin[(p * d_head/2 + i) * 2 + {0, 1}] = cos, sin of
 * p theta_i for p < max_pos, i < d_head/2, evaluated in double precision and
 * rounded to float.  cos_sin: float[max_pos * d_head], 8-byte aligned,
 * written on `stream`.  d_head even; base finite and > 0 (10000 in the
 * original RoPE, 500000 in LLaMA 3). */
coda_status coda_rope_cache(float* cos_sin, int64_t max_pos, int64_t d_head, double base,
                            void* stream);

/* Second GEMM with the deferred row scale and RoPE in the epilogue: with
 * y = r_i * (X W2)_ik (fp32), Y = round(rotate(y)) as above, using the
 * table entries cos_sin[positions[i]] (so theta and base are the table's).
 *   X: [M,D] (ldx, e.g. Hg); W2: [D,N2] (ldw2, W_qkv); r: float[M] or NULL;
 *   positions: int32[M]; cos_sin: the table of coda_rope_cache, float
 *   [max_pos * d_head], 16-byte aligned; Y: [M,N2] (ldy).
 * d_head a multiple of 8 in [8, 4096]; n_q, n_k whole heads (>= 0) with
 * n_q + n_k <= N2.  A position outside [0, max_pos) is not read: the row's
 * rotated columns become NaN (its V columns stay valid).  Y must not overlap
 * any input. */
coda_status coda_gemm_rowscale_rope(coda_dtype dt, int64_t M, int64_t D, int64_t N2,
                                    const void* X, int64_t ldx, const void* W2, int64_t ldw2,
                                    const float* r, const int32_t* positions,
                                    const float* cos_sin, int64_t max_pos,
                                    int64_t n_q, int64_t n_k, int64_t d_head,
                                    void* Y, int64_t ldy, void* stream);

/* coda_gemm_rowscale_rope (bfloat16) reading X = Hg tile-packed (Xp, as
 * written by coda_gemm_res_prms_packed for the same M and D).  Y is
 * bit-identical to coda_gemm_rowscale_rope's. */
coda_status coda_gemm_rowscale_rope_packed(int64_t M, int64_t D, int64_t N2,
                                           const void* Xp, const void* W2, int64_t ldw2,
                                           const float* r, const int32_t* positions,
                                           const float* cos_sin, int64_t max_pos,
                                           int64_t n_q, int64_t n_k, int64_t d_head,
                                           void* Y, int64_t ldy, void* stream);

/* Backward through RoPE (the derivative of the reading above; the rotation
 * is orthogonal, so the gradient turns back by the same angle):
 *   dY_m,2i = g_2i cos + g_2i+1 sin,   dY_m,2i+1 = g_2i+1 cos - g_2i sin
 * in the rotated columns (NaN for a position outside [0, max_pos)), dY = g in
 * the V columns.  dYr: the gradient of the rotated output [M,N2] (ldg); dY:
 * [M,N2] (lddy), the dY that coda_chain_bwd takes.  Arguments and limits as
 * coda_gemm_rowscale_rope; dY must not overlap dYr, positions or cos_sin. */
coda_status coda_rope_bwd(coda_dtype dt, int64_t M, int64_t N2, const void* dYr, int64_t ldg,
                          const int32_t* positions, const float* cos_sin, int64_t max_pos,
                          int64_t n_q, int64_t n_k, int64_t d_head,
                          void* dY, int64_t lddy, void* stream);

/* Backward of the cross-entropy head (the derivative of the reading above):
 * recomputes y = r_i * (X W_v)_ij in fp32 and writes the gradient of
 * sum_i dloss_i loss_i with respect to the logits,
 *   dY_ij = round(dloss_i * (e^(y_ij - lse_i) - [j == targets[i]])),
 * the dY that coda_chain_bwd takes (with W2 = W_v).  lse: the forward's
 * (coda_ce_combine); dloss: float[M] upstream gradient per token (1/M for a
 * mean over tokens).  A target outside [0, V) makes the row NaN.  X, Wv, r,
 * targets as coda_gemm_rowscale_lse; dY: [M,V] (lddy), not overlapping any
 * input.  The [M,V] logits are recomputed, never read. */
coda_status coda_gemm_rowscale_ce_bwd(coda_dtype dt, int64_t M, int64_t D, int64_t V,
                                      const void* X, int64_t ldx, const void* Wv, int64_t ldw,
                                      const float* r, const int32_t* targets, const float* lse,
                                      const float* dloss, void* dY, int64_t lddy, void* stream);

/* coda_gemm_rowscale_ce_bwd (bfloat16) reading X = Hg tile-packed (Xp, as
 * written by coda_gemm_res_prms_packed for the same M and D).  dY is
 * bit-identical to coda_gemm_rowscale_ce_bwd's. */
coda_status coda_gemm_rowscale_ce_bwd_packed(int64_t M, int64_t D, int64_t V,
                                             const void* Xp, const void* Wv, int64_t ldw,
                                             const float* r, const int32_t* targets,
                                             const float* lse, const float* dloss,
                                             void* dY, int64_t lddy, void* stream);

/* ---- fp8 operands -------------------------------------------------------
 * The article's opening section notes that FP8 makes the matrix products
 * faster while the memory-bound operations around them do not shrink, so
 * fusing them matters more at low precision; it gives no fp8 recipe.  The
 * one taken here: GEMM operands are OCP e4m3 codes (1 sign, 4 exponent bits,
 * bias 7, 3 mantissa bits; largest finite 448; no infinities) with float32
 * dequantisation scales, A per row and the weights per output channel, the
 * weights stored transposed ([N, K], contraction contiguous).  H stays bf16;
 * the second GEMM's operand x = H g is quantised with one power-of-two scale
 * per row and block of 32 columns, the block scaling of the OCP microscaling
 * (MX) formats: its exponent E is the smallest integer with
 * max |x| over the block <= 448 * 2^E (clamped to [-127, 127], 0 for an
 * all-zero block), so no code saturates, and the codes are e4m3_rne(x 2^-E).
 * Products run on v_mfma_scale_f32_32x32x64_f8f6f4 with fp32 accumulation;
 * the MX exponents ride along as the instruction's A-side scales.  Sizes:
 * K, D, N2 multiples of 16; e4m3 leading dimensions multiples of 16
 * elements, bf16 ones multiples of 8.
 *
 * Block-exponent arrays (hg_exp, x_exp): coda_mx_exp_bytes(M, D) bytes,
 * 16-byte aligned.  E + 127 (an E8M0 code) for row i and columns
 * [64 t + 32 h, 64 t + 32 h + 32) of D lies at byte
 *   ((t/4 * ceil(M/128) + i/128) * 64 + 32 h + i%32) * 16 + ((i/32)%4) * 4 + t%4
 * (groups of 4 k-tiles of 64 columns, then blocks of 128 rows: each lane of
 * the second GEMM finds the 4 exponents it needs per k-tile group in 16
 * consecutive bytes).  The first GEMM writes every byte, 127 (E = 0) for
 * the blocks past D and the rows past M in the last block; the second GEMM
 * reads the bytes of t < ceil(D / 64) only. */

/* Bytes of the block-exponent array of a [rows, cols] MX operand:
 * 1024 * ceil(rows / 128) * ceil(cols / 256).  -1 for bad arguments. */
int64_t coda_mx_exp_bytes(int64_t rows, int64_t cols);

/* First GEMM, fp8 operands:
 *   H_ij   = round_bf16((acc_ij * sa_i) * sw1_j + R_ij)     acc = sum_k A8_ik W1t8_jk
 *   x_ij   = float(H_ij) * g_j                               (float32 product)
 *   hg_exp = the MX block exponents E of x (layout above)
 *   Hg8_ij = e4m3_rne(x_ij * 2^-E)                           (never saturates)
 *   partials as coda_gemm_res_prms (coda_prms_num_partials(CODA_BF16, D) rows)
 *   A8: e4m3 [M,K] (lda); sa: float[M]; W1t8: e4m3 [D,K] (ldw1t); sw1: float[D],
 *   16-byte aligned; R, g, H: bf16; Hg8: e4m3 [M,D] (ldhg); hg_exp as above.
 *   The block maximum is taken inside the epilogue (the 32 columns of a
 *   block sit in 4 lanes of one row).  x must be finite: a NaN is left out
 *   of its block's maximum and coded as -448, an infinity as +-448. */
coda_status coda_gemm_res_prms_fp8(int64_t M, int64_t K, int64_t D,
                                   const void* A8, int64_t lda, const float* sa,
                                   const void* W1t8, int64_t ldw1t, const float* sw1,
                                   const void* R, int64_t ldr, const void* g,
                                   void* H, int64_t ldh, void* Hg8, int64_t ldhg,
                                   void* hg_exp, float* partials, void* stream);

/* Quantisation of a bf16 operand for the fp8 GEMMs (the recipe above): per
 * row of X [M,K], scale = amax / 448 (1 for an all-zero row) and
 * X8 = e4m3_rne(clamp(x / scale, +-448)), the division correctly rounded in
 * float32.  X: bf16 [M,K] (ldx); X8: e4m3 [M,K] (ldx8); scales: float[M].
 * K a multiple of 16; inputs finite.  X8 and scales must not overlap X. */
coda_status coda_quantize_rows_e4m3(int64_t M, int64_t K, const void* X, int64_t ldx,
                                    void* X8, int64_t ldx8, float* scales, void* stream);

/* The weight variant: W bf16 [K,N] (ldw, N contiguous) gives the transposed
 * codes Wt8 [N,K] (ldwt, K contiguous) with one scale per output channel n,
 * the layout coda_gemm_res_prms_fp8 and coda_gemm_rowscale_fp8 take.  K and
 * N multiples of 16, K <= 4194240.  scales also serves as the column maxima
 * while the call runs. */
coda_status coda_quantize_cols_e4m3(int64_t K, int64_t N, const void* W, int64_t ldw,
                                    void* Wt8, int64_t ldwt, float* scales, void* stream);

/* Both quantisations of one bf16 activation X [M,N] (ldx), as the fp8
 * backward needs them for dY and dH: the row codes X8 [M,N] (ldx8) with
 * row_scales[M], exactly as coda_quantize_rows_e4m3, and the transposed
 * column codes Xt8 [N,M] (ldxt) with col_scales[N], exactly as
 * coda_quantize_cols_e4m3 (X in the role of W).  One pass over X finds both
 * maxima, a second writes both codes.  M and N multiples of 16,
 * M <= 4194240; the outputs must not overlap X or each other.  The scale
 * arrays also serve as the maxima while the call runs. */
coda_status coda_quantize_rows_cols_e4m3(int64_t M, int64_t N, const void* X, int64_t ldx,
                                         void* X8, int64_t ldx8, float* row_scales,
                                         void* Xt8, int64_t ldxt, float* col_scales,
                                         void* stream);

/* Second GEMM, fp8 operands, deferred row scale:
 *   Y_ik = round_bf16((acc_ik * r_i) * sw2_k)
 *   acc  = sum_j e4m3(X8_ij) 2^E(i, j) e4m3(W2t8_kj)
 *   X8: e4m3 [M,D] (ldx), e.g. Hg8; x_exp: its MX block exponents E (layout
 *   above, e.g. hg_exp), or NULL for E = 0; W2t8: e4m3 [N2,D] (ldw2t); sw2:
 *   float[N2], 16-byte aligned; r: float[M] or NULL; Y: bf16 [M,N2] (ldy). */
coda_status coda_gemm_rowscale_fp8(int64_t M, int64_t D, int64_t N2,
                                   const void* X8, int64_t ldx, const void* x_exp,
                                   const void* W2t8, int64_t ldw2t, const float* sw2,
                                   const float* r, void* Y, int64_t ldy, void* stream);

/* The fp8 forward with tile-packed operands (the layout of
 * coda_gemm_res_prms_packed, with 16 codes per 16-byte piece): element
 * (i, 16c + e) of an e4m3 [rows, cols] matrix at byte
 * ((i/16 * cols/16 + c) * 16 + i%16) * 16 + e, rows padded to a multiple of
 * 16 (never written nor read).  The second GEMM then reads both operands
 * with contiguous 1 KiB direct loads and full-rate fragment reads.  Codes,
 * scales, H, partials and Y are bit-identical to the row-major calls. */

/* Bytes of a tile-packed e4m3 matrix: cols * (rows rounded up to 16); cols a
 * multiple of 16.  -1 for bad arguments. */
int64_t coda_packed_bytes_e4m3(int64_t rows, int64_t cols);

/* coda_quantize_cols_e4m3 with the transposed codes Wt8 [N,K] written
 * tile-packed into Wt8p (coda_packed_bytes_e4m3(N, K) bytes, 16-byte aligned). */
coda_status coda_quantize_cols_e4m3_packed(int64_t K, int64_t N, const void* W, int64_t ldw,
                                           void* Wt8p, float* scales, void* stream);

/* coda_quantize_rows_e4m3 with the codes X8 [M,K] written tile-packed into
 * X8p (coda_packed_bytes_e4m3(M, K) bytes, 16-byte aligned; the rows past M
 * in the last 16-row block are not written).  Same recipe, scales and codes.
 * coda_gemm_res_prms_fp8_all_packed takes A's codes in this layout. */
coda_status coda_quantize_rows_e4m3_packed(int64_t M, int64_t K, const void* X, int64_t ldx,
                                           void* X8p, float* scales, void* stream);

/* coda_quantize_rows_cols_e4m3 with both code arrays tile-packed: X8p holds
 * the row codes [M,N] (coda_packed_bytes_e4m3(M, N) bytes) and Xt8p the
 * transposed column codes [N,M] (coda_packed_bytes_e4m3(N, M) bytes), both
 * 16-byte aligned.  M a multiple of 16, M <= 4194240; scales as in
 * coda_quantize_rows_cols_e4m3. */
coda_status coda_quantize_rows_cols_e4m3_packed(int64_t M, int64_t N, const void* X, int64_t ldx,
                                                void* X8p, float* row_scales, void* Xt8p,
                                                float* col_scales, void* stream);

/* coda_gemm_res_prms_fp8 with Hg8 written tile-packed into Hg8p
 * (coda_packed_bytes_e4m3(M, D) bytes, 16-byte aligned); A8 and W1t8 as in
 * coda_gemm_res_prms_fp8. */
coda_status coda_gemm_res_prms_fp8_packed(int64_t M, int64_t K, int64_t D,
                                          const void* A8, int64_t lda, const float* sa,
                                          const void* W1t8, int64_t ldw1t, const float* sw1,
                                          const void* R, int64_t ldr, const void* g,
                                          void* H, int64_t ldh, void* Hg8p, void* hg_exp,
                                          float* partials, void* stream);

/* coda_gemm_res_prms_fp8_packed with both operands tile-packed as well:
 * A8p [M,K] as coda_quantize_rows_e4m3_packed writes it
 * (coda_packed_bytes_e4m3(M, K) bytes) and W1t8p [D,K] as
 * coda_quantize_cols_e4m3_packed writes W1's transposed codes
 * (coda_packed_bytes_e4m3(D, K) bytes), both 16-byte aligned; sa, sw1, R,
 * g, H, Hg8p, hg_exp and partials as in coda_gemm_res_prms_fp8_packed.  The
 * same arithmetic on the same codes as with row-major operands, so the
 * outputs are bit-identical; the packed operands let the kernel's LDS reads
 * take whole 16-byte fragments. */
coda_status coda_gemm_res_prms_fp8_all_packed(int64_t M, int64_t K, int64_t D,
                                              const void* A8p, const float* sa,
                                              const void* W1t8p, const float* sw1,
                                              const void* R, int64_t ldr, const void* g,
                                              void* H, int64_t ldh, void* Hg8p, void* hg_exp,
                                              float* partials, void* stream);

/* coda_gemm_rowscale_fp8 with both operands tile-packed: X8p [M,D] (as
 * coda_gemm_res_prms_fp8_packed writes Hg8) and W2t8p [N2,D] (as
 * coda_quantize_cols_e4m3_packed writes it).  x_exp (row-major, never
 * packed), sw2, r, Y as in coda_gemm_rowscale_fp8. */
coda_status coda_gemm_rowscale_fp8_packed(int64_t M, int64_t D, int64_t N2,
                                          const void* X8p, const void* x_exp,
                                          const void* W2t8p, const float* sw2,
                                          const float* r, void* Y, int64_t ldy, void* stream);

/* Bytes of workspace coda_ref_chain needs: float C[M,D] + X_n[M,D]. */
size_t coda_ref_chain_workspace_bytes(coda_dtype dt, int64_t M, int64_t D);

/* Unfused reference chain (the operator-by-operator order: GEMM, residual add,
 * RMSNorm, GEMM), for A/B comparison with the fused path.  Four kernels:
 *   C  = A W1 (float32, same GEMM main loop as coda_gemm_res_prms)
 *   H  = round(C + R)                 -> bit-identical to the fused H
 *   r_i = 1/sqrt(mean_j float(H_ij)^2 + eps);  X_n = round(float(H) * r * g)
 *   Y  = round(X_n W2)
 * All matrices dense (ld = width).  ws: coda_ref_chain_workspace_bytes(). */
coda_status coda_ref_chain(coda_dtype dt, int64_t M, int64_t K, int64_t D, int64_t N2,
                           float eps,
                           const void* A, const void* W1, const void* R,
                           const void* g, const void* W2,
                           void* H, float* r, void* Y,
                           void* ws, size_t ws_bytes, void* stream);

/* ---- backward ------------------------------------------------------------
 * Gradients of a scalar loss L through the chain, given dY = dL/dY.  The
 * article (section "CODA：「尾声」里藏着宝藏") notes that the backward pass
 * keeps the tile-local structure of the forward; written out with
 * G = dY W2^T, P = G diag(g) and s_i = <P_i, H_i>:
 *
 *     dW2 = X_n^T dY,        X_n = diag(r) H diag(g)
 *     dg_j = sum_i r_i H_ij G_ij
 *     dH_i = r_i P_i - (r_i^3 s_i / D) H_i        (through X_n and through r)
 *     dR = dH,   dA = dH W1^T,   dW1 = A^T dH
 *
 * Only s and dg need reductions across tiles.  Six kernels, in stream order:
 *   1. GEMM G = dY W2^T; epilogue: P = round(g_j G_ij) into dR, X_n =
 *      round((float(H_ij) r_i) g_j) into the workspace, per-row partial sums
 *      of P_ij H_ij per 64 columns (unrounded P), per-column partial sums of
 *      r_i H_ij G_ij per 128 rows;
 *   2. combine: c_i = r_i^3 (sum of the row partials) / D, dg_j = sum of the
 *      column partials (both in fixed order);
 *   3. dH = round(r_i float(P_ij) - c_i float(H_ij)), in place in dR;
 *   4. dA = round(dH W1^T);  5. dW1 = round(A^T dH);  6. dW2 = round(X_n^T dY).
 * H and r are the forward's stored values (coda_gemm_res_prms, coda_rms_combine).
 * All float32 accumulation.  With M = 0, dW1, dW2 and dg are written as zeros
 * and the M-row arguments (dY, A, H, r, dA, dR) may be NULL. */

/* Bytes of workspace coda_chain_bwd needs: X_n[M,D] (dtype), row partials
 * float[T*M] (T = coda_prms_num_partials(dt, D)), column partials
 * float[ceil(M/128)*D], c float[M], and the transposed weights W2^T [N2,D]
 * and W1^T [D,K] (dtype; G and dA read them row-contiguously), each part
 * 256-byte aligned; at least 256 bytes.  0 for invalid arguments. */
size_t coda_chain_bwd_workspace_bytes(coda_dtype dt, int64_t M, int64_t K, int64_t D, int64_t N2);

/* Backward of the chain.  All matrices dense (ld = width).
 *   dY[M,N2], A[M,K], W1[K,D], g[D], W2[D,N2], H[M,D] (dtype); r[M] float
 *   dA[M,K], dR[M,D] (= dH; also the operand of dA and dW1), dW1[K,D],
 *   dW2[D,N2] (dtype); dg[D] float
 * ws: device memory of coda_chain_bwd_workspace_bytes(), 256-byte aligned,
 * overwritten.  Outputs and workspace must not overlap any input or each
 * other.  Errors as in the forward calls. */
coda_status coda_chain_bwd(coda_dtype dt, int64_t M, int64_t K, int64_t D, int64_t N2,
                           const void* dY, const void* A, const void* W1, const void* g,
                           const void* W2, const void* H, const float* r,
                           void* dA, void* dR, void* dW1, void* dW2, float* dg,
                           void* ws, size_t ws_bytes, void* stream);

/* Bytes of the scratch array coda_chain_bwd_noalloc keeps in device memory
 * (one copy on each GPU the library runs on, held until the process ends). */
#define CODA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* coda_chain_bwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving or training loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and errors as coda_chain_bwd, without
 * the workspace: the call allocates nothing (no hipMalloc, no library
 * allocation) and keeps X_n, the partial sums and c in the library's static
 * scratch array instead.  G and dA read W2 and W1 in place (no transposed
 * copies), which gives bit-identical results.
 * Limit: the shape must need at most CODA_NOALLOC_SCRATCH_BYTES of scratch,
 *   X_n M*D (dtype) + 4*T*M + 4*U*D + 4*M bytes, each part rounded up to a
 *   multiple of 256, with T = 4*ceil(D/256) and U = ceil(M/128)
 *   (bf16: M*D up to about 31M elements, e.g. M = 7680 at D = 4096).
 * Larger shapes fail with CODA_ERR_WORKSPACE before anything is enqueued.
 * The scratch is shared by every call on one GPU and keeps the last call's
 * contents (nothing in it needs to start at zero): calls that overlap on
 * one GPU -- on two streams, or from two host threads -- race on it, so
 * the caller orders them.  The first call on each device looks up the
 * array's device address (hipGetSymbolAddress); a failure there is
 * CODA_ERR_HIP. */
coda_status coda_chain_bwd_noalloc(coda_dtype dt, int64_t M, int64_t K, int64_t D, int64_t N2,
                                   const void* dY, const void* A, const void* W1, const void* g,
                                   const void* W2, const void* H, const float* r,
                                   void* dA, void* dR, void* dW1, void* dW2, float* dg,
                                   void* stream);

/* MX (OCP microscaling) e4m3 quantisation of a bf16 matrix X [M, N] (row-
 * major, ldx) along its rows and/or its columns, as the fp8 backward takes
 * its operands; one read of X serves both.  Each block of 32 consecutive
 * elements along the quantised direction gets its own exponent E, the
 * smallest integer with the block's largest magnitude <= 448 2^E (clamped to
 * [-127, 127], 0 for an all-zero block; the rule of the fp8 first GEMM's
 * block exponents), stored as the E8M0 byte E + 127, and its elements the
 * codes e4m3(x 2^-E), nearest-even (no value saturates).
 *   Xr8p, Er: the row codes [M, N] tile-packed (coda_packed_bytes_e4m3(M, N)
 *     bytes) and their exponents, one per row and 32 columns, in the layout
 *     of coda_mx_exp_bytes (rows M, cols N: coda_mx_exp_bytes(M, N) bytes);
 *   Xc8p, Ec: the codes of X^T [N, M] tile-packed (coda_packed_bytes_e4m3(N,
 *     M) bytes), one exponent per column of X and 32 rows (rows N, cols M:
 *     coda_mx_exp_bytes(N, M) bytes).
 * Either pair may be NULL (not both; a pair is both set or both NULL).  Every
 * byte of an exponent array is written, those of padding rows and of blocks
 * past the end as 127.  M, N multiples of 16, N <= 16776960; M = 0 is a
 * no-op.  All outputs 16-byte aligned; none may overlap X or another. */
coda_status coda_quantize_mx_e4m3_packed(int64_t M, int64_t N, const void* X, int64_t ldx,
                                         void* Xr8p, void* Er, void* Xc8p, void* Ec, void* stream);

/* Backward of the chain with e4m3 products (the fp8 recipe above, carried to
 * the backward; the pages give none).  Every product takes e4m3 operands
 * with MX block exponents along its contraction, as
 * coda_quantize_mx_e4m3_packed makes them, and the matrix core applies the
 * exponents of both operands:
 *   G = dY W2^T       dY along its rows, W2 [D,N2] along its rows
 *   dW2 = X_n^T dY    X_n and dY along their columns (contraction over M)
 *   dA = dH W1^T      dH along its rows, W1 [K,D] along its rows
 *   dW1 = A^T dH      A and dH along their columns
 * with fp32 accumulation; everything else (P, X_n, the partial sums, c, dg,
 * dH = r P - c H, dR = dH) is the bf16 backward's.  The quantisers count as
 * the identity when differentiating (straight-through).  Arguments as
 * coda_chain_bwd, all bf16 (r, dg float); M, K, D, N2 multiples of 16,
 * M <= 4194240; ws of coda_chain_bwd_fp8_workspace_bytes(): the bf16
 * backward's partial sums and c, and the e4m3 operands with their
 * exponents (X_n is never held in bf16: G's epilogue writes its column
 * codes and exponents directly). */
size_t coda_chain_bwd_fp8_workspace_bytes(int64_t M, int64_t K, int64_t D, int64_t N2);
coda_status coda_chain_bwd_fp8(int64_t M, int64_t K, int64_t D, int64_t N2,
                               const void* dY, const void* A, const void* W1, const void* g,
                               const void* W2, const void* H, const float* r,
                               void* dA, void* dR, void* dW1, void* dW2, float* dg,
                               void* ws, size_t ws_bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* coda_status_string(coda_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if
 * none).  Valid until the next libcoda call on that thread. */
const char* coda_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CODA_H */
