/*
 * bsg.h -- C ABI of libbsg, the binary sign-GEMV library for AMD Instinct
 * MI355X (gfx950).
 *
 * The decode-time product with binary-compressed weights
 *
 *     y = sum_k alpha_k (.) (B_k (c_k (.) x))                  binary bases
 *       + sum_j alpha_r[j] * u_j * (v_j . x)                     low-rank signs
 *       + (protected int8 rows)
 *
 * Sources (the web pages this library is built from):
 *  - "FluxBin: Flexible LUT-based Ultra-low-bit LLM Inference by
 *    Algorithm-Kernel Synergy": Sec. 2 (weights approximated by a greedy
 *    residual sum of binary bases), Sec. 3.1 (decoupled row and column scales;
 *    the quantised matrix is the sum over bases), Sec. 3.2 Stage 1 (a set bit b
 *    means +1 and a clear bit -1, i.e. 2b-1; the column scale is folded into
 *    the activation before the main loop).
 *  - "BiLoCo: Binary Low-Rank Corrections for Post-Training Quantization":
 *    "The core idea" (correction alpha*u*(v.x) with u, v in {+1,-1}, computed
 *    with additions and subtractions only).
 *  - "BiSCo-LLM: Lookup-Free Binary Spherical Coding for Extreme Low-Bit LLM
 *    Compression", technical summary, "Sensitivity Protection" (about 1% of
 *    sensitive channels, chosen from activation statistics and weight
 *    magnitudes, kept in 8 bits apart from the binary payload).
 *
 * General rules for every entry point:
 *  - Pointers marked (device) are device memory of the current HIP device;
 *    (host) pointers are host memory.  Every buffer is owned by the caller;
 *    the library allocates no device memory and keeps no state between calls
 *    other than its loaded code objects.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL means
 *    the null stream).  No entry point synchronises.  Asynchronous faults
 *    surface at the caller's next synchronisation.
 *  - Arguments are validated on the host before any HIP call; a non-zero
 *    return means nothing was enqueued (except BSG_ERR_HIP, reported when a
 *    launch fails).  Validation never dereferences device pointers.
 *  - Sign buffers and workspaces must be 16-byte aligned; every other
 *    pointer must be aligned to its element size (BSG_ERR_ALIGN).
 *  - N (the input dimension) must be a positive multiple of 32; M >= 0; an
 *    M of 0 is a no-op returning BSG_OK.  Each product addresses its
 *    operands with 32-bit offsets: K*M, N*B and K*N must stay below 2^30
 *    (BSG_ERR_SHAPE otherwise).
 *
 * Logical sign layout: word w of row m of base k holds columns 32w..32w+31,
 * bit j of the word is column 32w+j.  A set bit is +1, a clear bit is -1.
 *
 * Device sign layout (what every kernel reads), for K bases of an M x N
 * matrix with ND = N/32 words per row:
 *   MP = round_up(M, 64), NDP = round_up(ND, 4)     padded rows, words per row
 *   plane = MP*NDP                                  words per base
 *   offset(k, m, w) = k*plane + (m/64)*64*NDP + (w/4)*256 + (m%64)*4 + w%4
 * i.e. tiles of 64 rows x 4 words (128 columns), each one contiguous KiB
 * stored row-major, one after the other along the words of a 64-row block,
 * then the next row block.  Rows M..MP-1 and words ND..NDP-1 are padding and
 * hold zero words (every writer of this layout writes them).  A wavefront
 * reads a tile with one 16-byte load per lane.
 */
#ifndef BSG_H
#define BSG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSG_API __attribute__((visibility("default")))

typedef int32_t bsg_status;

#define BSG_OK 0
#define BSG_ERR_NULL (-1)        /* a required pointer is NULL */
#define BSG_ERR_SHAPE (-2)       /* a size is negative, N % 32 != 0, a count out of range */
#define BSG_ERR_DTYPE (-3)       /* unknown dtype code */
#define BSG_ERR_ALIGN (-4)       /* a device pointer is not 16-byte aligned */
#define BSG_ERR_UNSUPPORTED (-5) /* a valid combination this build does not implement */
#define BSG_ERR_WORKSPACE (-6)   /* workspace missing or smaller than required */
#define BSG_ERR_HIP (-7)         /* a HIP runtime call or kernel launch failed */

/* Activation / input dtypes. */
#define BSG_F32 0
#define BSG_F16 1
#define BSG_BF16 2

/* bsq_pack flags. */
#define BSG_PACK_COLSCALE 1

/* Version of this ABI (bumped on any incompatible change). */
BSG_API int32_t bsg_abi_version(void);

/* Static, NUL-terminated description of a status code. */
BSG_API const char* bsg_status_string(bsg_status status);

/* The HIP error behind the last BSG_ERR_HIP returned on the calling host
 * thread (hipSuccess = 0 if none yet), and its description. */
BSG_API int32_t bsg_last_hip_error(void);
BSG_API const char* bsg_last_hip_error_string(void);

/* Number of uint32 words of a device sign buffer for K bases of an M x N
 * matrix (K * plane, see the layout above).  0 if a size is invalid. */
BSG_API size_t bsg_layout_words(int K, int M, int N);

/* Word offset of logical word w of row m of base k in the device layout, or
 * -1 if an index is out of range.  A pure host function. */
BSG_API int64_t bsg_layout_word_offset(int K, int M, int N, int k, int m, int w);

/* Device workspace bytes needed by binlr_apply: z = alpha_r (.) (V x), fp32
 * [r][B].  No initial contents are required.  Calls that overlap in time
 * must not share a workspace. */
BSG_API size_t bsg_binlr_workspace_bytes(int r, int M, int N, int B);

/* ------------------------------------------------------------------ */
/* Packing (offline).                                                  */
/* ------------------------------------------------------------------ */

/* Device workspace bytes bsq_pack needs: the fp64 residual, 8*M*N bytes. */
BSG_API size_t bsq_pack_workspace_bytes(int M, int N);

/*
 * bsq_pack -- greedy residual binary bases (FluxBin Sec. 2 and Sec. 3.1).
 * For k = 1..K, on the residual R (R = W at first, kept in fp64):
 *   B_k      = sign(R), sign(0) = +1                  -> bits (device layout)
 *   alpha_k  = fp32( sum_n |R[m,n]| / N )   per row   -> alpha [K][M] fp32
 *   c_k[n]   = fp16(fp32( sum_m alpha_k[m] |R[m,n]| / sum_m alpha_k[m]^2 ))
 *              (least-squares column scale, 1 if the denominator is 0) when
 *              flags has BSG_PACK_COLSCALE, else 1   -> colscale [K][N] fp16
 *   R       <- R - alpha_k[m] c_k[n] B_k[m,n]         (stored, rounded scales)
 * Every sum runs in fp64 in ascending index order, so the result is bit-exact
 * with a sequential CPU implementation.
 *   W         (device) fp32 [M][N], row-major; must hold no NaN (not checked)
 *   bits      (device) uint32 [bsg_layout_words(K, M, N)]
 *   alpha     (device) fp32 [K][M]
 *   colscale  (device) uint16 (fp16 bits) [K][N]; required iff COLSCALE
 *   workspace (device) >= bsq_pack_workspace_bytes(M, N)
 * 1 <= K <= 8.
 */
BSG_API bsg_status bsq_pack(const float* W, int M, int N, int K, int flags,
                    uint32_t* bits, float* alpha, uint16_t* colscale,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * bsq_pack_signs -- pack a real matrix S (device, fp32 [M][N]) into device
 * sign layout with K = 1: bit = [S >= 0].  Used for the +-1 low-rank
 * factors: U as an M x r matrix, V as an r x N matrix (BiLoCo "The core
 * idea").  N % 32 == 0.
 */
BSG_API bsg_status bsq_pack_signs(const float* S, int M, int N, uint32_t* bits, void* stream);

/*
 * bsq_absmean -- activation statistic for choosing protected rows (BiSCo,
 * "Sensitivity Protection"): xbar[n] = fp32( sum_s |X[s][n]| / S ) in fp64,
 * s ascending.  X (device) fp32 [S][N]; xbar (device) fp32 [N].  Any N > 0.
 */
BSG_API bsg_status bsq_absmean(const float* X, int S, int N, float* xbar, void* stream);

/* Device workspace bytes bsq_salient needs. */
BSG_API size_t bsq_salient_workspace_bytes(int M, int N);

/*
 * bsq_salient -- protected int8 rows (BiSCo, "Sensitivity Protection"):
 *   score_m = sum_n |W[m,n]| xbar[n]          (fp64, n ascending)
 *   rows    = the ns highest scores, ties to the smaller m, ascending
 *   s_i     = fp16(fp32( max_n |W[m,n]| / 127 ))         symmetric per row
 *   q[i,n]  = clamp(rint_even(W[m,n] / s_i), -127, 127), 0 if s_i == 0
 *   alpha[k][m] = 0 for every base k on the kept rows (the int8 row replaces
 *   the binary row; the sign bits stay).
 *   W (device) fp32 [M][N]; xbar (device) fp32 [N]; rows (device) int32 [ns];
 *   q (device) int8 [ns][N]; s_f16 (device) uint16 [ns];
 *   alpha (device) fp32 [K][M] (updated in place; may be NULL when K == 0).
 * 0 <= ns <= M.  Any N > 0.
 */
BSG_API bsg_status bsq_salient(const float* W, int M, int N, const float* xbar, int ns,
                       int32_t* rows, int8_t* q, uint16_t* s_f16,
                       float* alpha, int K, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * bsq_quantize_i8 -- symmetric per-column int8 quantisation of activations
 * for the int8 mode: sx[b] = fp32(max_n |x[n,b]| / 127) (fp32 division),
 * xq = clamp(rint_even(fp32(x / sx)), -127, 127), 0 if sx == 0.
 *   x (device) [N][B] of dtype x_dtype; xq (device) int8 [N][B];
 *   sx (device) fp32 [B].  Any N > 0, B >= 1.
 */
BSG_API bsg_status bsq_quantize_i8(const void* x, int x_dtype, int N, int B,
                           int8_t* xq, float* sx, void* stream);

/* Device-side layout conversions (K bases, M x N, N % 32 == 0).
 * logical (device) uint32 [K][M][N/32]; bits (device) device layout. */
BSG_API bsg_status bsg_logical_to_layout(const uint32_t* logical, int K, int M, int N,
                                 uint32_t* bits, void* stream);
BSG_API bsg_status bsg_layout_to_logical(const uint32_t* bits, int K, int M, int N,
                                 uint32_t* logical, void* stream);

/* ------------------------------------------------------------------ */
/* The decode-time product (hot path).                                 */
/* ------------------------------------------------------------------ */

/*
 * bs_gemv -- binary-base product (FluxBin Sec. 3.1 and Sec. 3.2):
 *   y[m,b] (= or +=) sum_k alpha[k][m] * sum_n (2 bit_k(m,n) - 1) * c_k[n] * x[n,b]
 *   bits      (device) device sign layout, K bases of M x N
 *   alpha     (device) fp32 [K][M]
 *   colscale  (device) fp16 bits [K][N], or NULL for c == 1
 *   x         (device) [N][B] (element (n, b) at n*B + b) of dtype x_dtype
 *   y         (device) fp32 [M][B]; overwritten when accumulate == 0,
 *             added to otherwise
 * 1 <= K <= 8, 1 <= B <= 64.  Accumulation is fp32 in a fixed order (the
 * result does not depend on scheduling); it is within
 * 2e-3 * sum_k |alpha_k[m]| * sum_n |c_k[n] x[n,b]| of the exact value.
 * With B >= 4 columns of bf16 or fp16 x and no column scales the product
 * runs on the matrix cores (one launch per 16 batch columns and per 4
 * bases; products exact, sums fp32, within 2e-4 of the same bound).
 * Needs no workspace: every output row is reduced inside one workgroup.
 */
BSG_API bsg_status bs_gemv(const uint32_t* bits, int K, int M, int N, const float* alpha,
                   const uint16_t* colscale, const void* x, int x_dtype, int B,
                   float* y, int accumulate, void* stream);

/*
 * bsq_pack_grouped -- bsq_pack with one row scale per row and per group of g
 * consecutive columns (FluxBin Sec. 3.1: a row scale per weight group;
 * g = 128 in its Kb-g128 configurations; App. C.2: scales stored in fp16):
 *   alpha_k[m][j] = fp16(fp32( sum_{n in group j} |R[m,n]| / g ))
 *   c_k[n] = fp16(fp32( sum_m a_k[m][j] |R[m,n]| / sum_m a_k[m][j]^2 ))
 *            with a the stored fp16 scales of the group j of column n
 *            (BSG_PACK_COLSCALE; 1 when the denominator is 0)
 *   R <- R - a_k[m][j(n)] c_k[n] B_k[m,n]
 *   alpha     (device) out: fp16 [K][N/g][M], group-major (alpha_k[m][j] at
 *             (k * (N/g) + j) * M + m: the scales of one group are contiguous
 *             over the rows, so a wavefront's rows read them in one access)
 *   other arguments as bsq_pack; workspace >= bsq_pack_grouped_workspace_bytes.
 * g a power of two >= 64 dividing N (N % 32 == 0).  fp64 sums in ascending
 * order: bit-exact with a sequential double-precision implementation of the
 * recipe.  Same as bsq_pack_hybrid with s = 0.
 */
BSG_API size_t bsq_pack_grouped_workspace_bytes(int M, int N, int g);
BSG_API bsg_status bsq_pack_grouped(const float* W, int M, int N, int K, int g, int flags, uint32_t* bits,
                                    uint16_t* alpha, uint16_t* colscale, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * bsq_pack_hybrid -- bsq_pack_grouped plus K salient-column bases (FluxBin
 * Sec. 3.1 "Structural Saliency Search": hybrid bases, extra bases on s
 * salient columns per group of g; Sec. 3.2 Virtual Columnar Mapping: the
 * sparse salient columns stored as a dense physical matrix, read through an
 * index list; Sec. 4: the Kb-sS-gG configurations use the same K for both).
 * After the K global bases, the residual at the S = s * (N/g) columns idx[p]
 * (normally the s salient columns of group j at p = j*s .. j*s+s-1, chosen
 * by the caller) is gathered into Rs [M][S] and fitted by the same grouped
 * recipe with groups of s physical columns:
 *   sbits     (device) out: K bases of M x S signs in the device layout with
 *             ceil(S/32) words per row (bits at or beyond S clear)
 *   salpha    (device) out: fp16 row scales, word-grouped: the 32/s scales of
 *             one sign word of one row adjacent, (k, w, m, t) at
 *             ((k * ceil(S/32) + w) * M + m) * (32/s) + t for group
 *             j = w * (32/s) + t (slots past the last group are 0); 8-byte aligned
 *   scolscale (device) out: fp16 [K][S] (with BSG_PACK_COLSCALE)
 *   idx       (device) in: int32 [S], 16-byte aligned; an index outside
 *             [0, N) reads a zero column
 * s = 8, 16 or 32; s = 0 packs the global bases only.  workspace >=
 * bsq_pack_hybrid_workspace_bytes (0 for invalid sizes).  Bit-exact as
 * bsq_pack_grouped.
 */
BSG_API size_t bsq_pack_hybrid_workspace_bytes(int M, int N, int g, int s);
BSG_API bsg_status bsq_pack_hybrid(const float* W, int M, int N, int K, int g, int s, const int32_t* idx, int flags,
                                   uint32_t* bits, uint16_t* alpha, uint16_t* colscale, uint32_t* sbits,
                                   uint16_t* salpha, uint16_t* scolscale, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * bs_gemv_grouped -- bs_gemv with group-wise row scales (FluxBin Sec. 3.1):
 *   y[m,b] (= or +=) sum_k sum_j alpha_k[m][j] *
 *                    sum_{n in group j} (2 bit_k(m,n) - 1) * c_k[n] * x[n,b]
 *   alpha     (device) fp16 [K][N/g][M], group-major as bsq_pack_grouped writes it
 *   other arguments as bs_gemv.
 * 1 <= K <= 4, g a power of two >= 64 dividing N, 1 <= B <= 64 (one launch
 * per batch column).  fp32 sums in a fixed order, within
 * 2e-3 * sum_k sum_j |alpha_k[m][j]| * sum_{n in j} |c_k[n] x[n,b]|.
 */
BSG_API bsg_status bs_gemv_grouped(const uint32_t* bits, int K, int M, int N, int g, const uint16_t* alpha,
                                   const uint16_t* colscale, const void* x, int x_dtype, int B, float* y,
                                   int accumulate, void* stream);

/*
 * bs_gemv_hybrid -- bs_gemv_grouped plus the salient-column bases of
 * bsq_pack_hybrid, in the same launch (FluxBin Sec. 3.2: the salient phase
 * runs through the same kernel, its activations gathered by the index list):
 *   y[m,b] += sum_k sum_j salpha_k[m][j] *
 *             sum_{i < s} (2 sbit_k(m, j*s+i) - 1) * sc_k[j*s+i] * x[idx[j*s+i], b]
 * Arguments as written by bsq_pack_hybrid; s = 8, 16 or 32 (0: no salient
 * branch, as bs_gemv_grouped).  Column scales on both branches or on
 * neither (BSG_ERR_SHAPE otherwise); scolscale 8-byte aligned.  Within the bs_gemv_grouped bound plus
 * the same term for the salient branch.
 */
BSG_API bsg_status bs_gemv_hybrid(const uint32_t* bits, int K, int M, int N, int g, const uint16_t* alpha,
                                  const uint16_t* colscale, const uint32_t* sbits, int s, const int32_t* idx,
                                  const uint16_t* salpha, const uint16_t* scolscale, const void* x, int x_dtype,
                                  int B, float* y, int accumulate, void* stream);

/*
 * bs_gemv_grouped_multi -- several bs_gemv_grouped products that share x
 * (e.g. the query, key and value projections in FluxBin's Kb-gG format), in
 * one launch at B = 1 (each workgroup looks up its projection's rows); for
 * B > 1 or one projection, a bs_gemv_grouped call each.
 *   projs[p].alpha: fp16 [K][N/g][projs[p].M], group-major, as bs_gemv_grouped
 * 1 <= P <= 8, 1 <= K <= 4, g as bs_gemv_grouped; column scales on every
 * projection or on none (BSG_ERR_SHAPE otherwise); M = 0 projections are
 * skipped.  Errors and bound as bs_gemv_grouped.
 */
typedef struct bsg_proj_grouped {
  const uint32_t* bits;
  const uint16_t* alpha;
  const uint16_t* colscale;
  float* y;
  int M;
} bsg_proj_grouped;
BSG_API bsg_status bs_gemv_grouped_multi(const bsg_proj_grouped* projs, int P, int K, int N, int g, const void* x,
                                         int x_dtype, int B, int accumulate, void* stream);

/*
 * bs_gemv_multi -- several bs_gemv products that share x, in one launch
 * (projections that read the same activations, e.g. the query, key and
 * value projections, or the two projections of a gated MLP):
 *   for each i < P:  projs[i].y (= or +=) bs_gemv term of projs[i]
 *   projs     (host) P descriptors, read during the call only:
 *             bits (device layout, K bases of M x N), alpha fp32 [K][M],
 *             colscale fp16 [K][N] or NULL, y fp32 [M][B], M (>= 0)
 *   x         (device) [N][B] of dtype x_dtype, shared by all projections
 * 1 <= P <= 8; K, N, B, x and accumulate are common; colscale must be given
 * for every projection or for none (BSG_ERR_SHAPE otherwise).  Each y is
 * what bs_gemv would write, within the same bound (the fused plan may sum in
 * another order).  The grid holds the row blocks of every projection in
 * turn, so small projections share one launch and its latency.  With B > 1
 * batch columns one fused launch is made per 16 columns on the matrix-core
 * path (B % 4 == 0, x 8-byte aligned); otherwise the projections are
 * launched one after another.
 */
typedef struct bsg_proj {
  const uint32_t* bits;
  const float* alpha;
  const uint16_t* colscale;
  float* y;
  int M;
} bsg_proj;
BSG_API bsg_status bs_gemv_multi(const bsg_proj* projs, int P, int K, int N, const void* x, int x_dtype, int B,
                                 int accumulate, void* stream);

/*
 * bs_gemv_i8 -- the same product with int8 activations, exact in integers:
 *   acc[k][m][b] = sum_n (2 bit_k(m,n) - 1) * xq[n,b]            (int32, exact)
 *   y[m,b] (= or +=) sx[b] * sum_k alpha[k][m] * acc[k][m][b]    (fp32)
 *   xq (device) int8 [N][B]; sx (device) fp32 [B] (may be NULL iff y is NULL);
 *   acc (device) int32 [K][M][B] or NULL; y (device) fp32 [M][B] or NULL
 *   (at least one of acc, y).  No column scales in this mode.
 * 1 <= K <= 8, 1 <= B <= 64, N <= 2^24.
 */
BSG_API bsg_status bs_gemv_i8(const uint32_t* bits, int K, int M, int N, const float* alpha,
                      const int8_t* xq, const float* sx, int B, int32_t* acc,
                      float* y, int accumulate, void* stream);

/*
 * binlr_apply -- binary low-rank correction (BiLoCo "The core idea"):
 *   z[j,b]  = alpha_r[j] * sum_n sv(j,n) * x[n,b]      (fp32, in the workspace)
 *   y[m,b] += sum_j su(m,j) * z[j,b]
 *   U_bits  (device) device sign layout of the M x r sign matrix (row m holds
 *           u_j[m] for j = 0..r-1), K = 1
 *   V_bits  (device) device sign layout of the r x N sign matrix, K = 1
 *   alpha_r (device) fp16 bits [r]
 * r % 32 == 0 (pad unused ranks with alpha_r = 0).  y always accumulates.
 *   workspace (device) >= bsg_binlr_workspace_bytes(r, M, N, B)
 */
BSG_API bsg_status binlr_apply(const uint32_t* U_bits, const uint32_t* V_bits,
                       const uint16_t* alpha_r, int r, int M, int N,
                       const void* x, int x_dtype, int B, float* y,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * salient_int8_apply -- protected int8 rows (BiSCo "Sensitivity Protection"):
 *   y[rows[i], b] += s_i * sum_n q[i][n] * x[n,b]
 *   rows (device) int32 [ns], distinct, each in [0, M) (others are skipped);
 *   q (device) int8 [ns][N]; s_f16 (device) fp16 bits [ns].
 * Any N > 0 (q rows need no padding); 0 <= ns.  y always accumulates.
 */
BSG_API bsg_status salient_int8_apply(const int32_t* rows, int ns, const int8_t* q,
                              const uint16_t* s_f16, int M, int N,
                              const void* x, int x_dtype, int B, float* y,
                              void* stream);

/*
 * binlr_fit -- offline fit of the binary low-rank correction (BiLoCo,
 * "Finding the sign vectors" and "Joint refit"):
 *   R = W;  for j < r:  v = v_init[j];  `rounds` times { u = sign(R v);
 *           v = sign(R^T u) };  alpha_j = u^T R v / (M N);  R -= alpha_j u v^T
 *   then all coefficients refitted at once: alpha = argmin over alpha of
 *   || W - sum_j alpha_j u_j v_j^T ||_F, from the normal equations
 *   G alpha = c, G_ij = (u_i . u_j)(v_i . v_j), c_j = u_j^T W v_j (Gaussian
 *   elimination with partial pivoting; if a pivot falls below 1e-12 max G_ii
 *   the greedy coefficients are kept).  sign(0) = +1; the residual and all
 *   sums are fp64.
 *   W         (device) fp32 [M][N], row-major
 *   v_init    (device) start vectors, logical sign words [r][N/32]
 *             (bit 1 -> +1); the caller draws them
 *   U_bits    (device) out: device layout, M x rp signs (u_j is column j)
 *   V_bits    (device) out: device layout, rp x N signs (v_j is row j)
 *   alpha_r_f16 (device) out: fp16 [rp], the refitted coefficients
 *   alpha, alpha_greedy (host, optional) out: fp64 [r]
 *   sse       (host, optional) out: [0] = ||R||^2 after the greedy pass,
 *             [1] = the squared error with the refitted coefficients
 *             (from ||W||^2 - 2 alpha.c + alpha^T G alpha)
 *   solved    (host, optional) out: 1 if the refit was solved, else 0
 *   workspace (device, 256-byte aligned) >= binlr_fit_workspace_bytes(M, N, r)
 *             (8 M N bytes of fp64 residual plus O(r^2 + M r + N r))
 * rp = r rounded up to a multiple of 32; the padding components are u = v =
 * +1 with coefficient 0, so U_bits, V_bits, alpha_r_f16 and rp go straight
 * to binlr_apply / bsg_linear.  1 <= r <= 2048, 1 <= rounds <= 64,
 * N % 32 == 0.  Offline: the call synchronises the stream (the r x r system
 * is solved on the host) and returns when the outputs are written.
 */
BSG_API size_t binlr_fit_workspace_bytes(int M, int N, int r);
BSG_API bsg_status binlr_fit(const float* W, int M, int N, int r, int rounds, const uint32_t* v_init,
                             uint32_t* U_bits, uint32_t* V_bits, uint16_t* alpha_r_f16, double* alpha,
                             double* alpha_greedy, double* sse, int* solved, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * bsg_linear -- the whole layer in one pass over x: the binary bases
 * (FluxBin Sec. 3.1/3.2), the binary low-rank correction (BiLoCo "The core
 * idea") and the protected int8 rows (BiSCo-LLM "Sensitivity Protection"):
 *   y[m,b] (= or +=) bs_gemv term + sum_j su(m,j) alpha_r[j] (v_j . x_b)
 *                    + [m = rows[i]] s_i (q_i . x_b)
 * Arguments as in bs_gemv, binlr_apply and salient_int8_apply, with:
 *   U_bits, V_bits, alpha_r: all NULL with r == 0 (no correction), or all
 *     given with r > 0, r % 32 == 0;
 *   rows, q, s_f16: all NULL with ns == 0, or all given with ns > 0; rows
 *     strictly ascending, each in [0, M); q 16-byte aligned.
 *   workspace (device) >= bsg_linear_workspace_bytes(r, B) (may be NULL when
 *     that is 0).
 * Two launches when r > 0 (z = V x, then everything else in one kernel that
 * reads x once per workgroup), one otherwise.  Fixed-order fp32 sums; within
 * the sum of the three terms' bounds above.
 */
BSG_API size_t bsg_linear_workspace_bytes(int r, int B);
BSG_API bsg_status bsg_linear(const uint32_t* bits, int K, int M, int N, const float* alpha,
                      const uint16_t* colscale, const uint32_t* U_bits,
                      const uint32_t* V_bits, const uint16_t* alpha_r, int r,
                      const int32_t* rows, int ns, const int8_t* q,
                      const uint16_t* s_f16, const void* x, int x_dtype, int B,
                      float* y, int accumulate, void* workspace,
                      size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSG_H */
