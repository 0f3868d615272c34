/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU implementation of the binary sign-GEMV
 * path, written in double precision.  Only tests/, __graft_entry__.smoke()
 * and bench.py's cpu_baseline leg may load it.  It shares no code, header,
 * table or helper with the HIP library under bit_gemv_packed_amd/csrc; the
 * physical-layout formula below is a second, independent implementation of
 * the formula documented in include/bsg.h.
 *
 * Sources (the web pages this path is built from):
 *  [BiLoCo]  "BiLoCo: Binary Low-Rank Corrections for Post-Training
 *            Quantization", sections "The core idea" (alpha*u*(v.x) computed
 *            with additions only; worked example), "Finding the sign
 *            vectors" (greedy alternating signs, error-minimising
 *            coefficient) and "Joint refit".
 *  [FluxBin] "FluxBin: Flexible LUT-based Ultra-low-bit LLM Inference by
 *            Algorithm-Kernel Synergy", Sec. 2 (greedy residual binary bases,
 *            R(k) = R(k-1) - alpha_k B(k)), Sec. 3.1 (decoupled row/column
 *            scales; quantised matrix is the sum of the bases), Sec. 3.2
 *            Stage 1 (bits map to signs by 2b-1).
 *  [BiSCo]   "BiSCo-LLM: Lookup-Free Binary Spherical Coding ...", technical
 *            summary, "Sensitivity Protection" (about 1% of sensitive channels
 *            chosen from activation statistics and weight magnitudes, stored
 *            in 8 bits apart from the binary payload).
 *
 * Conventions (readings where the pages are silent; each is listed in
 * the design doc):
 *  - logical bits: word w of row m of base k holds columns 32w..32w+31, bit j
 *    of the word is column 32w+j (LSB first); a set bit is +1, a clear bit -1.
 *  - every sum runs in double, in ascending index order, one bit at a time.
 *  - fp16 / fp32 roundings are round-to-nearest-even.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no fast-math, no FMA
 * contraction, so every rounding below is the one written).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#define OR_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------ */
/* IEEE-754 binary16 conversions, written from the format definition.  */
/* ------------------------------------------------------------------ */

/* binary16 bit pattern -> exact double value. */
OR_API double or_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int exp = (h >> 10) & 0x1f;
  int frac = h & 0x3ff;
  double v;
  if (exp == 0) {
    v = ldexp((double)frac, -24);                 /* subnormal: frac * 2^-24 */
  } else if (exp == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp((double)(frac | 0x400), exp - 25);  /* 1.frac * 2^(exp-15) */
  }
  return sign ? -v : v;
}

/* binary32 value -> binary16 bit pattern, round to nearest, ties to even. */
OR_API uint16_t or_f32_to_f16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t exp = (u >> 23) & 0xffu;
  uint32_t man = u & 0x7fffffu;
  if (exp == 0xff) return (uint16_t)(sign | 0x7c00u | (man ? 0x200u : 0u));
  /* value = 1.man * 2^(exp-127) (normal) or 0.man * 2^-126 (subnormal) */
  if (exp == 0) return sign;  /* fp32 subnormals are far below fp16's least subnormal */
  int e = (int)exp - 127;     /* unbiased exponent */
  uint32_t sig = man | 0x800000u; /* 24-bit significand, value = sig * 2^(e-23) */
  if (e > 15) return (uint16_t)(sign | 0x7c00u);   /* overflow -> inf */
  int shift;                   /* bits of sig to drop */
  uint32_t base_exp;
  if (e >= -14) {              /* fp16 normal range: keep 11 significant bits */
    shift = 13;
    base_exp = (uint32_t)(e + 15);
  } else {                     /* fp16 subnormal: value = q * 2^-24 */
    shift = 13 + (-14 - e);
    base_exp = 0;
    if (shift > 24) return sign; /* rounds to zero (below half the least subnormal) */
  }
  uint32_t q = sig >> shift;
  uint32_t rem = sig & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) q += 1u;
  uint32_t out;
  if (base_exp == 0) {
    out = q;                   /* q <= 0x400; 0x400 is the least normal, encoded correctly */
  } else {
    /* q in [0x400, 0x800]; carry into the exponent when it reaches 0x800 */
    if (q >= 0x800u) { q >>= 1; base_exp += 1; }
    if (base_exp >= 31) return (uint16_t)(sign | 0x7c00u);
    out = (base_exp << 10) | (q & 0x3ffu);
  }
  return (uint16_t)(sign | out);
}

/* ------------------------------------------------------------------ */
/* The product itself.                                                 */
/* ------------------------------------------------------------------ */

static inline int or_bit(const uint32_t* row_words, int n) {
  return (int)((row_words[n >> 5] >> (n & 31)) & 1u);
}

/*
 * Binary-base product [FluxBin Sec. 3.1, Sec. 3.2 Stage 1]:
 *   y[m,b] = sum_k alpha[k][m] * sum_n (2 bit_k(m,n) - 1) * c_k[n] * x[n,b]
 * bits: logical [K][M][ceil(N/32)]; alpha [K][M]; colscale [K][N] or NULL
 * (then c == 1); x [N][B]; y [M][B] (overwritten).  Any N >= 0.
 */
OR_API void or_sign_gemv(const uint32_t* bits, int K, int M, int N,
                         const double* alpha, const double* colscale,
                         const double* x, int B, double* y) {
  int nd = (N + 31) / 32;
  for (int m = 0; m < M; ++m) {
    for (int b = 0; b < B; ++b) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k) {
        const uint32_t* row = bits + ((size_t)k * M + m) * nd;
        double s = 0.0;
        for (int n = 0; n < N; ++n) {
          double sgn = or_bit(row, n) ? 1.0 : -1.0;
          double c = colscale ? colscale[(size_t)k * N + n] : 1.0;
          s += sgn * c * x[(size_t)n * B + b];
        }
        acc += alpha[(size_t)k * M + m] * s;
      }
      y[(size_t)m * B + b] = acc;
    }
  }
}

/*
 * Binary low-rank correction [BiLoCo, "The core idea"]:
 *   z[j,b]  = alpha_r[j] * sum_n sv(j,n) * x[n,b]
 *   y[m,b]  = sum_j su(m,j) * z[j,b]
 * U: logical [M][ceil(r/32)] (row m holds u_j[m] for j = 0..r-1),
 * V: logical [r][ceil(N/32)], alpha_r [r]; y [M][B] overwritten.
 */
OR_API void or_binlr(const uint32_t* ubits, const uint32_t* vbits,
                     const double* alpha_r, int r, int M, int N,
                     const double* x, int B, double* y) {
  int nd = (N + 31) / 32, rd = (r + 31) / 32;
  double* z = (double*)calloc((size_t)(r > 0 ? r : 1) * (B > 0 ? B : 1), sizeof(double));
  for (int j = 0; j < r; ++j)
    for (int b = 0; b < B; ++b) {
      double s = 0.0;
      for (int n = 0; n < N; ++n)
        s += (or_bit(vbits + (size_t)j * nd, n) ? 1.0 : -1.0) * x[(size_t)n * B + b];
      z[(size_t)j * B + b] = alpha_r[j] * s;
    }
  for (int m = 0; m < M; ++m)
    for (int b = 0; b < B; ++b) {
      double s = 0.0;
      for (int j = 0; j < r; ++j)
        s += (or_bit(ubits + (size_t)m * rd, j) ? 1.0 : -1.0) * z[(size_t)j * B + b];
      y[(size_t)m * B + b] = s;
    }
  free(z);
}

/*
 * Protected int8 rows [BiSCo, "Sensitivity Protection"]:
 *   y[rows[i], b] = s[i] * sum_n q[i][n] * x[n,b]; every other row is 0.
 * y [M][B] overwritten.  Rows outside [0, M) are skipped.
 */
OR_API void or_salient(const int32_t* rows, int ns, const int8_t* q, const double* s,
                       int M, int N, const double* x, int B, double* y) {
  memset(y, 0, sizeof(double) * (size_t)M * (B > 0 ? B : 0));
  for (int i = 0; i < ns; ++i) {
    int m = rows[i];
    if (m < 0 || m >= M) continue;
    for (int b = 0; b < B; ++b) {
      double acc = 0.0;
      for (int n = 0; n < N; ++n) acc += (double)q[(size_t)i * N + n] * x[(size_t)n * B + b];
      y[(size_t)m * B + b] += s[i] * acc;
    }
  }
}

/*
 * Integer sign product for int8 activations (exact):
 *   acc[k][m][b] = sum_n (2 bit_k(m,n) - 1) * xq[n,b]   (int64)
 */
OR_API void or_sign_gemv_i8(const uint32_t* bits, int K, int M, int N,
                            const int8_t* xq, int B, int64_t* acc) {
  int nd = (N + 31) / 32;
  for (int k = 0; k < K; ++k)
    for (int m = 0; m < M; ++m) {
      const uint32_t* row = bits + ((size_t)k * M + m) * nd;
      for (int b = 0; b < B; ++b) {
        int64_t s = 0;
        for (int n = 0; n < N; ++n)
          s += (or_bit(row, n) ? 1 : -1) * (int64_t)xq[(size_t)n * B + b];
        acc[((size_t)k * M + m) * B + b] = s;
      }
    }
}

/*
 * Symmetric per-column int8 quantisation of activations (the caller's rule
 * for the int8 mode; a reading, the pages fix none):
 *   sx[b] = fp32( max_n |x[n,b]| / 127 )     (fp32 division)
 *   xq    = clamp( rint_half_even( fp32(x / sx) ), -127, 127 ), 0 if sx == 0
 * x holds fp32 values [N][B].
 */
OR_API void or_quantize_i8(const float* x, int N, int B, int8_t* xq, float* sx) {
  for (int b = 0; b < B; ++b) {
    float mx = 0.0f;
    for (int n = 0; n < N; ++n) {
      float a = fabsf(x[(size_t)n * B + b]);
      if (a > mx) mx = a;
    }
    volatile float s = mx / 127.0f;
    sx[b] = s;
    for (int n = 0; n < N; ++n) {
      int8_t v = 0;
      if (s != 0.0f) {
        volatile float t = x[(size_t)n * B + b] / s;
        float r = nearbyintf(t);  /* default rounding mode: nearest, ties to even */
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        v = (int8_t)r;
      }
      xq[(size_t)n * B + b] = v;
    }
  }
}

/* ------------------------------------------------------------------ */
/* Packing (offline): greedy residual binary bases.                     */
/* ------------------------------------------------------------------ */

/*
 * Greedy residual bases [FluxBin Sec. 2, QBB/DB-LLM residual; Sec. 3.1 row
 * and column scales], in the pages' order, one base at a time:
 *   R <- W
 *   for k = 1..K:
 *     B_k = sign(R) with sign(0) = +1                     (bit = [R >= 0])
 *     alpha_k[m] = fp32( (sum_n |R[m,n]|) / N )            (error-minimising
 *                  row scale for a sign matrix: mean absolute value)
 *     if colscale: c_k[n] = fp16(fp32( num_n / den )),
 *                  num_n = sum_m alpha_k[m] |R[m,n]|, den = sum_m alpha_k[m]^2
 *                  (least-squares column scale given alpha_k and B_k;
 *                   c = 1 when den == 0), else c_k = 1
 *     R <- R - alpha_k[m] * c_k[n] * B_k[m,n]   (with the stored, rounded
 *                                               alpha and c)
 * Outputs: logical bits [K][M][ceil(N/32)] (padding bits zero), alpha fp32
 * [K][M], colscale fp16 bits [K][N] (only written when with_colscale).
 * Returns 0, or -1 on allocation failure, -2 on a NaN in W.
 */
OR_API int or_pack(const float* W, int M, int N, int K, int with_colscale,
                   uint32_t* bits, float* alpha, uint16_t* colscale) {
  int nd = (N + 31) / 32;
  size_t mn = (size_t)M * N;
  double* R = (double*)malloc(sizeof(double) * (mn ? mn : 1));
  if (!R) return -1;
  for (size_t i = 0; i < mn; ++i) {
    if (isnan(W[i])) { free(R); return -2; }
    R[i] = (double)W[i];
  }
  memset(bits, 0, sizeof(uint32_t) * (size_t)K * M * nd);
  double* cdbl = (double*)malloc(sizeof(double) * (N > 0 ? N : 1));
  for (int k = 0; k < K; ++k) {
    uint32_t* bk = bits + (size_t)k * M * nd;
    float* ak = alpha + (size_t)k * M;
    /* 1. signs */
    for (int m = 0; m < M; ++m)
      for (int n = 0; n < N; ++n)
        if (R[(size_t)m * N + n] >= 0.0) bk[(size_t)m * nd + (n >> 5)] |= 1u << (n & 31);
    /* 2. row scales */
    for (int m = 0; m < M; ++m) {
      double s = 0.0;
      for (int n = 0; n < N; ++n) s += fabs(R[(size_t)m * N + n]);
      ak[m] = (float)(N > 0 ? s / (double)N : 0.0);
    }
    /* 3. column scales */
    for (int n = 0; n < N; ++n) cdbl[n] = 1.0;
    if (with_colscale) {
      double den = 0.0;
      for (int m = 0; m < M; ++m) den += (double)ak[m] * (double)ak[m];
      for (int n = 0; n < N; ++n) {
        uint16_t h;
        if (den == 0.0) {
          h = 0x3c00u; /* 1.0 */
        } else {
          double num = 0.0;
          for (int m = 0; m < M; ++m) num += (double)ak[m] * fabs(R[(size_t)m * N + n]);
          h = or_f32_to_f16((float)(num / den));
        }
        colscale[(size_t)k * N + n] = h;
        cdbl[n] = or_f16_to_f64(h);
      }
    }
    /* 4. residual */
    for (int m = 0; m < M; ++m)
      for (int n = 0; n < N; ++n) {
        double sgn = (bk[(size_t)m * nd + (n >> 5)] >> (n & 31)) & 1u ? 1.0 : -1.0;
        double t = (double)ak[m] * cdbl[n];   /* exact: 24-bit x 11-bit significands */
        R[(size_t)m * N + n] = R[(size_t)m * N + n] - t * sgn;
      }
  }
  free(cdbl);
  free(R);
  return 0;
}

/*
 * Pack an arbitrary real matrix into logical sign bits: bit = [S >= 0].
 * Used for the +-1 low-rank factors U [M][r] and V [r][N].
 */
OR_API void or_pack_signs(const float* S, int M, int N, uint32_t* bits) {
  int nd = (N + 31) / 32;
  memset(bits, 0, sizeof(uint32_t) * (size_t)M * nd);
  for (int m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n)
      if (S[(size_t)m * N + n] >= 0.0f) bits[(size_t)m * nd + (n >> 5)] |= 1u << (n & 31);
}

/*
 * Activation statistic for choosing protected rows [BiSCo, "Sensitivity
 * Protection": activation statistics]:  xbar[n] = fp32( sum_s |X[s][n]| / S ).
 * X holds S calibration vectors of N fp32 values.
 */
OR_API void or_absmean(const float* X, int S, int N, float* xbar) {
  for (int n = 0; n < N; ++n) {
    double s = 0.0;
    for (int i = 0; i < S; ++i) s += fabs((double)X[(size_t)i * N + n]);
    xbar[n] = (float)(S > 0 ? s / (double)S : 0.0);
  }
}

/*
 * Protected rows [BiSCo, "Sensitivity Protection"]: score each output row by
 * weight magnitude times activation statistic, keep the ns highest as int8.
 *   score_m = sum_n |W[m,n]| * xbar[n]              (double, n ascending)
 *   rows    = the ns largest scores, ties to the smaller m, stored ascending
 *   s_i     = fp16(fp32( max_n |W[m,n]| / 127 ))     (symmetric, per row)
 *   q[i,n]  = clamp(rint_half_even(W[m,n] / s_i), -127, 127), 0 if s_i == 0
 *   alpha[k][m] = 0 for every base k on the kept rows (the int8 row replaces
 *   the binary row).
 * Selection is by plain repeated maximum search (O(ns*M)).
 * Returns 0, -1 if ns is out of range.
 */
OR_API int or_salient_select(const float* W, int M, int N, const float* xbar, int ns,
                             int32_t* rows, int8_t* q, uint16_t* s_f16,
                             float* alpha, int K) {
  if (ns < 0 || ns > M) return -1;
  double* score = (double*)malloc(sizeof(double) * (M > 0 ? M : 1));
  char* taken = (char*)calloc(M > 0 ? M : 1, 1);
  for (int m = 0; m < M; ++m) {
    double s = 0.0;
    for (int n = 0; n < N; ++n) s += fabs((double)W[(size_t)m * N + n]) * (double)xbar[n];
    score[m] = s;
  }
  for (int i = 0; i < ns; ++i) {
    int best = -1;
    for (int m = 0; m < M; ++m) {
      if (taken[m]) continue;
      if (best < 0 || score[m] > score[best]) best = m;  /* strict: ties keep the smaller m */
    }
    taken[best] = 1;
  }
  int i = 0;
  for (int m = 0; m < M; ++m) {
    if (!taken[m]) continue;
    rows[i] = m;
    float mx = 0.0f;
    for (int n = 0; n < N; ++n) {
      float a = fabsf(W[(size_t)m * N + n]);
      if (a > mx) mx = a;
    }
    uint16_t h = or_f32_to_f16((float)((double)mx / 127.0));
    s_f16[i] = h;
    double sd = or_f16_to_f64(h);
    for (int n = 0; n < N; ++n) {
      int8_t v = 0;
      if (sd != 0.0) {
        double r = nearbyint((double)W[(size_t)m * N + n] / sd);
        if (r > 127.0) r = 127.0;
        if (r < -127.0) r = -127.0;
        v = (int8_t)r;
      }
      q[(size_t)i * N + n] = v;
    }
    for (int k = 0; k < K; ++k) alpha[(size_t)k * M + m] = 0.0f;
    ++i;
  }
  free(taken);
  free(score);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Physical tile layout (second, independent implementation of the      */
/* formula documented in include/bsg.h).                               */
/* ------------------------------------------------------------------ */

/*
 * The device layout pads the rows of each base to a multiple of 64 and the
 * words of each row to a multiple of 4 (zero words), and stores the result
 * as tiles of 64 rows by 4 words (128 columns): a tile is 256 consecutive
 * words in row-major order; tiles follow each other along the words of a
 * 64-row block, then along the row blocks; the bases follow each other.
 */
static size_t or_round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

OR_API size_t or_layout_plane_words(int M, int N) {
  size_t nd = (size_t)(N + 31) / 32;
  return or_round_up((size_t)M, 64) * or_round_up(nd, 4);
}

OR_API size_t or_layout_offset(int K, int M, int N, int k, int m, int w) {
  (void)K;
  size_t ndp = or_round_up((size_t)(N + 31) / 32, 4);
  size_t block = (size_t)m / 64, row = (size_t)m % 64; /* row block, row in it */
  size_t tile = (size_t)w / 4, col = (size_t)w % 4;    /* tile along the row, word in it */
  return (size_t)k * or_layout_plane_words(M, N) + block * 64 * ndp + tile * 256 + row * 4 + col;
}

OR_API void or_logical_to_layout(const uint32_t* logical, int K, int M, int N, uint32_t* phys) {
  size_t nd = (size_t)(N + 31) / 32;
  memset(phys, 0, sizeof(uint32_t) * (size_t)K * or_layout_plane_words(M, N));
  for (int k = 0; k < K; ++k)
    for (int m = 0; m < M; ++m)
      for (size_t w = 0; w < nd; ++w)
        phys[or_layout_offset(K, M, N, k, m, (int)w)] = logical[((size_t)k * M + m) * nd + w];
}

OR_API void or_layout_to_logical(const uint32_t* phys, int K, int M, int N, uint32_t* logical) {
  size_t nd = (size_t)(N + 31) / 32;
  for (int k = 0; k < K; ++k)
    for (int m = 0; m < M; ++m)
      for (size_t w = 0; w < nd; ++w)
        logical[((size_t)k * M + m) * nd + w] = phys[or_layout_offset(K, M, N, k, m, (int)w)];
}

/*
 * Group-wise row scales [FluxBin Sec. 3.1: one row scale per weight group;
 * Sec. 4 setup: group size g = 128 in the Kb-g128 configurations; App. C.2:
 * every scale is stored in fp16].  The greedy residual recipe of or_pack on
 * a residual R [M][NC], with the row scale taken per row and per group of g
 * consecutive columns (g divides NC):
 *   alpha_k[m][j] = fp16(fp32( sum_{n in group j} |R[m,n]| / g ))
 *   if colscale: c_k[n] = fp16(fp32( num_n / den_j )),
 *                num_n = sum_m a_k[m][j] |R[m,n]|, den_j = sum_m a_k[m][j]^2
 *                with a the stored fp16 group scales, for the group j of
 *                column n (least squares given the group scales; c = 1 when
 *                den_j == 0), else c = 1
 *   R <- R - a_k[m][j(n)] * c_k[n] * B_k[m,n]     (after every base)
 * bits: logical [K][M][nd] words (nd >= ceil(NC/32); bits past NC clear);
 * alpha: fp16 bits [K][M][NC/g]; colscale fp16 bits [K][NC] or NULL.
 * cdbl: NC doubles of scratch.
 */
static void grouped_bases(double* R, int M, int NC, int nd, int K, int g, uint32_t* bits, uint16_t* alpha,
                          uint16_t* colscale, double* cdbl) {
  const int G = NC / g;
  for (int k = 0; k < K; ++k) {
    uint32_t* bk = bits + (size_t)k * M * nd;
    uint16_t* ak = alpha + (size_t)k * M * G;   /* ak[m * G + j] */
    for (int m = 0; m < M; ++m)
      for (int n = 0; n < NC; ++n)
        if (R[(size_t)m * NC + n] >= 0.0) bk[(size_t)m * nd + (n >> 5)] |= 1u << (n & 31);
    for (int m = 0; m < M; ++m)
      for (int j = 0; j < G; ++j) {
        double s = 0.0;
        for (int n = j * g; n < (j + 1) * g; ++n) s += fabs(R[(size_t)m * NC + n]);
        ak[(size_t)m * G + j] = or_f32_to_f16((float)(s / (double)g));
      }
    for (int n = 0; n < NC; ++n) cdbl[n] = 1.0;
    if (colscale) {
      for (int j = 0; j < G; ++j) {
        double den = 0.0;
        for (int m = 0; m < M; ++m) {
          const double a = or_f16_to_f64(ak[(size_t)m * G + j]);
          den += a * a;
        }
        for (int n = j * g; n < (j + 1) * g; ++n) {
          uint16_t h;
          if (den == 0.0) {
            h = 0x3c00u;
          } else {
            double num = 0.0;
            for (int m = 0; m < M; ++m) num += or_f16_to_f64(ak[(size_t)m * G + j]) * fabs(R[(size_t)m * NC + n]);
            h = or_f32_to_f16((float)(num / den));
          }
          colscale[(size_t)k * NC + n] = h;
          cdbl[n] = or_f16_to_f64(h);
        }
      }
    }
    for (int m = 0; m < M; ++m)
      for (int n = 0; n < NC; ++n) {
        double sgn = (bk[(size_t)m * nd + (n >> 5)] >> (n & 31)) & 1u ? 1.0 : -1.0;
        double t = or_f16_to_f64(ak[(size_t)m * G + n / g]) * cdbl[n];
        R[(size_t)m * NC + n] = R[(size_t)m * NC + n] - t * sgn;
      }
  }
}

/*
 * or_pack_grouped: grouped_bases on R = W [M][N].  alpha is fp16 bits
 * [K][M][N/g].  Returns 0, -1 on bad sizes or allocation failure, -2 on a
 * NaN in W.
 */
OR_API int or_pack_grouped(const float* W, int M, int N, int K, int g, int with_colscale,
                           uint32_t* bits, uint16_t* alpha, uint16_t* colscale) {
  if (g <= 0 || N % g != 0) return -1;
  const int nd = (N + 31) / 32;
  const size_t mn = (size_t)M * N;
  double* R = (double*)malloc(sizeof(double) * (mn ? mn : 1));
  double* cdbl = (double*)malloc(sizeof(double) * (N > 0 ? N : 1));
  if (!R || !cdbl) { free(R); free(cdbl); return -1; }
  for (size_t i = 0; i < mn; ++i) {
    if (isnan(W[i])) { free(R); free(cdbl); return -2; }
    R[i] = (double)W[i];
  }
  memset(bits, 0, sizeof(uint32_t) * (size_t)K * M * nd);
  grouped_bases(R, M, N, nd, K, g, bits, alpha, with_colscale ? colscale : NULL, cdbl);
  free(cdbl);
  free(R);
  return 0;
}

/*
 * Hybrid bases with salient-column refinement [FluxBin Sec. 3.1 "Structural
 * Saliency Search" (extra bases on the salient columns), Sec. 3.2 "Virtual
 * Columnar Mapping" (the sparse salient columns are stored as a dense
 * physical matrix; an index list gathers x and the scales), Sec. 4 setup
 * (Kb-sS-gG: the same base count K for both branches, s salient columns per
 * group of g)].  Reading (the pages give no equation for the refinement):
 *   1. the global branch: grouped_bases on R = W with K bases and groups of g;
 *   2. the salient branch: the residual left by step 1 at the S = s * (N/g)
 *      columns idx[0..S) (idx[j*s .. j*s+s) normally the salient columns of
 *      group j, chosen by the caller: the saliency search needs calibration
 *      Hessians) gathered into the dense matrix Rs[m][p] = R[m][idx[p]], and
 *      grouped_bases on Rs with K bases and groups of s physical columns.
 * sbits: logical [K][M][ceil(S/32)] (bits past S clear); salpha fp16 bits
 * [K][M][S/s]; scolscale fp16 bits [K][S] or NULL (with colscale).
 * Returns 0, -1 on bad sizes, an index outside [0, N) or allocation failure,
 * -2 on a NaN in W.
 */
OR_API int or_pack_hybrid(const float* W, int M, int N, int K, int g, int s, const int32_t* idx, int with_colscale,
                          uint32_t* bits, uint16_t* alpha, uint16_t* colscale, uint32_t* sbits, uint16_t* salpha,
                          uint16_t* scolscale) {
  if (g <= 0 || N % g != 0 || s <= 0 || s > g) return -1;
  const int nd = (N + 31) / 32, S = s * (N / g), nds = (S + 31) / 32;
  for (int p = 0; p < S; ++p)
    if (idx[p] < 0 || idx[p] >= N) return -1;
  const size_t mn = (size_t)M * N;
  double* R = (double*)malloc(sizeof(double) * (mn ? mn : 1));
  double* Rs = (double*)malloc(sizeof(double) * ((size_t)M * S > 0 ? (size_t)M * S : 1));
  double* cdbl = (double*)malloc(sizeof(double) * (N > 0 ? N : 1));
  if (!R || !Rs || !cdbl) { free(R); free(Rs); free(cdbl); return -1; }
  for (size_t i = 0; i < mn; ++i) {
    if (isnan(W[i])) { free(R); free(Rs); free(cdbl); return -2; }
    R[i] = (double)W[i];
  }
  memset(bits, 0, sizeof(uint32_t) * (size_t)K * M * nd);
  memset(sbits, 0, sizeof(uint32_t) * (size_t)K * M * nds);
  grouped_bases(R, M, N, nd, K, g, bits, alpha, with_colscale ? colscale : NULL, cdbl);
  for (int m = 0; m < M; ++m)
    for (int p = 0; p < S; ++p) Rs[(size_t)m * S + p] = R[(size_t)m * N + idx[p]];
  grouped_bases(Rs, M, S, nds, K, s, sbits, salpha, with_colscale ? scolscale : NULL, cdbl);
  free(cdbl);
  free(Rs);
  free(R);
  return 0;
}

/*
 * The product with group-wise row scales [FluxBin Sec. 3.1]:
 *   y[m,b] = sum_k sum_j alpha_k[m][j] sum_{n in group j} (2 bit_k(m,n) - 1) c_k[n] x[n,b]
 * alpha fp16 bits [K][M][N/g]; colscale fp16 bits [K][N] or NULL; x [N][B]
 * (double); y [M][B] double.  Sums in double, ascending order.
 */
OR_API void or_sign_gemv_grouped(const uint32_t* bits, int K, int M, int N, int g, const uint16_t* alpha,
                                 const uint16_t* colscale, const double* x, int B, double* y) {
  const int nd = (N + 31) / 32, G = N / g;
  for (int m = 0; m < M; ++m)
    for (int b = 0; b < B; ++b) {
      double tot = 0.0;
      for (int k = 0; k < K; ++k)
        for (int j = 0; j < G; ++j) {
          double acc = 0.0;
          for (int n = j * g; n < (j + 1) * g; ++n) {
            const int bit = (bits[((size_t)k * M + m) * nd + (n >> 5)] >> (n & 31)) & 1u;
            const double c = colscale ? or_f16_to_f64(colscale[(size_t)k * N + n]) : 1.0;
            acc += (bit ? 1.0 : -1.0) * c * x[(size_t)n * B + b];
          }
          tot += or_f16_to_f64(alpha[((size_t)k * M + m) * G + j]) * acc;
        }
      y[(size_t)m * B + b] = tot;
    }
}

/*
 * The hybrid product [FluxBin Sec. 3.2 VCM]: the global grouped product plus
 * the salient branch on the gathered activations,
 *   y[m,b] += sum_k sum_j salpha_k[m][j] sum_{i < s} (2 sbit_k(m, j*s+i) - 1)
 *                                        sc_k[j*s+i] x[idx[j*s+i], b]
 * (S = s * (N/g) physical salient columns; sbits logical [K][M][ceil(S/32)]).
 */
OR_API void or_sign_gemv_hybrid(const uint32_t* bits, int K, int M, int N, int g, const uint16_t* alpha,
                                const uint16_t* colscale, const uint32_t* sbits, int s, const int32_t* idx,
                                const uint16_t* salpha, const uint16_t* scolscale, const double* x, int B,
                                double* y) {
  or_sign_gemv_grouped(bits, K, M, N, g, alpha, colscale, x, B, y);
  const int G = N / g, S = s * G, nds = (S + 31) / 32;
  for (int m = 0; m < M; ++m)
    for (int b = 0; b < B; ++b) {
      double tot = 0.0;
      for (int k = 0; k < K; ++k)
        for (int j = 0; j < G; ++j) {
          double acc = 0.0;
          for (int p = j * s; p < (j + 1) * s; ++p) {
            const int bit = (sbits[((size_t)k * M + m) * nds + (p >> 5)] >> (p & 31)) & 1u;
            const double c = scolscale ? or_f16_to_f64(scolscale[(size_t)k * S + p]) : 1.0;
            acc += (bit ? 1.0 : -1.0) * c * x[(size_t)idx[p] * B + b];
          }
          tot += or_f16_to_f64(salpha[((size_t)k * M + m) * G + j]) * acc;
        }
      y[(size_t)m * B + b] += tot;
    }
}

/* ------------------------------------------------------------------ */
/* Offline fit of the binary low-rank correction.                       */
/* ------------------------------------------------------------------ */

/*
 * [BiLoCo, "Finding the sign vectors" and "Joint refit"]: rank-one sign
 * components found one at a time on the residual, then every coefficient
 * refitted at once.
 *   R = W                                             (double)
 *   for j = 0 .. r-1:
 *     v = the j-th given start vector (vinit row j; bit 1 -> +1, 0 -> -1)
 *     repeat `rounds` times:  u = sign(R v);  v = sign(R^T u)
 *                             (sign(0) = +1; sums in ascending index order)
 *     alpha_j = u^T R v / (M N)                       (the error-minimising
 *               coefficient of a +-1 rank-one term; with the last R^T u = b
 *               and v = sign(b) it equals sum_n |b_n| / (M N))
 *     R = R - alpha_j u v^T
 *   joint refit: alpha minimises || W - sum_j alpha_j u_j v_j^T ||_F, i.e.
 *     G alpha = c with G_ij = (u_i . u_j)(v_i . v_j), c_j = u_j^T W v_j,
 *     solved by Gaussian elimination with partial pivoting.  If a pivot is
 *     below 1e-12 * max_i G_ii the system counts as singular and the greedy
 *     coefficients are kept (reading: the pages do not treat that case).
 * The random start vectors are an input (drawn by the caller).
 * Out: ubits logical [M][ceil(r/32)] (bit j of row m = u_j[m]), vbits logical
 * [r][ceil(N/32)] (any N > 0), alpha_greedy[r], alpha[r] (refit), sse[0] = ||R||^2 after the
 * greedy pass, sse[1] = the squared error with the refitted coefficients.
 * Returns 1 if the refit was solved, 0 if it kept the greedy coefficients,
 * -1 on bad sizes.
 */
OR_API int or_binlr_fit(const float* W, int M, int N, int r, int rounds, const uint32_t* vinit,
                        uint32_t* ubits, uint32_t* vbits, double* alpha_greedy, double* alpha, double* sse) {
  if (M <= 0 || N <= 0 || r <= 0 || rounds < 1) return -1;
  const int nd = (N + 31) / 32, rd = (r + 31) / 32;
  double* R = (double*)malloc(sizeof(double) * (size_t)M * N);
  double* b = (double*)malloc(sizeof(double) * N);
  signed char* U = (signed char*)malloc((size_t)M * r);  /* U[m * r + j] = u_j[m] */
  signed char* V = (signed char*)malloc((size_t)r * N);  /* V[j * N + n] = v_j[n] */
  for (size_t i = 0; i < (size_t)M * N; ++i) R[i] = (double)W[i];
  for (int j = 0; j < r; ++j) {
    signed char* v = V + (size_t)j * N;
    for (int n = 0; n < N; ++n) v[n] = ((vinit[(size_t)j * nd + (n >> 5)] >> (n & 31)) & 1u) ? 1 : -1;
    for (int t = 0; t < rounds; ++t) {
      for (int m = 0; m < M; ++m) {
        double a = 0.0;
        for (int n = 0; n < N; ++n) a += R[(size_t)m * N + n] * (double)v[n];
        U[(size_t)m * r + j] = a >= 0.0 ? 1 : -1;
      }
      for (int n = 0; n < N; ++n) {
        double c = 0.0;
        for (int m = 0; m < M; ++m) c += R[(size_t)m * N + n] * (double)U[(size_t)m * r + j];
        b[n] = c;
        v[n] = c >= 0.0 ? 1 : -1;
      }
    }
    double num = 0.0;  /* u^T R v = sum_n b_n v_n */
    for (int n = 0; n < N; ++n) num += b[n] * (double)v[n];
    const double aj = num / ((double)M * (double)N);
    alpha_greedy[j] = aj;
    for (int m = 0; m < M; ++m)
      for (int n = 0; n < N; ++n) R[(size_t)m * N + n] -= aj * (double)U[(size_t)m * r + j] * (double)v[n];
  }
  double s0 = 0.0;
  for (size_t i = 0; i < (size_t)M * N; ++i) s0 += R[i] * R[i];
  sse[0] = s0;

  /* joint refit: normal equations, augmented matrix [G | c] */
  double* A = (double*)malloc(sizeof(double) * (size_t)r * (r + 1));
  double gmax = 0.0;
  for (int i = 0; i < r; ++i) {
    for (int j = 0; j < r; ++j) {
      long long du = 0, dv = 0;
      for (int m = 0; m < M; ++m) du += (long long)U[(size_t)m * r + i] * U[(size_t)m * r + j];
      for (int n = 0; n < N; ++n) dv += (long long)V[(size_t)i * N + n] * V[(size_t)j * N + n];
      A[(size_t)i * (r + 1) + j] = (double)du * (double)dv;
    }
    double c = 0.0;
    for (int m = 0; m < M; ++m) {
      double w = 0.0;
      for (int n = 0; n < N; ++n) w += (double)W[(size_t)m * N + n] * (double)V[(size_t)i * N + n];
      c += (double)U[(size_t)m * r + i] * w;
    }
    A[(size_t)i * (r + 1) + r] = c;
    if (A[(size_t)i * (r + 1) + i] > gmax) gmax = A[(size_t)i * (r + 1) + i];
  }
  int solved = 1;
  for (int k = 0; k < r && solved; ++k) {
    int p = k;
    for (int i = k + 1; i < r; ++i)
      if (fabs(A[(size_t)i * (r + 1) + k]) > fabs(A[(size_t)p * (r + 1) + k])) p = i;
    if (fabs(A[(size_t)p * (r + 1) + k]) < 1e-12 * gmax) {
      solved = 0;
      break;
    }
    if (p != k)
      for (int j = 0; j <= r; ++j) {
        double t = A[(size_t)k * (r + 1) + j];
        A[(size_t)k * (r + 1) + j] = A[(size_t)p * (r + 1) + j];
        A[(size_t)p * (r + 1) + j] = t;
      }
    for (int i = k + 1; i < r; ++i) {
      const double f = A[(size_t)i * (r + 1) + k] / A[(size_t)k * (r + 1) + k];
      for (int j = k; j <= r; ++j) A[(size_t)i * (r + 1) + j] -= f * A[(size_t)k * (r + 1) + j];
    }
  }
  if (solved) {
    for (int i = r - 1; i >= 0; --i) {
      double t = A[(size_t)i * (r + 1) + r];
      for (int j = i + 1; j < r; ++j) t -= A[(size_t)i * (r + 1) + j] * alpha[j];
      alpha[i] = t / A[(size_t)i * (r + 1) + i];
    }
  } else {
    for (int j = 0; j < r; ++j) alpha[j] = alpha_greedy[j];
  }
  double s1 = 0.0;
  for (int m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n) {
      double e = (double)W[(size_t)m * N + n];
      for (int j = 0; j < r; ++j) e -= alpha[j] * (double)U[(size_t)m * r + j] * (double)V[(size_t)j * N + n];
      s1 += e * e;
    }
  sse[1] = s1;

  memset(ubits, 0, sizeof(uint32_t) * (size_t)M * rd);
  memset(vbits, 0, sizeof(uint32_t) * (size_t)r * nd);
  for (int m = 0; m < M; ++m)
    for (int j = 0; j < r; ++j)
      if (U[(size_t)m * r + j] > 0) ubits[(size_t)m * rd + (j >> 5)] |= 1u << (j & 31);
  for (int j = 0; j < r; ++j)
    for (int n = 0; n < N; ++n)
      if (V[(size_t)j * N + n] > 0) vbits[(size_t)j * nd + (n >> 5)] |= 1u << (n & 31);
  free(A);
  free(V);
  free(U);
  free(b);
  free(R);
  return solved;
}

/* Array forms of the binary16 conversions. */
OR_API void or_f16_array_to_f64(const uint16_t* h, size_t n, double* out) {
  for (size_t i = 0; i < n; ++i) out[i] = or_f16_to_f64(h[i]);
}

OR_API void or_f32_array_to_f16(const float* f, size_t n, uint16_t* out) {
  for (size_t i = 0; i < n; ++i) out[i] = or_f32_to_f16(f[i]);
}
