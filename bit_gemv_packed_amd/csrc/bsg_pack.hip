// Offline packing on gfx950: greedy residual binary bases (FluxBin Sec. 2,
// Sec. 3.1), with per-row or group-wise fp16 row scales and the salient-
// column bases of its hybrid format (Sec. 3.1, 3.2), sign packing of the
// low-rank factors (BiLoCo "The core idea"), and the protected int8 rows
// (BiSCo "Sensitivity Protection").
//
// Every floating-point sum here runs in fp64 in ascending index order, with
// FMA contraction off, so the packed bits and scales are bit-exact with a
// sequential CPU implementation of the same recipe.  Row sums are made
// sequential per thread by staging 64x64 tiles of the residual in LDS
// (coalesced loads, one thread per row); column sums are naturally
// coalesced with one thread per column.
#include "bsg_internal.h"

#pragma clang fp contract(off)

namespace bsg {

constexpr int kT = 64;  // tile edge for row-sequential sums

__global__ void k_widen(const float* __restrict__ W, double* __restrict__ R, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    R[i] = (double)W[i];
}

// mode 0: out[m] = fp32(sum_n |R[m,n]| / N)                (row scale)
// mode 1: outd[m] = sum_n |W[m,n]| * xbar[n]  (W fp32)      (protected-row score)
template <int MODE>
__global__ void __launch_bounds__(kT) k_rowsum(const double* __restrict__ R, const float* __restrict__ W,
                                              const float* __restrict__ xbar, int M, int N,
                                              float* __restrict__ out, double* __restrict__ outd) {
  __shared__ double tile[kT][kT + 1];
  const int t = threadIdx.x;
  const int m0 = blockIdx.x * kT;
  double acc = 0.0;
  for (int n0 = 0; n0 < N; n0 += kT) {
    const int n = n0 + t;
    for (int i = 0; i < kT; ++i) {
      const int m = m0 + i;
      double v = 0.0;
      if (m < M && n < N) {
        if (MODE == 0) {
          v = fabs(R[(size_t)m * N + n]);
        } else {
          v = fabs((double)W[(size_t)m * N + n]) * (double)xbar[n];
        }
      }
      tile[i][t] = v;
    }
    __syncthreads();
    const int lim = min(kT, N - n0);
    for (int j = 0; j < lim; ++j) acc = acc + tile[t][j];
    __syncthreads();
  }
  const int m = m0 + t;
  if (m < M) {
    if (MODE == 0) out[m] = (float)(acc / (double)N);
    else if (MODE == 1) outd[m] = acc;
  }
}

// Sign bits of a row-major real matrix (fp64 residual or fp32 input) into
// the device layout: one wavefront per row, one ballot per 64 columns.  NC
// columns (the row stride), ND >= NC / 32 words per row; bits at or beyond
// NC are clear.
template <typename T>
__global__ void __launch_bounds__(64) k_signs(const T* __restrict__ R, int M, int NC, int ND,
                                             uint32_t* __restrict__ bits, size_t plane, int k) {
  // one workgroup per padded row: every word of the row, padding included
  const int m = blockIdx.x;
  const int NP = pad_words(ND) * 32;
  for (int n0 = 0; n0 < NP; n0 += 64) {
    const int n = n0 + threadIdx.x;
    const bool pos = m < M && n < NC && R[(size_t)m * NC + n] >= (T)0;
    const unsigned long long b = __ballot(pos);
    if (threadIdx.x == 0) {
      const int w = n0 / 32;  // even; w + 1 < NP / 32
      bits[layout_offset(M, ND, plane, k, m, w)] = (uint32_t)b;
      bits[layout_offset(M, ND, plane, k, m, w + 1)] = (uint32_t)(b >> 32);
    }
  }
}

__global__ void k_den(const float* __restrict__ alpha, int M, double* __restrict__ den) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    double s = 0.0;
    for (int m = 0; m < M; ++m) s = s + (double)alpha[m] * (double)alpha[m];
    *den = s;
  }
}

__global__ void k_colscale(const double* __restrict__ R, const float* __restrict__ alpha,
                           const double* __restrict__ den, int M, int N, uint16_t* __restrict__ cs) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const double d = *den;
  uint16_t h;
  if (d == 0.0) {
    h = 0x3c00u;
  } else {
    double num = 0.0;
    for (int m = 0; m < M; ++m) num = num + (double)alpha[m] * fabs(R[(size_t)m * N + n]);
    const float c32 = (float)(num / d);
    const _Float16 c16 = (_Float16)c32;
    __builtin_memcpy(&h, &c16, 2);
  }
  cs[n] = h;
}

__global__ void k_residual(double* __restrict__ R, const float* __restrict__ alpha,
                           const uint16_t* __restrict__ cs, int M, int N) {
  const size_t total = (size_t)M * N;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(i / N);
    const int n = (int)(i % N);
    const double r = R[i];
    const double sgn = r >= 0.0 ? 1.0 : -1.0;
    const double c = cs ? (double)f16_bits_to_float(cs[n]) : 1.0;
    const double t = (double)alpha[m] * c;
    R[i] = r - t * sgn;
  }
}

// Group-wise row scales in fp16 (one per row and group of g consecutive
// columns of a residual R [M][NC]; G = NC / g groups), stored word-grouped:
// the gpw = max(1, 32 / g) scales of one 32-column word of a row are
// adjacent, rows consecutive, i.e. scale (m, j) at scale_index(...).
__device__ inline size_t scale_index(int M, int gpw, int m, int j) {
  return ((size_t)(j / gpw) * M + m) * gpw + j % gpw;
}

// a[m][j] = fp16(fp32(sum_{n in group j} |R[m,n]| / g)), ascending n; the
// slots of a last partly used word (j >= G) get 0
__global__ void k_gscale(const double* __restrict__ R, int M, int NC, int g, int gpw, uint16_t* __restrict__ a) {
  const int G = NC / g, GS = (G + gpw - 1) / gpw * gpw;
  const size_t total = (size_t)M * GS;
  for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < total; t += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(t % M), j = (int)(t / M);
    uint16_t hb = 0;
    if (j < G) {
      const double* r = R + (size_t)m * NC + (size_t)j * g;
      double s = 0.0;
      for (int i = 0; i < g; ++i) s = s + fabs(r[i]);
      const _Float16 h = (_Float16)(float)(s / (double)g);
      __builtin_memcpy(&hb, &h, 2);
    }
    a[scale_index(M, gpw, m, j)] = hb;
  }
}

// den[j] = sum_m a[m][j]^2, ascending m
__global__ void k_gden(const uint16_t* __restrict__ a, int M, int G, int gpw, double* __restrict__ den) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= G) return;
  double s = 0.0;
  for (int m = 0; m < M; ++m) {
    const double v = (double)f16_bits_to_float(a[scale_index(M, gpw, m, j)]);
    s = s + v * v;
  }
  den[j] = s;
}

// cs[n] = fp16(fp32(sum_m a[m][j] |R[m,n]| / den[j])) for the group j of n
// (1 when den[j] == 0)
__global__ void k_gcolscale(const double* __restrict__ R, const uint16_t* __restrict__ a,
                            const double* __restrict__ den, int M, int NC, int g, int gpw, uint16_t* __restrict__ cs) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= NC) return;
  const int j = n / g;
  const double d = den[j];
  uint16_t h;
  if (d == 0.0) {
    h = 0x3c00u;
  } else {
    double num = 0.0;
    for (int m = 0; m < M; ++m)
      num = num + (double)f16_bits_to_float(a[scale_index(M, gpw, m, j)]) * fabs(R[(size_t)m * NC + n]);
    const _Float16 c16 = (_Float16)(float)(num / d);
    __builtin_memcpy(&h, &c16, 2);
  }
  cs[n] = h;
}

// R <- R - a[m][j(n)] c[n] (2 bit - 1), the sign being that of R itself
__global__ void k_gresidual(double* __restrict__ R, const uint16_t* __restrict__ a, const uint16_t* __restrict__ cs,
                            int M, int NC, int g, int gpw) {
  const size_t total = (size_t)M * NC;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(i / NC);
    const int n = (int)(i % NC);
    const double r = R[i];
    const double sgn = r >= 0.0 ? 1.0 : -1.0;
    const double c = cs ? (double)f16_bits_to_float(cs[n]) : 1.0;
    const double t = (double)f16_bits_to_float(a[scale_index(M, gpw, m, n / g)]) * c;
    R[i] = r - t * sgn;
  }
}

// Rs[m][p] = R[m][idx[p]] (0 for an index outside [0, N))
__global__ void k_gather_cols(const double* __restrict__ R, int M, int N, const int32_t* __restrict__ idx, int S,
                              double* __restrict__ Rs) {
  const size_t total = (size_t)M * S;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(i / S);
    const int n = idx[i % S];
    Rs[i] = (n >= 0 && n < N) ? R[(size_t)m * N + n] : 0.0;
  }
}

__global__ void k_absmean(const float* __restrict__ X, int S, int N, float* __restrict__ xbar) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  double s = 0.0;
  for (int i = 0; i < S; ++i) s = s + fabs((double)X[(size_t)i * N + n]);
  xbar[n] = (float)(S > 0 ? s / (double)S : 0.0);
}

// sel[m] = 1 iff fewer than ns rows rank above m (higher score, or equal
// score and smaller index).
__global__ void __launch_bounds__(256) k_rank(const double* __restrict__ score, int M, int ns, int* __restrict__ sel) {
  __shared__ double tile[256];
  const int m = blockIdx.x * 256 + threadIdx.x;
  const double sm = m < M ? score[m] : 0.0;
  int rank = 0;
  for (int b0 = 0; b0 < M; b0 += 256) {
    const int j = b0 + threadIdx.x;
    tile[threadIdx.x] = j < M ? score[j] : 0.0;
    __syncthreads();
    const int lim = min(256, M - b0);
    for (int t = 0; t < lim; ++t) {
      const double v = tile[t];
      const int mp = b0 + t;
      rank += (v > sm) || (v == sm && mp < m);
    }
    __syncthreads();
  }
  if (m < M) sel[m] = rank < ns;
}

// rows[] = the selected row indices in ascending order (one workgroup scan).
__global__ void __launch_bounds__(1024) k_compact(const int* __restrict__ sel, int M, int ns, int32_t* __restrict__ rows) {
  __shared__ int sums[1024];
  const int t = threadIdx.x;
  const int per = (M + 1023) / 1024;
  const int lo = min(M, t * per), hi = min(M, lo + per);
  int c = 0;
  for (int m = lo; m < hi; ++m) c += sel[m];
  sums[t] = c;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = t >= off ? sums[t - off] : 0;
    __syncthreads();
    sums[t] += v;
    __syncthreads();
  }
  int pos = sums[t] - c;
  for (int m = lo; m < hi; ++m) {
    if (sel[m] && pos < ns) rows[pos++] = m;   // bound: NaN scores could select extra rows
  }
}

__global__ void __launch_bounds__(256) k_quant_rows(const float* __restrict__ W, int M, int N,
                                                    const int32_t* __restrict__ rows, int8_t* __restrict__ q,
                                                    uint16_t* __restrict__ s_out, float* __restrict__ alpha, int K) {
  __shared__ float red[256];
  __shared__ double s_sh;
  const int i = blockIdx.x;
  const int m = rows[i];
  if (m < 0 || m >= M) return;   // only with NaN scores (fewer rows selected)
  const float* Wm = W + (size_t)m * N;
  float mx = 0.0f;
  for (int n = threadIdx.x; n < N; n += 256) mx = fmaxf(mx, fabsf(Wm[n]));
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + off]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float s32 = (float)((double)red[0] / 127.0);
    const _Float16 s16 = (_Float16)s32;
    uint16_t h;
    __builtin_memcpy(&h, &s16, 2);
    s_out[i] = h;
    s_sh = (double)(float)s16;
    for (int k = 0; k < K; ++k) alpha[(size_t)k * M + m] = 0.0f;
  }
  __syncthreads();
  const double sd = s_sh;
  for (int n = threadIdx.x; n < N; n += 256) {
    int8_t v = 0;
    if (sd != 0.0) {
      double r = __builtin_rint((double)Wm[n] / sd);
      r = r > 127.0 ? 127.0 : (r < -127.0 ? -127.0 : r);
      v = (int8_t)r;
    }
    q[(size_t)i * N + n] = v;
  }
}

// --------------------------------------------------------------- launchers

static int grid_for(size_t n, int threads) {
  size_t g = (n + threads - 1) / threads;
  if (g > 65536) g = 65536;
  return (int)(g ? g : 1);
}

hipError_t launch_pack(const float* W, int M, int N, int K, bool colscale, uint32_t* bits, float* alpha,
                       uint16_t* cs, void* ws, hipStream_t st) {
  double* R = (double*)ws;
  double* den = (double*)((char*)ws + align_up((size_t)M * N * 8, 256));
  const size_t mn = (size_t)M * N;
  const int ND = N / 32;
  const size_t plane = plane_words(M, ND);
  hipLaunchKernelGGL(k_widen, dim3(grid_for(mn, 256)), dim3(256), 0, st, W, R, mn);
  for (int k = 0; k < K; ++k) {
    float* ak = alpha + (size_t)k * M;
    uint16_t* ck = colscale ? cs + (size_t)k * N : nullptr;
    hipLaunchKernelGGL(k_signs<double>, dim3(pad_rows(M)), dim3(64), 0, st, R, M, N, N / 32, bits, plane, k);
    hipLaunchKernelGGL(k_rowsum<0>, dim3((M + kT - 1) / kT), dim3(kT), 0, st, R, (const float*)nullptr,
                       (const float*)nullptr, M, N, ak, (double*)nullptr);
    if (colscale) {
      hipLaunchKernelGGL(k_den, dim3(1), dim3(64), 0, st, ak, M, den);
      hipLaunchKernelGGL(k_colscale, dim3((N + 255) / 256), dim3(256), 0, st, R, ak, den, M, N, ck);
    }
    if (k + 1 < K) hipLaunchKernelGGL(k_residual, dim3(grid_for(mn, 256)), dim3(256), 0, st, R, ak, ck, M, N);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// K greedy bases with fp16 group scales on the residual R [M][NC] (groups of
// g columns, scales word-grouped with gpw per word); updates R after every
// base but the last unless update_last.
static hipError_t grouped_bases(double* R, int M, int NC, int ND, int g, int gpw, int K, uint32_t* bits,
                                uint16_t* alpha, uint16_t* cs, double* den, bool update_last, hipStream_t st) {
  const size_t mn = (size_t)M * NC;
  const int G = NC / g, GS = (G + gpw - 1) / gpw * gpw;
  const size_t plane = plane_words(M, ND), aplane = (size_t)GS * M;
  for (int k = 0; k < K; ++k) {
    uint16_t* ak = alpha + (size_t)k * aplane;
    uint16_t* ck = cs ? cs + (size_t)k * NC : nullptr;
    hipLaunchKernelGGL(k_signs<double>, dim3(pad_rows(M)), dim3(64), 0, st, R, M, NC, ND, bits, plane, k);
    hipLaunchKernelGGL(k_gscale, dim3(grid_for((size_t)M * GS, 256)), dim3(256), 0, st, R, M, NC, g, gpw, ak);
    if (cs) {
      hipLaunchKernelGGL(k_gden, dim3((G + 255) / 256), dim3(256), 0, st, ak, M, G, gpw, den);
      hipLaunchKernelGGL(k_gcolscale, dim3((NC + 255) / 256), dim3(256), 0, st, R, ak, den, M, NC, g, gpw, ck);
    }
    if (k + 1 < K || update_last)
      hipLaunchKernelGGL(k_gresidual, dim3(grid_for(mn, 256)), dim3(256), 0, st, R, ak, ck, M, NC, g, gpw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_pack_hybrid(const float* W, int M, int N, int K, int g, int s, const int32_t* idx, bool colscale,
                              uint32_t* bits, uint16_t* alpha, uint16_t* cs, uint32_t* sbits, uint16_t* salpha,
                              uint16_t* scs, void* ws, hipStream_t st) {
  const int G = N / g, S = s * G;
  double* R = (double*)ws;
  double* Rs = (double*)((char*)ws + align_up((size_t)M * N * 8, 256));
  double* den = (double*)((char*)Rs + align_up((size_t)M * S * 8, 256));
  const size_t mn = (size_t)M * N;
  hipLaunchKernelGGL(k_widen, dim3(grid_for(mn, 256)), dim3(256), 0, st, W, R, mn);
  hipError_t e = grouped_bases(R, M, N, N / 32, g, 1, K, bits, alpha, colscale ? cs : nullptr, den, s > 0, st);
  if (e != hipSuccess || s == 0) return e;
  hipLaunchKernelGGL(k_gather_cols, dim3(grid_for((size_t)M * S, 256)), dim3(256), 0, st, R, M, N, idx, S, Rs);
  return grouped_bases(Rs, M, S, (S + 31) / 32, s, s < 32 ? 32 / s : 1, K, sbits, salpha, colscale ? scs : nullptr,
                       den, false, st);
}

hipError_t launch_pack_signs(const float* S, int M, int N, uint32_t* bits, hipStream_t st) {
  hipLaunchKernelGGL(k_signs<float>, dim3(pad_rows(M)), dim3(64), 0, st, S, M, N, N / 32, bits, plane_words(M, N / 32),
                     0);
  return hipGetLastError();
}

hipError_t launch_absmean(const float* X, int S, int N, float* xbar, hipStream_t st) {
  hipLaunchKernelGGL(k_absmean, dim3((N + 255) / 256), dim3(256), 0, st, X, S, N, xbar);
  return hipGetLastError();
}

hipError_t launch_salient(const float* W, int M, int N, const float* xbar, int ns, int32_t* rows, int8_t* q,
                          uint16_t* s, float* alpha, int K, void* ws, hipStream_t st) {
  double* score = (double*)ws;
  int* sel = (int*)((char*)ws + align_up((size_t)M * 8, 256));
  hipLaunchKernelGGL(k_rowsum<1>, dim3((M + kT - 1) / kT), dim3(kT), 0, st, (const double*)nullptr, W, xbar, M, N,
                     (float*)nullptr, score);
  hipLaunchKernelGGL(k_rank, dim3((M + 255) / 256), dim3(256), 0, st, score, M, ns, sel);
  hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, st, sel, M, ns, rows);
  if (ns > 0) hipLaunchKernelGGL(k_quant_rows, dim3(ns), dim3(256), 0, st, W, M, N, rows, q, s, alpha, K);
  return hipGetLastError();
}

}  // namespace bsg
