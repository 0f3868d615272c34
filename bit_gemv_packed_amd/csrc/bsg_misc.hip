// Protected int8 rows, int8 activation quantisation and layout conversions
// for gfx950.
#include <algorithm>

#include "bsg_internal.h"

namespace bsg {

// Sum over the workgroup of one value per thread (blockDim.x = 64 W), in a
// fixed order: a butterfly inside each wavefront, then the W wavefront sums
// in index order.  Every thread gets the result.  red: >= 16 floats of LDS.
template <bool MAX>
__device__ inline float block_reduce(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float u = __shfl_xor(v, o);
    v = MAX ? fmaxf(v, u) : v + u;
  }
  const int wv = threadIdx.x >> 6, W = blockDim.x >> 6;
  __syncthreads();  // red may still be read from a previous call
  if ((threadIdx.x & 63) == 0) red[wv] = v;
  __syncthreads();
  float t = red[0];
  for (int w = 1; w < W; ++w) t = MAX ? fmaxf(t, red[w]) : t + red[w];
  return t;
}

// 8 16-bit x values in one 16-byte word -> fp32
__device__ inline void cvt8_x16(const uint4 u, int xdt, float (&v)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint16_t h = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
    v[j] = xdt == BSG_BF16 ? bf16_bits_to_float(h) : f16_bits_to_float(h);
  }
}

// 8 consecutive 16-bit x values (one aligned 16-byte load) -> fp32
__device__ inline void load8_x16(const void* x, int xdt, size_t i, float (&v)[8]) {
  cvt8_x16(*(const uint4*)((const uint16_t*)x + i), xdt, v);
}

// y[rows[i], b] += s_i * sum_n q[i][n] * x[n, b]   (BiSCo "Sensitivity
// Protection": the protected rows are kept in 8 bits apart from the binary
// payload).  One workgroup of 1024 threads per protected row; int8 -> fp32
// conversions are exact; fp32 accumulation, fixed-order reduction.  VEC: one
// batch column of 16-bit x, N % 16 == 0, q row and x 16-byte aligned: each
// thread takes 16 columns with one 16-byte q load and two x loads.
template <bool VEC>
__global__ void __launch_bounds__(1024) k_salient(const int32_t* __restrict__ rows, const int8_t* __restrict__ q,
                                                  const uint16_t* __restrict__ s, int M, int N,
                                                  const void* __restrict__ x, int xdt, int B, float* __restrict__ y) {
  __shared__ float red[16];
  const int i = blockIdx.x;
  const int m = rows[i];
  if (m < 0 || m >= M) return;
  const int8_t* qi = q + (size_t)i * N;
  const float si = f16_bits_to_float(s[i]);
  if (VEC) {
    float acc = 0.0f;
    for (int n0 = threadIdx.x * 16; n0 < N; n0 += blockDim.x * 16) {
      const int4 qv = *(const int4*)(qi + n0);
      const int qw[4] = {qv.x, qv.y, qv.z, qv.w};
      float xv[16];
      load8_x16(x, xdt, n0, *(float(*)[8])xv);
      load8_x16(x, xdt, n0 + 8, *(float(*)[8])(xv + 8));
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc = __builtin_fmaf((float)(int8_t)((uint32_t)qw[j >> 2] >> (8 * (j & 3))), xv[j], acc);
    }
    const float t = block_reduce<false>(acc, red);
    if (threadIdx.x == 0) y[m] += si * t;
    return;
  }
  for (int b = 0; b < B; ++b) {
    float acc = 0.0f;
    for (int n = threadIdx.x; n < N; n += blockDim.x)
      acc = __builtin_fmaf((float)qi[n], load_x(x, xdt, (size_t)n * B + b), acc);
    const float t = block_reduce<false>(acc, red);
    if (threadIdx.x == 0) y[(size_t)m * B + b] += si * t;
  }
}

// The same for several batch columns, any layout of x: workgroup (i, t)
// takes protected row i and batch columns 16 t .. 16 t + 15; each thread
// takes columns n of x, keeps 16 sums and loads each value on its own.
// Each sum is reduced by a butterfly inside the wavefront, then over the
// wavefronts in index order.
__global__ void __launch_bounds__(1024) k_salient_bt(const int32_t* __restrict__ rows, const int8_t* __restrict__ q,
                                                   const uint16_t* __restrict__ s, int ns, int M, int N,
                                                   const void* __restrict__ x, int xdt, int B, float* __restrict__ y) {
  __shared__ float red[16][16];
  const int i = blockIdx.x, b0 = blockIdx.y * 16;
  const int8_t* qi = q + (size_t)i * N;
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
  for (int n = threadIdx.x; n < N; n += blockDim.x) {
    const float qn = (float)qi[n];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (b0 + j < B) acc[j] = __builtin_fmaf(qn, load_x(x, xdt, (size_t)n * B + b0 + j), acc[j]);
  }
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc[j] += __shfl_xor(acc[j], o);
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < 16; ++j) red[wv][j] = acc[j];
  }
  __syncthreads();
  const int j = threadIdx.x;
  if (j < 16 && b0 + j < B) {
    const int m = rows[i];
    if (m >= 0 && m < M) {
      const int W = blockDim.x >> 6;
      float t = red[0][j];
      for (int w = 1; w < W; ++w) t += red[w][j];
      y[(size_t)m * B + b0 + j] += f16_bits_to_float(s[i]) * t;
    }
  }
}

// Four protected rows and four batch columns per workgroup (16-bit x, B % 4
// == 0, x 8-byte aligned): 16 sums per thread.  QW (B == 4, N % 4 == 0, q
// 4-byte aligned): a thread takes groups of 4 consecutive columns, with one
// 4-byte q load per row and one 8-byte x load per column (B = 4: 138 rows of
// 5120 in 6.7 against 7.3 us, 287 of 8192 in 9.2 against 9.9 us); else
// single columns with one q byte per row.  A thread issues the loads of up to kSalCols columns
// before any product, so a row of up to kSalCols * 1024 columns costs one
// round of memory latency (a loop that waited for each column's loads cost
// about 2 us per column on 1024 threads); columns past N re-read column
// N - 1 and rows past ns re-read row ns - 1, with weight 0.
constexpr int kSalCols = 8;
template <int R, bool QW>
__global__ void __launch_bounds__(1024) k_salient_rb(const int32_t* __restrict__ rows, const int8_t* __restrict__ q,
                                                   const uint16_t* __restrict__ s, int ns, int M, int N,
                                                   const void* __restrict__ x, int xdt, int B, float* __restrict__ y) {
  constexpr int BC = 16 / R;  // batch columns per workgroup (4: one 8-byte load)
  static_assert(BC == 4, "one 8-byte x load per column");
  constexpr int CG = QW ? 4 : 1;     // columns per group
  constexpr int NGR = kSalCols / CG;  // groups per thread and round
  __shared__ float red[16][16];
  const int i0 = blockIdx.x * R, b0 = blockIdx.y * BC;
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
  const int8_t* qr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) qr[r] = q + (size_t)min(i0 + r, ns - 1) * N;
  const int NG = (N + CG - 1) / CG;
  for (int g0 = threadIdx.x; g0 < NG; g0 += NGR * blockDim.x) {
    uint2 xv[NGR][CG];
    uint32_t qv[NGR][R];
#pragma unroll
    for (int u = 0; u < NGR; ++u) {
      const int n = min(g0 + u * (int)blockDim.x, NG - 1) * CG;
#pragma unroll
      for (int c = 0; c < CG; ++c) xv[u][c] = *(const uint2*)((const uint16_t*)x + (size_t)min(n + c, N - 1) * B + b0);
#pragma unroll
      for (int r = 0; r < R; ++r) qv[u][r] = QW ? *(const uint32_t*)(qr[r] + n) : (uint32_t)(uint8_t)qr[r][n];
    }
#pragma unroll
    for (int u = 0; u < NGR; ++u) {
      const bool in = g0 + u * (int)blockDim.x < NG;
#pragma unroll
      for (int c = 0; c < CG; ++c) {
        const uint32_t w[2] = {xv[u][c].x, xv[u][c].y};
        float xf[BC];
#pragma unroll
        for (int b = 0; b < BC; ++b) {
          const uint16_t h = (uint16_t)(w[b >> 1] >> (16 * (b & 1)));
          xf[b] = xdt == BSG_BF16 ? bf16_bits_to_float(h) : f16_bits_to_float(h);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float qf = in && i0 + r < ns ? (float)(int8_t)(qv[u][r] >> (8 * c)) : 0.0f;
#pragma unroll
          for (int b = 0; b < BC; ++b) acc[r * BC + b] = __builtin_fmaf(qf, xf[b], acc[r * BC + b]);
        }
      }
    }
  }
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc[j] += __shfl_xor(acc[j], o);
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < 16; ++j) red[wv][j] = acc[j];
  }
  __syncthreads();
  const int j = threadIdx.x;
  if (j < 16) {
    const int i = i0 + j / BC, b = b0 + j % BC;
    if (i < ns && b < B) {
      const int m = rows[i];
      if (m >= 0 && m < M) {
        const int W = blockDim.x >> 6;
        float t = red[0][j];
        for (int w = 1; w < W; ++w) t += red[w][j];
        y[(size_t)m * B + b] += f16_bits_to_float(s[i]) * t;
      }
    }
  }
}

// sx[b] = fp32(max_n |x| / 127); xq = clamp(rint_even(fp32(x / sx)), -127, 127).
// One workgroup of 1024 threads per batch column.  VEC: one batch column of
// 16-bit x, N % 8 == 0, x 16-byte and xq 8-byte aligned: 8 values per thread
// and pass, kept in registers between the two phases.
template <bool VEC>
__global__ void __launch_bounds__(1024) k_quantize(const void* __restrict__ x, int xdt, int N, int B,
                                                   int8_t* __restrict__ xq, float* __restrict__ sx) {
  __shared__ float red[16];
  const int b = blockIdx.x;
  if (VEC) {
    constexpr int P = 4;  // passes kept in registers (N <= 32768); larger N re-reads x
    float v[P][8];
    float mx = 0.0f;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int n0 = (p * blockDim.x + threadIdx.x) * 8;
      if (n0 < N) {
        load8_x16(x, xdt, n0, v[p]);
#pragma unroll
        for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(v[p][j]));
      }
    }
    for (int n0 = (P * blockDim.x + threadIdx.x) * 8; n0 < N; n0 += blockDim.x * 8) {
      float u[8];
      load8_x16(x, xdt, n0, u);
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(u[j]));
    }
    const float sv = __fdiv_rn(block_reduce<true>(mx, red), 127.0f);
    if (threadIdx.x == 0) sx[0] = sv;
    auto quant8 = [&](const float (&u)[8], int n0) {
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        int c = 0;
        if (sv != 0.0f) {
          float r = __builtin_rintf(__fdiv_rn(u[j], sv));
          r = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
          c = (int)r;
        }
        w[j >> 2] |= ((uint32_t)c & 0xffu) << (8 * (j & 3));
      }
      *(uint2*)(xq + n0) = make_uint2(w[0], w[1]);
    };
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int n0 = (p * blockDim.x + threadIdx.x) * 8;
      if (n0 < N) quant8(v[p], n0);
    }
    for (int n0 = (P * blockDim.x + threadIdx.x) * 8; n0 < N; n0 += blockDim.x * 8) {
      float u[8];
      load8_x16(x, xdt, n0, u);
      quant8(u, n0);
    }
    return;
  }
  float mx = 0.0f;
  for (int n = threadIdx.x; n < N; n += blockDim.x) mx = fmaxf(mx, fabsf(load_x(x, xdt, (size_t)n * B + b)));
  const float sv = __fdiv_rn(block_reduce<true>(mx, red), 127.0f);
  if (threadIdx.x == 0) sx[b] = sv;
  for (int n = threadIdx.x; n < N; n += blockDim.x) {
    int8_t c = 0;
    if (sv != 0.0f) {
      float r = __builtin_rintf(__fdiv_rn(load_x(x, xdt, (size_t)n * B + b), sv));
      r = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
      c = (int8_t)r;
    }
    xq[(size_t)n * B + b] = c;
  }
}

// Writes every word of the K padded planes: the logical word, or 0 in the padding.
__global__ void k_to_layout(const uint32_t* __restrict__ logical, int K, int M, int ND, size_t plane,
                            uint32_t* __restrict__ bits) {
  const size_t total = (size_t)K * plane;
  const size_t ndp = (size_t)pad_words(ND);
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int k = (int)(i / plane);
    const size_t o = i % plane;
    const size_t rb = o / (64 * ndp), t = o % (64 * ndp);  // row block, offset in it
    const int m = (int)(rb * 64 + (t % 256) / 4);
    const int w = (int)((t / 256) * 4 + t % 4);
    bits[i] = (m < M && w < ND) ? logical[((size_t)k * M + m) * ND + w] : 0u;
  }
}

__global__ void k_from_layout(const uint32_t* __restrict__ bits, int K, int M, int ND, size_t plane,
                              uint32_t* __restrict__ logical) {
  const size_t total = (size_t)K * M * ND;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int w = (int)(i % ND);
    const size_t km = i / ND;
    const int m = (int)(km % M);
    const int k = (int)(km / M);
    logical[i] = bits[layout_offset(M, ND, plane, k, m, w)];
  }
}

static int grid_for(size_t n, int threads) {
  size_t g = (n + threads - 1) / threads;
  if (g > 65536) g = 65536;
  return (int)(g ? g : 1);
}

static bool aligned(const void* p, size_t a) { return (((uintptr_t)p) % a) == 0; }

bool salient_mfma_ok(int ns, int N, const int8_t* q, const void* x, int xdt, int B);
hipError_t launch_salient_mfma(const int32_t* rows, int ns, const int8_t* q, const uint16_t* s, int M, int N,
                               const void* x, int xdt, int B, float* y, hipStream_t st);

hipError_t launch_salient_apply(const int32_t* rows, int ns, const int8_t* q, const uint16_t* s, int M, int N,
                                const void* x, int xdt, int B, float* y, hipStream_t st) {
  // Batches: more than 256 protected rows on the matrix cores (16 rows per
  // workgroup, x read once per 16 rows); else four rows and four batch
  // columns per workgroup; else one row and 16 columns with one load per
  // value.  Measured (graph replay): 287 rows of 8192 at B = 16 take 15.8 us
  // on the matrix cores and 16.8 us four by four; 138 rows of 5120 take
  // 7.9 us four by four and 10.1 us on the matrix cores; at B = 4 four by
  // four takes 7.3 us (138 x 5120), 10.0 us (287 x 8192) and 10.7 us
  // (51 x 13824), against 12.5, 25.4 and 21.7 us one row at a time.
  if (ns > 256 && salient_mfma_ok(ns, N, q, x, xdt, B))
    return launch_salient_mfma(rows, ns, q, s, M, N, x, xdt, B, y, st);
  if (B > 1 && B % 4 == 0 && xdt != BSG_F32 && aligned(x, 8)) {
    const dim3 grid((ns + 3) / 4, B / 4);
    const int threads = std::min(1024, std::max(64, (N / kSalCols + 63) / 64 * 64));  // about kSalCols columns each
    // 4-column groups only at B = 4: a lane's x rows then lie 32 bytes from
    // its neighbour's (16 cache lines per load); at B = 16, 128 bytes apart,
    // they measured slower (13.5 against 11.5 us at 51 rows of 13824)
    if (B == 4 && N % 4 == 0 && aligned(q, 4))
      hipLaunchKernelGGL((k_salient_rb<4, true>), grid, dim3(threads), 0, st, rows, q, s, ns, M, N, x, xdt, B, y);
    else
      hipLaunchKernelGGL((k_salient_rb<4, false>), grid, dim3(threads), 0, st, rows, q, s, ns, M, N, x, xdt, B, y);
    return hipGetLastError();
  }
  if (B > 1) {
    const dim3 grid(ns, (B + 15) / 16);
    const int threads = std::min(1024, std::max(64, (N / 4 + 63) / 64 * 64));  // about 4 columns each
    hipLaunchKernelGGL(k_salient_bt, grid, dim3(threads), 0, st, rows, q, s, ns, M, N, x, xdt, B, y);
    return hipGetLastError();
  }
  const bool vec = xdt != BSG_F32 && N % 16 == 0 && aligned(q, 16) && aligned(x, 16);
  const int threads = std::min(1024, std::max(64, (N / (vec ? 16 : 1) + 63) / 64 * 64));
  if (vec)
    hipLaunchKernelGGL(k_salient<true>, dim3(ns), dim3(threads), 0, st, rows, q, s, M, N, x, xdt, B, y);
  else
    hipLaunchKernelGGL(k_salient<false>, dim3(ns), dim3(threads), 0, st, rows, q, s, M, N, x, xdt, B, y);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int xdt, int N, int B, int8_t* xq, float* sx, hipStream_t st) {
  const bool vec = B == 1 && xdt != BSG_F32 && N % 8 == 0 && aligned(x, 16) && aligned(xq, 8);
  const int threads = std::min(1024, std::max(64, (N / (vec ? 8 : 1) + 63) / 64 * 64));
  if (vec)
    hipLaunchKernelGGL(k_quantize<true>, dim3(B), dim3(threads), 0, st, x, xdt, N, B, xq, sx);
  else
    hipLaunchKernelGGL(k_quantize<false>, dim3(B), dim3(threads), 0, st, x, xdt, N, B, xq, sx);
  return hipGetLastError();
}

hipError_t launch_layout(const uint32_t* src, int K, int M, int N, uint32_t* dst, bool to_layout, hipStream_t st) {
  const int ND = N / 32;
  const size_t plane = plane_words(M, ND);
  const size_t total = (size_t)K * M * ND;
  if (to_layout)
    hipLaunchKernelGGL(k_to_layout, dim3(grid_for((size_t)K * plane, 256)), dim3(256), 0, st, src, K, M, ND, plane,
                       dst);
  else
    hipLaunchKernelGGL(k_from_layout, dim3(grid_for(total, 256)), dim3(256), 0, st, src, K, M, ND, plane, dst);
  return hipGetLastError();
}

}  // namespace bsg
