// Protected int8 rows, int8 activation quantisation and layout conversions
// for gfx950.
#include "bsg_internal.h"

namespace bsg {

// y[rows[i], b] += s_i * sum_n q[i][n] * x[n, b]   (BiSCo "Sensitivity
// Protection": the protected rows are kept in 8 bits apart from the binary
// payload).  One workgroup per protected row; int8 -> fp32 conversions are
// exact; fp32 accumulation, fixed-order tree reduction.
__global__ void __launch_bounds__(256) k_salient(const int32_t* __restrict__ rows, const int8_t* __restrict__ q,
                                                 const uint16_t* __restrict__ s, int M, int N,
                                                 const void* __restrict__ x, int xdt, int B, float* __restrict__ y) {
  __shared__ float red[256];
  const int i = blockIdx.x;
  const int m = rows[i];
  if (m < 0 || m >= M) return;
  const int8_t* qi = q + (size_t)i * N;
  const float si = f16_bits_to_float(s[i]);
  const bool vec = ((N & 15) == 0) && ((((uintptr_t)qi) & 15) == 0);
  for (int b = 0; b < B; ++b) {
    float acc = 0.0f;
    if (vec) {
      for (int n0 = threadIdx.x * 16; n0 < N; n0 += 256 * 16) {
        const int4 v = *(const int4*)(qi + n0);
        const int vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int qv = (int)(int8_t)((uint32_t)vv[c] >> (8 * j));
            acc += (float)qv * load_x(x, xdt, (size_t)(n0 + c * 4 + j) * B + b);
          }
        }
      }
    } else {
      for (int n = threadIdx.x; n < N; n += 256) acc += (float)qi[n] * load_x(x, xdt, (size_t)n * B + b);
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
      if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
      __syncthreads();
    }
    if (threadIdx.x == 0) y[(size_t)m * B + b] += si * red[0];
    __syncthreads();
  }
}

// sx[b] = fp32(max_n |x| / 127); xq = clamp(rint_even(fp32(x / sx)), -127, 127).
__global__ void __launch_bounds__(256) k_quantize(const void* __restrict__ x, int xdt, int N, int B,
                                                  int8_t* __restrict__ xq, float* __restrict__ sx) {
  __shared__ float red[256];
  const int b = blockIdx.x;
  float mx = 0.0f;
  for (int n = threadIdx.x; n < N; n += 256) mx = fmaxf(mx, fabsf(load_x(x, xdt, (size_t)n * B + b)));
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + off]);
    __syncthreads();
  }
  const float s = __fdiv_rn(red[0], 127.0f);
  if (threadIdx.x == 0) sx[b] = s;
  for (int n = threadIdx.x; n < N; n += 256) {
    int8_t v = 0;
    if (s != 0.0f) {
      float r = __builtin_rintf(__fdiv_rn(load_x(x, xdt, (size_t)n * B + b), s));
      r = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
      v = (int8_t)r;
    }
    xq[(size_t)n * B + b] = v;
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

hipError_t launch_salient_apply(const int32_t* rows, int ns, const int8_t* q, const uint16_t* s, int M, int N,
                                const void* x, int xdt, int B, float* y, hipStream_t st) {
  hipLaunchKernelGGL(k_salient, dim3(ns), dim3(256), 0, st, rows, q, s, M, N, x, xdt, B, y);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int xdt, int N, int B, int8_t* xq, float* sx, hipStream_t st) {
  hipLaunchKernelGGL(k_quantize, dim3(B), dim3(256), 0, st, x, xdt, N, B, xq, sx);
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
