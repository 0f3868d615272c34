// Protected int8 rows on the matrix cores, for several batch columns of bf16
// or fp16 x (BiSCo "Sensitivity Protection": the protected rows are kept in
// 8 bits apart from the binary payload):
//
//   y[rows[i], b] += s_i * sum_n q[i][n] * x[n, b]
//
// v_mfma_f32_16x16x32_{bf16,f16}: A = 16 protected rows x 32 columns of q
// (int8 values are exact in bf16 and fp16), B = 32 columns x 16 batch
// columns of x, fp32 sums, so the only rounding is that of the fp32 sums.
// A workgroup owns 16 protected rows and 16 batch columns and reads each
// row of x once for all 16 rows (one workgroup per row re-reads x for every
// row); its wavefronts split the columns into runs of 128 (4 MFMA steps),
// loading the next run's q and x while the current one is multiplied.  x is
// [N][B], so each wavefront transposes its run's 128 x 16 block through its
// own LDS tile for the B operand, as in the batched sign product.  The
// partial tiles are summed through LDS in a fixed order (no atomics).
// Rows past ns and columns past N load zero (buffer loads past the end).
// Chosen for more than 256 protected rows (B % 8 == 0), where it measured
// faster than four rows and four batch columns per workgroup.
#include <algorithm>

#include "bsg_prod_mfma.h"

namespace bsg {

// 8 int8 values (two words) as 8 bf16 / fp16 values, exact
template <int XT>
__device__ inline uint4 q_operand(uint2 w) {
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t src = i < 2 ? w.x : w.y;
    const float lo = (float)(int8_t)(src >> (16 * (i & 1)));
    const float hi = (float)(int8_t)(src >> (16 * (i & 1) + 8));
    if (XT == 1) {
      d[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
    } else {
      d[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
    }
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

struct SalRun {
  uint2 q[4];  // per step: columns 32 step + 8 g .. + 7 of the lane's row
  uint4 x[4];  // per step: batch values bb .. bb + 7 of column 32 step + lane % 32
};

// blockDim.x = 64 W; dynamic LDS: W (kXtBytes + 1 KiB)
template <int XT>
__global__ void __launch_bounds__(1024) k_salient_mfma(const int32_t* __restrict__ rows, const int8_t* __restrict__ q,
                                                     const uint16_t* __restrict__ s, int ns, int M, int N,
                                                     const void* __restrict__ x, int B, float* __restrict__ y) {
  extern __shared__ __align__(16) char lds[];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int i0 = blockIdx.x * 16, b0 = blockIdx.y * 16;
  const uint32_t xt = (uint32_t)(uintptr_t)lds + (uint32_t)wv * kXtBytes;
  float* red = (float*)(lds + (size_t)W * kXtBytes);  // [W][16 rows][16 columns]

  const rsrc_t qs = make_rsrc(q, (size_t)ns * N);
  const rsrc_t xs = make_rsrc(x, (size_t)N * B * 2);
  constexpr uint32_t kOut = 0x80000000u;  // an offset past the end: loads zero
  const uint32_t qrow = (uint32_t)(i0 + r16) * (uint32_t)N;
  const int nl = lane & 31, bh = lane >> 5;
  const int bb = b0 + 8 * bh;
  const uint32_t xo = bb < B ? (uint32_t)(nl * B + bb) * 2u : kOut;
  const uint32_t xstep = 64u * (uint32_t)B;  // bytes of x per 32 columns

  // this wavefront's runs of 128 columns: [rb, re)
  const int NR = (N + 127) >> 7;
  const int rb = wv * NR / W, re = (wv + 1) * NR / W;

  auto load_run = [&](int t, SalRun& d) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 128 * t + 32 * j + 8 * g;  // first column of the lane's A values
      d.q[j] = ld64(qs, c < N ? qrow + (uint32_t)c : kOut);
      d.x[j] = ld128(xs, xo == kOut ? kOut : xo + (uint32_t)(4 * t + j) * xstep);
    }
  };
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  auto run = [&](const SalRun& d) {
    // transpose: row b of the LDS tile = batch column b, 128 columns
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w[4] = {d.x[j].x, d.x[j].y, d.x[j].z, d.x[j].w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *(lds_u16*)(uintptr_t)(xt + (uint32_t)((bh * 8 + i) * kXtRow + j * 32 + nl) * 2u) =
            (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
    }
    wave_sync();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 bv = lds_u4(xt + (uint32_t)(r16 * kXtRow + j * 32 + 8 * g) * 2u);
      acc = mfma_step<XT>(q_operand<XT>(d.q[j]), bv, acc);
    }
    wave_sync();  // the next run's transpose overwrites the tile
  };
  if (rb < re) {
    SalRun ra, rc;
    load_run(rb, ra);
    int t = rb;
    for (; t + 2 <= re; t += 2) {
      load_run(t + 1, rc);
      run(ra);
      load_run(min(t + 2, re - 1), ra);  // past the last run: re-read it (a cache hit)
      run(rc);
    }
    if (t < re) run(ra);
  }

  // lane holds rows 4 g + i of the tile, batch column r16
#pragma unroll
  for (int i = 0; i < 4; ++i) red[(wv * 16 + 4 * g + i) * 16 + r16] = acc[i];
  __syncthreads();
  for (int e = threadIdx.x; e < 256; e += blockDim.x) {
    const int r = e >> 4, c = e & 15;
    const int i = i0 + r, b = b0 + c;
    if (i < ns && b < B) {
      const int m = rows[i];
      if (m >= 0 && m < M) {
        float t = red[e];
        for (int w = 1; w < W; ++w) t += red[w * 256 + e];
        y[(size_t)m * B + b] += f16_bits_to_float(s[i]) * t;
      }
    }
  }
}

bool salient_mfma_ok(int ns, int N, const int8_t* q, const void* x, int xdt, int B) {
  return B >= 4 && B % 8 == 0 && (xdt == BSG_BF16 || xdt == BSG_F16) && N % 8 == 0 &&
         (uintptr_t)q % 8 == 0 && (uintptr_t)x % 16 == 0 && ((size_t)ns + 16) * N < (1u << 31) &&
         (size_t)N * B * 2 < (1u << 31);
}

hipError_t launch_salient_mfma(const int32_t* rows, int ns, const int8_t* q, const uint16_t* s, int M, int N,
                               const void* x, int xdt, int B, float* y, hipStream_t st) {
  if (ns <= 0) return hipSuccess;
  const int NR = (N + 127) / 128;
  const int W = std::max(1, std::min(16, NR));  // at least one run each
  const size_t lds = (size_t)W * (kXtBytes + 1024);
  const dim3 grid((ns + 15) / 16, (B + 15) / 16);
  const void* kern = xdt == BSG_BF16 ? (const void*)k_salient_mfma<1> : (const void*)k_salient_mfma<2>;
  if (lds > 32768) {
    const hipError_t e = allow_large_lds(kern);
    if (e != hipSuccess) return e;
  }
  if (xdt == BSG_BF16)
    hipLaunchKernelGGL(k_salient_mfma<1>, grid, dim3(64 * W), lds, st, rows, q, s, ns, M, N, x, B, y);
  else
    hipLaunchKernelGGL(k_salient_mfma<2>, grid, dim3(64 * W), lds, st, rows, q, s, ns, M, N, x, B, y);
  return hipGetLastError();
}

}  // namespace bsg
