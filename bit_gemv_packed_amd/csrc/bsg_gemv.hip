// Sign-GEMV kernels for gfx950: the binary-base product with fp32
// accumulation through per-workgroup activation tables, and the exact int8
// variant through activation bit planes and popcounts.
//
// Mapping (both kernels): one wavefront per 64-row block, lane = row.  Every
// lane walks the same sign words of its own row, so all 64 lanes of a wave
// index the same activation table at the same time: the table reads are
// broadcasts that never conflict across LDS banks.  A 16-byte load per lane
// of a 64x4-word layout tile is one contiguous KiB per wavefront.
//
// Activation tables (FluxBin Sec. 2 "LUT-based Multiplication" and Sec. 3.2
// Stage 1, with the column scale folded into x first): for every group of 4
// input columns the workgroup stores the 16 signed sums +-x0 +-x1 +-x2 +-x3;
// a 4-bit slice of a sign word is the table index, so one LDS read and one
// add replace four signed adds.  Tables hold fp32 values; accumulation is
// fp32.
//
// int8 mode: sum_n s(n) xq(n) = 2 * sum_{bit=1} xq - sum xq, and
// sum_{bit=1} xq = sum_p 2^p popcount(word & plane_p) - 128 popcount(word &
// plane_7) over the two's-complement bit planes of xq: 8 AND + 8 popcount per
// 32 weights, exact in int32.
//
// Splits: when a row block alone gives too few workgroups, the input
// dimension is split across S workgroups.  Each writes fp32 (or int32)
// partial sums to the workspace; the last workgroup to arrive at a row block
// (an arrival counter per row block) adds the S partials in split order, so
// the result does not depend on scheduling, and resets the counter.
#include "bsg_internal.h"

#include <cstdlib>

namespace bsg {

__device__ inline void agent_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent"); }

// Returns true in every lane of the workgroup that arrives last at row block rb.
__device__ inline bool arrive_last(unsigned* cnt, int rb, int S) {
  __shared__ int s_last;
  agent_fence();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned prev = __hip_atomic_fetch_add(cnt + rb, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == (unsigned)(S - 1));
  }
  __syncthreads();
  bool last = s_last != 0;
  if (last) agent_fence();
  return last;
}

__device__ inline void reset_counter(unsigned* cnt, int rb) {
  if (threadIdx.x == 0) __hip_atomic_store(cnt + rb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float row_alpha(const GemvArgs& a, int k, int m) {
  if (a.alpha) return a.alpha[(size_t)k * a.M + m];
  if (a.alpha_h) return f16_bits_to_float(a.alpha_h[(size_t)k * a.M + m]);
  return 1.0f;
}

// Loads the (up to) 4 words of row `lane` of one layout tile.
__device__ inline void load_tile_words(const uint32_t* tile, int lane, int wg, uint32_t wd[4]) {
  if (wg == 4) {
    uint4 v = *(const uint4*)(tile + (size_t)lane * 4);
    wd[0] = v.x; wd[1] = v.y; wd[2] = v.z; wd[3] = v.w;
  } else {
    for (int j = 0; j < 4; ++j) wd[j] = j < wg ? tile[(size_t)lane * wg + j] : 0u;
  }
}

template <int BB>
__global__ void __launch_bounds__(64) k_gemv_f(GemvArgs a) {
  extern __shared__ __align__(16) float lut[];  // [KX][BB][G][16]
  const int lane = threadIdx.x;
  const int s = blockIdx.x;
  const int rb = blockIdx.y;
  const int w0 = s * a.wb;
  const int nw = min(a.wb, a.ND - w0);
  const int G = nw * 8;
  const int KX = a.colscale ? a.K : 1;

  // Stage: x' = c (.) x, then the 16 signed sums of every 4-column group.
  for (int idx = lane; idx < KX * BB * G; idx += 64) {
    const int g = idx % G;
    const int t = idx / G;
    const int b = t % BB;
    const int kx = t / BB;
    const int n0 = w0 * 32 + g * 4;
    const bool bok = (a.b0 + b) < a.B;
    float xv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = bok ? load_x(a.x, a.xdt, (size_t)(n0 + j) * a.B + a.b0 + b) : 0.0f;
      if (a.colscale) v *= f16_bits_to_float(a.colscale[(size_t)kx * a.N + n0 + j]);
      xv[j] = v;
    }
    const float p0 = xv[0] + xv[1], m0 = xv[0] - xv[1];
    const float p1 = xv[2] + xv[3], m1 = xv[2] - xv[3];
    const float A0 = -p0, A1 = m0, A2 = -m0, A3 = p0;
    const float Q[4] = {-p1, m1, -m1, p1};
    float4* dst = (float4*)(lut + ((size_t)(kx * BB + b) * G + g) * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = make_float4(A0 + Q[q], A1 + Q[q], A2 + Q[q], A3 + Q[q]);
  }
  __syncthreads();

  const int m = rb * 64 + lane;
  const bool valid = m < a.M;
  const int h = min(64, a.M - rb * 64);
  float tot[BB];
#pragma unroll
  for (int b = 0; b < BB; ++b) tot[b] = 0.0f;

  if (valid) {
    for (int k = 0; k < a.K; ++k) {
      const float* L = lut + (size_t)(a.colscale ? k : 0) * BB * G * 16;
      const uint32_t* base_k = a.bits + (size_t)k * a.plane + (size_t)rb * 64 * a.ND;
      float acc[BB];
#pragma unroll
      for (int b = 0; b < BB; ++b) acc[b] = 0.0f;
      for (int gw = 0; gw < nw; gw += 4) {
        const int g4 = (w0 + gw) >> 2;
        const int wg = min(4, a.ND - 4 * g4);
        uint32_t wd[4];
        load_tile_words(base_k + (size_t)g4 * 4 * h, lane, wg, wd);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j < wg) {
            const uint32_t word = wd[j];
            const float* Lw = L + (size_t)(gw + j) * 8 * 16;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int e = (word >> (4 * i)) & 15;
#pragma unroll
              for (int b = 0; b < BB; ++b) acc[b] += Lw[((size_t)b * G + i) * 16 + e];
            }
          }
        }
      }
      const float al = row_alpha(a, k, m);
#pragma unroll
      for (int b = 0; b < BB; ++b) tot[b] += al * acc[b];
    }
  }

  if (a.S == 1) {
    if (valid) {
#pragma unroll
      for (int b = 0; b < BB; ++b) {
        if (a.b0 + b < a.B) {
          const size_t yi = (size_t)m * a.B + a.b0 + b;
          a.y[yi] = (a.accumulate ? a.y[yi] : 0.0f) + tot[b];
        }
      }
    }
    return;
  }

  if (valid) {
#pragma unroll
    for (int b = 0; b < BB; ++b) a.part[((size_t)s * a.M + m) * BB + b] = tot[b];
  }
  if (!arrive_last(a.cnt, rb, a.S)) return;
  if (valid) {
    float sum[BB];
#pragma unroll
    for (int b = 0; b < BB; ++b) sum[b] = 0.0f;
    for (int s2 = 0; s2 < a.S; ++s2) {
#pragma unroll
      for (int b = 0; b < BB; ++b) sum[b] += a.part[((size_t)s2 * a.M + m) * BB + b];
    }
#pragma unroll
    for (int b = 0; b < BB; ++b) {
      if (a.b0 + b < a.B) {
        const size_t yi = (size_t)m * a.B + a.b0 + b;
        a.y[yi] = (a.accumulate ? a.y[yi] : 0.0f) + sum[b];
      }
    }
  }
  reset_counter(a.cnt, rb);
}

template <int BB>
__global__ void __launch_bounds__(64) k_gemv_i8(GemvI8Args a) {
  extern __shared__ __align__(16) uint32_t sh[];  // planes [nw][BB][8], then column sums [nw][BB]
  const int lane = threadIdx.x;
  const int s = blockIdx.x;
  const int rb = blockIdx.y;
  const int w0 = s * a.wb;
  const int nw = min(a.wb, a.ND - w0);
  uint32_t* planes = sh;
  int* csum = (int*)(sh + (size_t)nw * BB * 8);

  // Stage: two's-complement bit planes of xq for every sign word, and the
  // column sums of xq per word.
  for (int idx = lane; idx < nw * BB; idx += 64) {
    const int w = idx / BB;
    const int b = idx % BB;
    const bool bok = (a.b0 + b) < a.B;
    uint32_t pl[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int cs = 0;
    for (int j = 0; j < 32; ++j) {
      const int n = (w0 + w) * 32 + j;
      const int v = bok ? (int)a.xq[(size_t)n * a.B + a.b0 + b] : 0;
      cs += v;
      const uint32_t u = (uint32_t)(uint8_t)(int8_t)v;
#pragma unroll
      for (int p = 0; p < 8; ++p) pl[p] |= ((u >> p) & 1u) << j;
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) planes[((size_t)w * BB + b) * 8 + p] = pl[p];
    csum[(size_t)w * BB + b] = cs;
  }
  __syncthreads();

  const int m = rb * 64 + lane;
  const bool valid = m < a.M;
  const int h = min(64, a.M - rb * 64);
  float ysum[BB];
#pragma unroll
  for (int b = 0; b < BB; ++b) ysum[b] = 0.0f;

  for (int k = 0; k < a.K; ++k) {
    int acck[BB];
#pragma unroll
    for (int b = 0; b < BB; ++b) acck[b] = 0;
    if (valid) {
      const uint32_t* base_k = a.bits + (size_t)k * a.plane + (size_t)rb * 64 * a.ND;
      int cnt[BB][8];
      int xs[BB];
#pragma unroll
      for (int b = 0; b < BB; ++b) {
        xs[b] = 0;
#pragma unroll
        for (int p = 0; p < 8; ++p) cnt[b][p] = 0;
      }
      for (int gw = 0; gw < nw; gw += 4) {
        const int g4 = (w0 + gw) >> 2;
        const int wg = min(4, a.ND - 4 * g4);
        uint32_t wd[4];
        load_tile_words(base_k + (size_t)g4 * 4 * h, lane, wg, wd);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j < wg) {
            const uint32_t word = wd[j];
#pragma unroll
            for (int b = 0; b < BB; ++b) {
              const uint32_t* pl = planes + ((size_t)(gw + j) * BB + b) * 8;
#pragma unroll
              for (int p = 0; p < 8; ++p) cnt[b][p] += __builtin_popcount(word & pl[p]);
              xs[b] += csum[(size_t)(gw + j) * BB + b];
            }
          }
        }
      }
#pragma unroll
      for (int b = 0; b < BB; ++b) {
        int ones = -(cnt[b][7] << 7);
#pragma unroll
        for (int p = 0; p < 7; ++p) ones += cnt[b][p] << p;
        acck[b] = 2 * ones - xs[b];
      }
    }
    if (a.S == 1) {
      if (valid) {
        const float al = a.alpha ? a.alpha[(size_t)k * a.M + m] : 1.0f;
#pragma unroll
        for (int b = 0; b < BB; ++b) {
          if (a.b0 + b < a.B) {
            if (a.acc) a.acc[((size_t)k * a.M + m) * a.B + a.b0 + b] = acck[b];
            ysum[b] += al * (float)acck[b];
          }
        }
      }
    } else if (valid) {
#pragma unroll
      for (int b = 0; b < BB; ++b) a.part[(((size_t)s * a.K + k) * a.M + m) * BB + b] = acck[b];
    }
  }

  if (a.S > 1) {
    if (!arrive_last(a.cnt, rb, a.S)) return;
    if (valid) {
      for (int k = 0; k < a.K; ++k) {
        int sum[BB];
#pragma unroll
        for (int b = 0; b < BB; ++b) sum[b] = 0;
        for (int s2 = 0; s2 < a.S; ++s2) {
#pragma unroll
          for (int b = 0; b < BB; ++b) sum[b] += a.part[(((size_t)s2 * a.K + k) * a.M + m) * BB + b];
        }
        const float al = a.alpha ? a.alpha[(size_t)k * a.M + m] : 1.0f;
#pragma unroll
        for (int b = 0; b < BB; ++b) {
          if (a.b0 + b < a.B) {
            if (a.acc) a.acc[((size_t)k * a.M + m) * a.B + a.b0 + b] = sum[b];
            ysum[b] += al * (float)sum[b];
          }
        }
      }
    }
    reset_counter(a.cnt, rb);
  }

  if (valid && a.y) {
#pragma unroll
    for (int b = 0; b < BB; ++b) {
      if (a.b0 + b < a.B) {
        const size_t yi = (size_t)m * a.B + a.b0 + b;
        a.y[yi] = (a.accumulate ? a.y[yi] : 0.0f) + a.sx[a.b0 + b] * ysum[b];
      }
    }
  }
}

// ------------------------------------------------------------------ planning

static int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  int r = std::atoi(v);
  return r > 0 ? r : dflt;
}

static int batch_tile(int B, int K, bool i8) {
  int bb = B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : B <= 8 ? 8 : 16;
  if (!i8) {
    // fp32 tables: K * BB * 512 bytes per sign word must leave room for 4 words
    while (bb > 1 && K * bb > 32) bb >>= 1;
  }
  return bb;
}

GemvPlan plan_gemv(int K, int M, int N, int B, bool i8) {
  GemvPlan p{};
  const int ND = N / 32;
  p.BB = batch_tile(B, K, i8);
  p.nchunk = (B + p.BB - 1) / p.BB;
  p.nrb = (M + 63) / 64;
  const int target = env_int("BSG_TARGET_WGS", 1024);
  int S = (target + p.nrb - 1) / p.nrb;
  S = S < 1 ? 1 : S;
  if (p.nrb > kMaxRowBlocksSplit) S = 1;
  const int maxS = (ND + 3) / 4;
  S = S > maxS ? maxS : S;
  int wb = (ND + S - 1) / S;
  wb = (wb + 3) / 4 * 4;
  const size_t per_word = i8 ? (size_t)p.BB * 36 : (size_t)K * p.BB * 512;
  int wb_max = (int)(65536 / per_word) / 4 * 4;
  if (wb_max < 4) wb_max = 4;
  if (wb > wb_max) wb = wb_max;
  p.wb = wb;
  p.S = (ND + wb - 1) / wb;
  if (p.S > 1) {
    p.part_bytes = align_up((size_t)p.S * M * p.BB * 4 * (i8 ? K : 1), 256);
    p.ws_bytes = kCounterBytes + p.part_bytes;
  }
  return p;
}

hipError_t launch_gemv_f(const GemvArgs& a0, const GemvPlan& p, hipStream_t st) {
  const int KX = a0.colscale ? a0.K : 1;
  const size_t lds = (size_t)KX * p.BB * p.wb * 8 * 16 * sizeof(float);
  dim3 grid(p.S, p.nrb);
  for (int c = 0; c < p.nchunk; ++c) {
    GemvArgs a = a0;
    a.b0 = c * p.BB;
    switch (p.BB) {
      case 1: hipLaunchKernelGGL(k_gemv_f<1>, grid, dim3(64), lds, st, a); break;
      case 2: hipLaunchKernelGGL(k_gemv_f<2>, grid, dim3(64), lds, st, a); break;
      case 4: hipLaunchKernelGGL(k_gemv_f<4>, grid, dim3(64), lds, st, a); break;
      case 8: hipLaunchKernelGGL(k_gemv_f<8>, grid, dim3(64), lds, st, a); break;
      default: hipLaunchKernelGGL(k_gemv_f<16>, grid, dim3(64), lds, st, a); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemv_i8(const GemvI8Args& a0, const GemvPlan& p, hipStream_t st) {
  const size_t lds = (size_t)p.wb * p.BB * 9 * sizeof(uint32_t);
  dim3 grid(p.S, p.nrb);
  for (int c = 0; c < p.nchunk; ++c) {
    GemvI8Args a = a0;
    a.b0 = c * p.BB;
    switch (p.BB) {
      case 1: hipLaunchKernelGGL(k_gemv_i8<1>, grid, dim3(64), lds, st, a); break;
      case 2: hipLaunchKernelGGL(k_gemv_i8<2>, grid, dim3(64), lds, st, a); break;
      case 4: hipLaunchKernelGGL(k_gemv_i8<4>, grid, dim3(64), lds, st, a); break;
      case 8: hipLaunchKernelGGL(k_gemv_i8<8>, grid, dim3(64), lds, st, a); break;
      default: hipLaunchKernelGGL(k_gemv_i8<16>, grid, dim3(64), lds, st, a); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bsg
