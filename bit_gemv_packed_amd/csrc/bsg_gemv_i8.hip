// Sign product with int8 activations for gfx950, exact in int32:
//
//   acc_k[m,b] = sum_n (2 bit_k(m,n) - 1) xq[n,b]
//   y[m,b] (= or +=) sx[b] * sum_k alpha_k[m] acc_k[m,b]
//
// With the two's-complement bit planes P_p of xq over the 32 columns of a
// sign word, sum_{bit=1} xq = sum_{p<7} 2^p popcount(word & P_p)
// - 128 popcount(word & P_7), and sum_n (2 bit - 1) xq = 2 sum_{bit=1} xq -
// sum_n xq: per 32 weights 8 AND and 8 popcount-accumulate, no table.  Each
// wavefront makes the planes of its chunk with 8 ballots per two sign words
// and stores them as [word][batch column][8 planes, column sum, 3 pad]
// (48 bytes, two 16-byte reads).  The work decomposition is the one of the
// float path (bsg_gemv.hip): complete rows per workgroup, no cross-workgroup
// reduction, fixed summation order.
#include "bsg_prod.h"

namespace bsg {

template <int Q, int NWL, int KM, int BB, int XM>
__global__ void __launch_bounds__(64 * prod_max_waves(KM, BB)) k_prod_i8(ProdArgs a) {
  constexpr int RW = 64 / Q;
  constexpr int CW = Q * NWL;
  extern __shared__ __align__(16) char lds[];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wavefront index (uniform)
  const int q = lane / RW;
  const int r = lane % RW;
  const int m = blockIdx.x * RW + r;
  const bool valid = m < a.M;
  // rows beyond M read padding; their sums are dropped
  const SignRows<KM> srows = sign_rows<KM, RW>(a.bits, a.plane, a.K, a.ND, blockIdx.x, m);
  const rsrc_t xsrc = make_rsrc(a.xq, (size_t)a.N * a.B);
  uint32_t* pl = (uint32_t*)(lds + (size_t)wv * a.wave_lds);

  int cnt[KM][BB][8];
  int xs[BB];
#pragma unroll
  for (int b = 0; b < BB; ++b) {
    xs[b] = 0;
#pragma unroll
    for (int k = 0; k < KM; ++k)
#pragma unroll
      for (int p = 0; p < 8; ++p) cnt[k][b][p] = 0;
  }

  // activations of a chunk: column (cw0 + 2u) * 32 + lane for u < CW/2,
  // unconditional loads (columns beyond N read 0; batch columns beyond B
  // read column B-1 and are zeroed when used)
  int xv[CW / 2][BB], xn[CW / 2][BB];
  auto fetch_xq = [&](int cw0, int (&dst)[CW / 2][BB]) {
#pragma unroll
    for (int u = 0; u < CW / 2; ++u) {
      const int n = (cw0 + 2 * u) * 32 + lane;
#pragma unroll
      for (int b = 0; b < BB; ++b) {
        const int bb = a.b0 + b < a.B ? a.b0 + b : a.B - 1;
        dst[u][b] = (int)(int8_t)ld8(xsrc, (uint32_t)(n * a.B + bb));  // 0 beyond N
      }
    }
  };
  auto keep_xq = [&](int cw0, int u, int b, int v) {
    return ((cw0 + 2 * u) * 32 + lane < a.N && a.b0 + b < a.B) ? v : 0;
  };

  // activations first: loads complete in issue order, so the bit planes need
  // not wait for the sign words
  uint32_t cur[KM][NWL], nxt[KM][NWL];
  fetch_xq(wv * a.NCH * CW, xv);
  load_chunk<KM, NWL>(a, srows, wv * a.NCH * CW + q * NWL, cur);

  for (int c = 0; c < a.NCH; ++c) {
    const int cw0 = (wv * a.NCH + c) * CW;
    if (c + 1 < a.NCH) {
      fetch_xq(cw0 + CW, xn);
      load_chunk<KM, NWL>(a, srows, cw0 + CW + q * NWL, nxt);
    }

    // ---- bit planes: one ballot over 64 lanes covers two sign words
#pragma unroll
    for (int u = 0; u < CW / 2; ++u) {
#pragma unroll
      for (int b = 0; b < BB; ++b) {
        const int v = keep_xq(cw0, u, b, xv[u][b]);
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const unsigned long long bal = __ballot((v >> p) & 1);
          lo[p] = (uint32_t)bal;
          hi[p] = (uint32_t)(bal >> 32);
        }
        if (lane == 0 || lane == 32) {
          const int wl = 2 * u + (lane == 32 ? 1 : 0);
          uint32_t* dst = pl + ((size_t)wl * BB + b) * 12;
          int sum = 0;
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            const uint32_t bits = lane == 0 ? lo[p] : hi[p];
            dst[p] = bits;
            sum += (p == 7 ? -128 : (1 << p)) * __builtin_popcount(bits);
          }
          dst[8] = (uint32_t)sum;
        }
      }
    }
    wave_sync();  // the planes are private to this wavefront

    // words beyond ND are zero (padding, or out of range) and so are the
    // planes of their columns: they add 0, no guard
#pragma unroll
    for (int j = 0; j < NWL; ++j) {
      {
#pragma unroll
        for (int b = 0; b < BB; ++b) {
          const uint32_t* src = pl + ((size_t)(q * NWL + j) * BB + b) * 12;
          const uint4 P0 = *(const uint4*)src;
          const uint4 P1 = *(const uint4*)(src + 4);
          const uint32_t P[8] = {P0.x, P0.y, P0.z, P0.w, P1.x, P1.y, P1.z, P1.w};
          xs[b] += (int)src[8];
#pragma unroll
          for (int k = 0; k < KM; ++k) {
            if (base_active<KM>(a, k)) {
#pragma unroll
              for (int p = 0; p < 8; ++p) cnt[k][b][p] += __builtin_popcount(cur[k][j] & P[p]);
              // finish this word's counts here (left free, the compiler sinks
              // them to the end of the loop body and runs out of registers)
#pragma unroll
              for (int p = 0; p < 8; ++p) asm volatile("" : "+v"(cnt[k][b][p]));
            }
          }
        }
      }
    }
    wave_sync();  // the next chunk's planes overwrite these
    if (c + 1 < a.NCH) {
#pragma unroll
      for (int k = 0; k < KM; ++k)
#pragma unroll
        for (int j = 0; j < NWL; ++j) cur[k][j] = nxt[k][j];
#pragma unroll
      for (int u = 0; u < CW / 2; ++u)
#pragma unroll
        for (int b = 0; b < BB; ++b) xv[u][b] = xn[u][b];
    }
  }

  // exact int32 per (base, batch column): this lane, the Q lanes of the row,
  // then the W wavefronts
  int* red = (int*)(lds + (size_t)a.W * a.wave_lds);
#pragma unroll
  for (int k = 0; k < KM; ++k) {
#pragma unroll
    for (int b = 0; b < BB; ++b) {
      int ones = -(cnt[k][b][7] << 7);
#pragma unroll
      for (int p = 0; p < 7; ++p) ones += cnt[k][b][p] << p;
      int v = 2 * ones - xs[b];
      if (Q >= 4) v += __shfl_xor(v, 16);
      if (Q >= 2) v += __shfl_xor(v, 32);
      if (q == 0 && k < a.K) red[((wv * RW + r) * KM + k) * BB + b] = v;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < RW * BB; t += blockDim.x) {  // blockDim may be below RW * BB
    const int rr = t / BB, b = t % BB;
    const int mm = blockIdx.x * RW + rr;
    if (mm < a.M && a.b0 + b < a.B) {
      float ysum = 0.0f;
      for (int k = 0; k < a.K; ++k) {
        const int s = sum_waves(red + (rr * KM + k) * BB + b, RW * KM * BB, a.W);
        if (a.acc) a.acc[((size_t)k * a.M + mm) * a.B + a.b0 + b] = s;
        if (a.y) ysum += (a.alpha ? a.alpha[(size_t)k * a.M + mm] : 1.0f) * (float)s;
      }
      if (a.y) {
        const size_t yi = (size_t)mm * a.B + a.b0 + b;
        a.y[yi] = (a.accumulate ? a.y[yi] : 0.0f) + a.sx[a.b0 + b] * ysum;
      }
    }
  }
}

static hipError_t dispatch_i8(const ProdArgs& a, const ProdPlan& p, hipStream_t st) {
  switch (prod_key(p.Q, p.NWL, p.KM, p.BB, 0)) {
#define BSG_CASE(Q, NWL, KM, BB, XM) \
  case prod_key(Q, NWL, KM, BB, XM): return launch_one(k_prod_i8<Q, NWL, KM, BB, XM>, p, a, st);
    BSG_PROD_I8_INSTANCES(BSG_CASE)
#undef BSG_CASE
    default: return hipErrorInvalidConfiguration;
  }
}

hipError_t launch_prod_i8(const ProdArgs& a0, const ProdPlan& p, hipStream_t st) {
  for (int c = 0; c < p.nlaunch; ++c) {
    ProdArgs a = a0;
    a.b0 = c * p.BB;
    a.W = p.W;
    a.NCH = p.NCH;
    a.wave_lds = (uint32_t)p.wave_lds;
    const hipError_t e = dispatch_i8(a, p, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bsg
