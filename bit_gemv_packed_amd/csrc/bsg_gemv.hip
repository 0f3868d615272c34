// Binary-base product for gfx950 (float activations):
//
//   y[m,b] (= or +=) sum_k alpha_k[m] sum_n (2 bit_k(m,n) - 1) c_k[n] x[n,b]
//
// Work decomposition.  A workgroup owns RW = 64/Q complete output rows, so
// no reduction crosses workgroups: the result is deterministic and needs no
// workspace.  Q lanes of a wavefront share a row.  The W wavefronts of the
// workgroup split the input dimension into chunks of CW = Q*NWL sign words
// (NCH chunks each); inside a chunk, the lanes of quarter q read NWL
// consecutive words of their row.  The Q partial sums of a row are combined
// by two lane shuffles, the W wavefront sums through LDS, in a fixed order.
//
// Activation tables (FluxBin Sec. 2 "LUT-based Multiplication": split x into
// sub-vectors, precompute every signed combination, use the weight bit
// pattern as the table address; Sec. 3.2 Stage 1: fold the column scale into
// x while building the table).  Sub-vectors are 4 columns wide: 16 fp32
// entries per table.  Each wavefront builds the tables of its own chunk in
// its own LDS region, laid out [step][quarter][16 entries] with 16 pad bytes
// after each step row: at every lookup the lanes of a quarter read one
// 64-byte table and the Q tables of one instruction occupy disjoint bank
// groups, and the pad staggers the tables that different lanes write at
// once across the banks, so neither reads nor writes conflict.
// Table addresses take one SDWA add per 4-bit slice: the sign word is
// rotated by 2 bits each way and masked once, after which byte j of the
// masked rotation is (slice value) * 4.  Per 32 weights: 2 rotates, 2 masks,
// 8 SDWA adds, 8 LDS reads and 8 fp32 adds.
#include "bsg_prod.h"

#include <cstdlib>

namespace bsg {

// A float at an LDS byte address (the address already includes the base of
// the dynamic LDS block), read with the address in one VGPR.
typedef __attribute__((address_space(3))) const float lds_cf32;
__device__ inline float lds_f32(uint32_t addr) { return *(lds_cf32*)(uintptr_t)addr; }

__device__ inline float row_alpha(const ProdArgs& a, int k, int m) {
  if (a.alpha) return a.alpha[(size_t)k * a.M + m];
  if (a.alpha_h) return f16_bits_to_float(a.alpha_h[(size_t)k * a.M + m]);
  return 1.0f;
}

// Raw activation bits -> fp32 (fp32 bits, or a bf16 / fp16 pattern in the low half).
__device__ inline float decode_x(uint32_t raw, int xdt) {
  if (xdt == BSG_F32) return __uint_as_float(raw);
  if (xdt == BSG_BF16) return __uint_as_float(raw << 16);
  return f16_bits_to_float((uint16_t)raw);
}

// Activations and column scales of one 4-column group, as raw bits; loaded
// one chunk ahead of the table build so that their latency overlaps the
// sign-word loads and the previous chunk's lookups.
template <int KM, int BB>
struct ActRaw {
  uint32_t x[BB][4];
  uint2 c[KM];
};

// XM = 1 (bf16) and 2 (fp16): one batch column of 16-bit activations, x
// 16-byte and column scales 8-byte aligned: one 8-byte load of x and one per
// base of scales, straight-line (without column scales the scale loads read
// x instead and are ignored).  XM = 0: any batch, dtype and alignment,
// element loads.
template <int KM, int BB, int XM>
__device__ inline void fetch_act(const ProdArgs& a, bool cs, int n0, ActRaw<KM, BB>& r) {
  const int nc = n0 < a.N ? n0 : 0;  // columns beyond N load column 0 (the build zeroes them)
  if (XM != 0) {
    const uint2 v = *(const uint2*)((const uint16_t*)a.x + nc);
    r.x[0][0] = v.x & 0xffffu;
    r.x[0][1] = v.x >> 16;
    r.x[0][2] = v.y & 0xffffu;
    r.x[0][3] = v.y >> 16;
    const uint16_t* cbase = cs ? a.colscale : (const uint16_t*)a.x;
    const size_t cstride = cs ? (size_t)a.N : 0;
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (base_active<KM>(a, k)) r.c[k] = *(const uint2*)(cbase + (size_t)k * cstride + nc);
  } else {
#pragma unroll
    for (int b = 0; b < BB; ++b) {
      const int bb = a.b0 + b < a.B ? a.b0 + b : a.B - 1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t i = (size_t)(nc + j) * a.B + bb;
        r.x[b][j] = a.xdt == BSG_F32 ? __float_as_uint(((const float*)a.x)[i]) : (uint32_t)((const uint16_t*)a.x)[i];
      }
    }
    if (cs) {
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        if (base_active<KM>(a, k)) {
          const uint16_t* p = a.colscale + (size_t)k * a.N + nc;
          r.c[k] = make_uint2((uint32_t)p[0] | ((uint32_t)p[1] << 16), (uint32_t)p[2] | ((uint32_t)p[3] << 16));
        }
      }
    }
  }
}

// Lookups of one chunk: acc[k][b] += table entry of each 4-bit slice.
// FULL: every word of the chunk exists (no per-word guard).
template <int Q, int NWL, int KM, int BB, bool FULL>
__device__ inline void lookup_chunk(const ProdArgs& a, const char* lds, uint32_t wbase_lds, bool cs, int q, int lw0,
                                    const uint32_t (&cur)[KM][NWL], float (&acc)[KM][BB]) {
  constexpr uint32_t ROWB = Q * 64 + 16;             // bytes of one step row of tables
  constexpr uint32_t REG = NWL * 8 * ROWB;           // bytes of one (base, batch column) table set
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (base_active<KM>(a, k)) {
      const uint32_t lbase =
          (uint32_t)(uintptr_t)(lds + wbase_lds + (uint32_t)(cs ? k : 0) * BB * REG + (uint32_t)q * 64);
#pragma unroll
      for (int j = 0; j < NWL; ++j) {
        if (FULL || lw0 + j < a.ND) {
          const uint32_t word = cur[k][j];
          const uint32_t rl = __builtin_amdgcn_alignbit(word, word, 30) & 0x3c3c3c3cu;  // even slices * 4
          const uint32_t rr = __builtin_amdgcn_alignbit(word, word, 2) & 0x3c3c3c3cu;   // odd slices * 4
          uint32_t ad[8];
          ad[0] = byte_add<0>(lbase, rl);
          ad[1] = byte_add<0>(lbase, rr);
          ad[2] = byte_add<1>(lbase, rl);
          ad[3] = byte_add<1>(lbase, rr);
          ad[4] = byte_add<2>(lbase, rl);
          ad[5] = byte_add<2>(lbase, rr);
          ad[6] = byte_add<3>(lbase, rl);
          ad[7] = byte_add<3>(lbase, rr);
#pragma unroll
          for (int n = 0; n < 8; ++n) {
#pragma unroll
            for (int b = 0; b < BB; ++b)
              acc[k][b] += lds_f32(ad[n] + (uint32_t)(j * 8 + n) * ROWB + (uint32_t)b * REG);
          }
        }
      }
    }
  }
}

template <int Q, int NWL, int KM, int BB, int XM>
__global__ void __launch_bounds__(1024) k_prod_f(ProdArgs a) {
  constexpr int RW = 64 / Q;
  constexpr int CW = Q * NWL;
  constexpr int G = CW * 8;           // 4-column groups per chunk (<= 64: one per lane)
  constexpr int STEPS = NWL * 8;                // groups per lane quarter
  constexpr uint32_t ROWB = Q * 64 + 16;        // bytes of one step row: Q tables + 16 pad bytes
  constexpr uint32_t REG = STEPS * ROWB;        // bytes of one (base, batch column) table set
  extern __shared__ __align__(16) char lds[];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wavefront index (uniform)
  const int q = lane / RW;
  const int r = lane % RW;
  const int m = blockIdx.x * RW + r;
  const bool valid = m < a.M;
  const int mload = valid ? m : a.M - 1;  // rows beyond M load a valid row; their sums are dropped
  const bool cs = a.colscale != nullptr;
  const int KX = cs ? a.K : 1;
  const int ndfull = a.ND & ~3;           // words in complete 4-word layout tiles
  const uint32_t wbase_lds = (uint32_t)wv * a.wave_lds;
  const bool builder = lane < G;  // this lane builds the tables of group `lane`

  float acc[KM][BB];
#pragma unroll
  for (int k = 0; k < KM; ++k)
#pragma unroll
    for (int b = 0; b < BB; ++b) acc[k][b] = 0.0f;

  // First chunk: sign words, then activations and column scales, all in flight at once.
  uint32_t cur[KM][NWL], nxt[KM][NWL];
  ActRaw<KM, BB> act;
  {
    const int cw0 = wv * a.NCH * CW;
    load_chunk<KM, NWL>(a, cw0 + CW <= ndfull, mload, cw0 + q * NWL, cur);
    fetch_act<KM, BB, XM>(a, cs, cw0 * 32 + (builder ? lane : 0) * 4, act);
  }

  for (int c = 0; c < a.NCH; ++c) {
    const int cw0 = (wv * a.NCH + c) * CW;  // first word of the chunk
    if (c + 1 < a.NCH) load_chunk<KM, NWL>(a, cw0 + 2 * CW <= ndfull, mload, cw0 + CW + q * NWL, nxt);

    // ---- tables: the 16 signed sums of 4-column group `lane` of the chunk
    if (builder) {
      const int qq = lane / STEPS, ii = lane % STEPS;
      const bool inb = cw0 * 32 + lane * 4 < a.N;
#pragma unroll
      for (int kx = 0; kx < KM; ++kx) {
        if (kx < KX) {
#pragma unroll
          for (int b = 0; b < BB; ++b) {
            float xv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float d = XM == 1   ? bf16_bits_to_float((uint16_t)act.x[b][j])
                              : XM == 2 ? f16_bits_to_float((uint16_t)act.x[b][j])
                                        : decode_x(act.x[b][j], a.xdt);
              xv[j] = (inb && a.b0 + b < a.B) ? d : 0.0f;
            }
            if (cs) {
              xv[0] *= f16_bits_to_float((uint16_t)(act.c[kx].x & 0xffffu));
              xv[1] *= f16_bits_to_float((uint16_t)(act.c[kx].x >> 16));
              xv[2] *= f16_bits_to_float((uint16_t)(act.c[kx].y & 0xffffu));
              xv[3] *= f16_bits_to_float((uint16_t)(act.c[kx].y >> 16));
            }
            // entry e = sum_j (2 bit_j(e) - 1) xv[j]: bits 0,1 select the first pair sum, bits 2,3 the second
            const float p0 = xv[0] + xv[1], m0 = xv[0] - xv[1];
            const float p1 = xv[2] + xv[3], m1 = xv[2] - xv[3];
            const float hi[4] = {-p1, m1, -m1, p1};
            float4* dst = (float4*)(lds + wbase_lds + (uint32_t)(kx * BB + b) * REG + (uint32_t)ii * ROWB +
                                    (uint32_t)qq * 64);
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[e] = make_float4(-p0 + hi[e], m0 + hi[e], -m0 + hi[e], p0 + hi[e]);
          }
        }
      }
    }
    if (c + 1 < a.NCH) fetch_act<KM, BB, XM>(a, cs, (cw0 + CW) * 32 + (builder ? lane : 0) * 4, act);
    __syncthreads();

    // ---- lookups: one table read and one add per 4 weights
    if (cw0 + CW <= a.ND)
      lookup_chunk<Q, NWL, KM, BB, true>(a, lds, wbase_lds, cs, q, cw0 + q * NWL, cur, acc);
    else
      lookup_chunk<Q, NWL, KM, BB, false>(a, lds, wbase_lds, cs, q, cw0 + q * NWL, cur, acc);

    if (c + 1 < a.NCH) {
      __syncthreads();  // the next chunk's tables overwrite these
#pragma unroll
      for (int k = 0; k < KM; ++k)
#pragma unroll
        for (int j = 0; j < NWL; ++j) cur[k][j] = nxt[k][j];
    }
  }

  // ---- row scales, then the Q lanes of a row, then the W wavefronts
  float tot[BB];
#pragma unroll
  for (int b = 0; b < BB; ++b) tot[b] = 0.0f;
  if (valid) {
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (base_active<KM>(a, k)) {
        const float al = row_alpha(a, k, m);
#pragma unroll
        for (int b = 0; b < BB; ++b) tot[b] += al * acc[k][b];
      }
    }
  }
#pragma unroll
  for (int b = 0; b < BB; ++b) {
    if (Q >= 4) tot[b] += __shfl_xor(tot[b], 16);
    if (Q >= 2) tot[b] += __shfl_xor(tot[b], 32);
  }
  float* red = (float*)(lds + (size_t)a.W * a.wave_lds);
  if (q == 0) {
#pragma unroll
    for (int b = 0; b < BB; ++b) red[(wv * RW + r) * BB + b] = tot[b];
  }
  __syncthreads();
  for (int t = threadIdx.x; t < RW * BB; t += blockDim.x) {  // blockDim may be below RW * BB
    const int rr = t / BB, b = t % BB;
    const int mm = blockIdx.x * RW + rr;
    if (mm < a.M && a.b0 + b < a.B) {
      float s = 0.0f;
      for (int w = 0; w < a.W; ++w) s += red[(w * RW + rr) * BB + b];
      const size_t yi = (size_t)mm * a.B + a.b0 + b;
      a.y[yi] = (a.accumulate ? a.y[yi] : 0.0f) + s;
    }
  }
}

// ------------------------------------------------------------------ planning

static int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  const int r = std::atoi(v);
  return r > 0 ? r : dflt;
}

ProdPlan plan_prod(int K, int M, int N, int B, bool colscale, bool i8) {
  ProdPlan p{};
  const int ND = N / 32;
  p.KM = K <= 4 ? K : 8;
  p.BB = B <= 1 ? 1 : B <= 2 ? 2 : 4;
  p.nlaunch = (B + p.BB - 1) / p.BB;
  // lanes per row: the fewest that still give at least 256 workgroups
  const int forceQ = env_int("BSG_Q", 0);
  if (forceQ == 1 || forceQ == 2 || forceQ == 4) {
    p.Q = forceQ;
  } else {
    p.Q = 4;
    for (int qq = 1; qq <= 4; qq *= 2) {
      if ((M + 64 / qq - 1) / (64 / qq) >= 256) {
        p.Q = qq;
        break;
      }
    }
  }
  p.RW = 64 / p.Q;
  const int KX = (colscale && !i8) ? K : 1;
  // 8-word chunks (256 columns) for one batch column and K <= 2; 4-word
  // chunks otherwise (smaller tables and register sets)
  p.CW = (p.BB == 1 && p.KM <= 2) ? 8 : 4;
  p.NWL = p.CW / p.Q;
  p.wave_lds = i8 ? (size_t)p.CW * p.BB * 12 * 4 : (size_t)KX * p.BB * (p.NWL * 8) * (p.Q * 64 + 16);
  const int T = (ND + p.CW - 1) / p.CW;  // chunks
  int W = env_int("BSG_WAVES", 16);
  W = W > 16 ? 16 : W;
  W = W > T ? T : W;
  const size_t red_per_wave = (size_t)p.RW * p.BB * 4 * (i8 ? p.KM : 1);
  while (W > 1 && (size_t)W * (p.wave_lds + red_per_wave) > kMaxLds) --W;
  p.W = W < 1 ? 1 : W;
  p.NCH = (T + p.W - 1) / p.W;
  p.nwg = (M + p.RW - 1) / p.RW;
  p.lds = (size_t)p.W * (p.wave_lds + red_per_wave);
  return p;
}

static hipError_t dispatch_f(const ProdArgs& a, const ProdPlan& p, hipStream_t st) {
  switch (prod_key(p.Q, p.NWL, p.KM, p.BB, p.XM)) {
#define BSG_CASE(Q, NWL, KM, BB, XM) \
  case prod_key(Q, NWL, KM, BB, XM): return launch_one(k_prod_f<Q, NWL, KM, BB, XM>, p, a, st);
    BSG_PROD_F_INSTANCES(BSG_CASE)
#undef BSG_CASE
    default: return hipErrorInvalidConfiguration;
  }
}

hipError_t launch_prod_f(const ProdArgs& a0, const ProdPlan& p0, hipStream_t st) {
  ProdPlan p = p0;
  p.XM = (a0.B == 1 && a0.xvec && a0.xdt != BSG_F32) ? (a0.xdt == BSG_BF16 ? 1 : 2) : 0;
  for (int c = 0; c < p.nlaunch; ++c) {
    ProdArgs a = a0;
    a.b0 = c * p.BB;
    a.W = p.W;
    a.NCH = p.NCH;
    a.wave_lds = (uint32_t)p.wave_lds;
    const hipError_t e = dispatch_f(a, p, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bsg
