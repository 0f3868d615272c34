// Batched sign product on the matrix cores (gfx950), for B >= 4 batch
// columns of bf16 or fp16 activations without column scales:
//
//   y[m,b] (= or +=) sum_k alpha_k[m] sum_n (2 bit_k(m,n) - 1) x[n,b]
//
// With several batch columns the product is a dense contraction, so it runs
// as v_mfma_f32_16x16x32_{bf16,f16}: A = 16 rows x 32 columns of signs,
// B = 32 columns x 16 batch columns of x, C = fp32 16 x 16.  The A values
// are +-2 (exact in bf16 and fp16), so the products with x are exact and
// the sums are fp32; the result is scaled by -1/2 at the end (exact).
//
// Work decomposition.  A workgroup owns RT tiles of 16 complete rows (16 RT
// divides 64: all in one row block of the sign layout); its W wavefronts
// split the 4-step layout tiles (NCH / 4 each).  Each wavefront streams its
// tiles: the sign words and the x block of tile t + 1 are loaded while tile
// t is multiplied, so every load has a whole tile of work to arrive.
//
// A operand.  Tile t holds 4 sign words of each row (one per 32-column
// step); lane l (row l % 16, k group g = l / 16) loads word g of its row (4
// bytes, no two lanes alike), and MFMA j of the tile uses byte j of it:
// columns 32 g + 8 j .. + 7.  The byte is copied into both 16-bit halves of
// a word (one byte permute) and each half shifted so that bits 2i, 2i + 1
// land on the sign bits of word i; masking and or-ing in the exponent of 2.0
// gives -2 for a set bit and +2 for a clear one.  Nine VALU operations per 8
// values, no memory traffic.
//
// B operand.  x is stored [N][B] (a batch row per column), so each wavefront
// transposes the 128 x 16 x block of a tile through its own LDS tile,
// [batch column][128 + 8 pad] (32 two-byte writes per lane), and lane l
// (batch column l % 16, k group g) reads the same 8 columns as its A operand
// with one 16-byte read per MFMA, shared by the RT * KM products; row stride
// 68 banks: conflict-free.
//
// Reduction.  The W partial C tiles are summed through LDS in a fixed
// order: no atomics, deterministic.
//
// Steps beyond N read zero sign words (layout padding) and zero x (offsets
// past the end of x) and add nothing.
#include <algorithm>
#include <cstdlib>

#include "bsg_prod.h"

namespace bsg {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((address_space(3))) const u32x4 lds_cu4;
__device__ inline uint4 lds_u4(uint32_t addr) {
  const u32x4 v = *(lds_cu4*)(uintptr_t)addr;
  return make_uint4(v[0], v[1], v[2], v[3]);
}
typedef __attribute__((address_space(3))) uint16_t lds_u16;

template <int XT>
__device__ inline f32x4 mfma_step(uint4 av, uint4 bv, f32x4 c) {
  if (XT == 1)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv),
                                                   c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av), __builtin_bit_cast(f16x8, bv), c,
                                                0, 0, 0);
}

// A operand of one lane: the 8 signs of byte J of sign word w as -2 (bit
// set) / +2 (bit clear) in bf16 / fp16 (both encode 2.0 as 0x4000).
// msk = 0x80008000, passed in a scalar register so that mask and or-in take
// one v_and_or_b32.
template <int J>
__device__ inline uint4 a_operand(uint32_t w, uint32_t msk) {
  const u16x2 t = __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(0u, w, 0x0c000c00u | (J << 16) | J));
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u16x2 sh = t << u16x2{(unsigned short)(15 - 2 * i), (unsigned short)(14 - 2 * i)};
    d[i] = (__builtin_bit_cast(uint32_t, sh) & msk) | 0x40004000u;
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

constexpr int kXtRow = 136;                      // halves per batch row of a tile (128 + 8 pad)
constexpr uint32_t kXtBytes = 16 * kXtRow * 2;   // one 4-step tile of x in LDS

// Most wavefronts per workgroup: 16, or 8 where the accumulators, sign words
// and x loads in flight need more than 128 VGPRs (RT * KM >= 4; 2-byte
// loads: 32 per tile; 4-byte loads with RT * KM = 3): up to 256, no spills.
constexpr int mfma_max_waves(int RT, int KM, int VW) {
  return (RT * KM >= 4 || VW == 1 || (VW == 2 && RT * KM >= 3)) ? 8 : 16;
}

template <int RT, int KM>
struct MfTile {
  uint32_t w[RT][KM];  // word g of the lane's row, per row tile and base
  uint32_t x[4][4];    // per step: 8 batch values of column 32 step + lane % 32
};

// XT: 1 bf16, 2 fp16 activations.  VW: batch values per x load (8, 4, 2 or
// 1: B % VW == 0 and x aligned to 2 VW bytes).  MP = 1: the fused launch of
// several projections (bs_gemv_multi).
template <int RT, int KM, int XT, int VW, int MP>
__global__ void __launch_bounds__(64 * mfma_max_waves(RT, KM, VW)) k_prod_mfma(ProdArgs a) {
  asm volatile("" ::"s"(a.bits), "s"(a.alpha), "s"(a.x), "s"(a.y), "s"(a.plane), "s"(a.K), "s"(a.M), "s"(a.N),
               "s"(a.ND), "s"(a.B), "s"(a.b0), "s"(a.accumulate), "s"(a.NCH), "s"(a.x_bytes), "s"(a.al_bytes));
  // fused launch: this workgroup's projection (constant indices only: a
  // computed index would copy the arguments to scratch memory)
  uint32_t blk = blockIdx.x;
  if (MP) {
    ProjDesc d = a.proj[0];
#pragma unroll
    for (int i = 1; i < kMaxProj; ++i)
      if (i < a.np && (int)blockIdx.x >= a.proj[i].wg0) d = a.proj[i];
    a.bits = d.bits;
    a.alpha = d.alpha;
    a.y = d.y;
    a.plane = d.plane;
    a.M = d.M;
    a.al_bytes = d.al_bytes;
    blk = blockIdx.x - d.wg0;
  }
  extern __shared__ __align__(16) char lds[];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int m0 = (int)(blk * 16 * RT);
  const uint32_t xt = (uint32_t)(uintptr_t)lds + (uint32_t)wv * kXtBytes;
  uint32_t msk;
  asm volatile("s_mov_b32 %0, 0x80008000" : "=s"(msk));

  SignRows<KM> sr[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) sr[rt] = sign_rows<KM, 16 * RT>(a.bits, a.plane, a.K, a.ND, blk, m0 + rt * 16 + r16);
  const rsrc_t xs = make_rsrc(a.x, a.x_bytes);

  f32x4 acc[RT][KM];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int k = 0; k < KM; ++k) acc[rt][k] = f32x4{0.f, 0.f, 0.f, 0.f};

  // This lane's x: column 32 step + lane % 32, batch columns bb .. bb + 7.
  // Loads of batch columns >= B start at an offset past the end of x and
  // read zero (so do columns >= N).
  const int nl = lane & 31, bh = lane >> 5;
  const int bb = a.b0 + bh * 8;
  constexpr int NL = 8 / VW;  // loads per step
  constexpr uint32_t kOut = 0x80000000u;
  uint32_t xo[NL];
#pragma unroll
  for (int q = 0; q < NL; ++q) xo[q] = bb + q * VW < a.B ? (uint32_t)(nl * a.B + bb + q * VW) * 2u : kOut;
  const uint32_t xstep = 64u * (uint32_t)a.B;  // bytes of x per step

  auto load_tile = [&](int t, MfTile<RT, KM>& d) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int k = 0; k < KM; ++k) d.w[rt][k] = ld32(sr[rt].r[k], (uint32_t)t * 1024u + sr[rt].row_off + (uint32_t)g * 4u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t so = (uint32_t)(4 * t + j) * xstep;
#pragma unroll
      for (int q = 0; q < NL; ++q) {
        if (VW == 8) {
          const uint4 v = ld128(xs, xo[q] + so);
          d.x[j][0] = v.x;
          d.x[j][1] = v.y;
          d.x[j][2] = v.z;
          d.x[j][3] = v.w;
        } else if (VW == 4) {
          const uint2 v = ld64(xs, xo[q] + so);
          d.x[j][2 * q] = v.x;
          d.x[j][2 * q + 1] = v.y;
        } else if (VW == 2) {
          d.x[j][q] = ld32(xs, xo[q] + so);
        } else {
          const uint32_t h = ld16(xs, xo[q] + so);
          d.x[j][q >> 1] = (q & 1) ? (d.x[j][q >> 1] | (h << 16)) : h;
        }
      }
    }
  };

  auto run_tile = [&](const MfTile<RT, KM>& d) {
    // transpose the tile's x block: row b of the LDS tile = batch column b
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t v = (d.x[j][i >> 1] >> (16 * (i & 1))) & 0xffffu;
        *(lds_u16*)(uintptr_t)(xt + (uint32_t)((bh * 8 + i) * kXtRow + j * 32 + nl) * 2u) = (uint16_t)v;
      }
    wave_sync();
    // k group g of MFMA j: columns 32 g + 8 j .. + 7 of the tile
    const uint32_t brow = xt + (uint32_t)(r16 * kXtRow + g * 32) * 2u;
    const uint4 bv0 = lds_u4(brow), bv1 = lds_u4(brow + 16u), bv2 = lds_u4(brow + 32u), bv3 = lds_u4(brow + 48u);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        const uint32_t w = d.w[rt][k];
        acc[rt][k] = mfma_step<XT>(a_operand<0>(w, msk), bv0, acc[rt][k]);
        acc[rt][k] = mfma_step<XT>(a_operand<1>(w, msk), bv1, acc[rt][k]);
        acc[rt][k] = mfma_step<XT>(a_operand<2>(w, msk), bv2, acc[rt][k]);
        acc[rt][k] = mfma_step<XT>(a_operand<3>(w, msk), bv3, acc[rt][k]);
      }
    wave_sync();  // the next tile's transpose overwrites the LDS tile
  };

  // tiles [tb, tb + NT) of this wavefront, two register sets in turn (no
  // copies between them: a copy would wait for the loads)
  const int NT = a.NCH >> 2;
  const int tb = wv * NT;
  MfTile<RT, KM> ta, tc;
  load_tile(tb, ta);
  int t = 0;
  for (; t + 2 <= NT; t += 2) {
    load_tile(tb + t + 1, tc);
    run_tile(ta);
    load_tile(tb + min(t + 2, NT - 1), ta);  // past the last tile: re-read it (a cache hit)
    run_tile(tc);
  }
  if (t < NT) run_tile(ta);

  // row scales: lane holds C rows 4 g + i, batch column r16, of each row tile
  const rsrc_t als = make_rsrc(a.alpha, a.al_bytes);
  float* red = (float*)(lds + (size_t)W * kXtBytes);  // [W][RT][16 rows][16 cols]
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + rt * 16 + 4 * g + i;
      float v = 0.0f;
#pragma unroll
      for (int k = 0; k < KM; ++k)
        v += (a.alpha ? __uint_as_float(ld32(als, (uint32_t)(k * a.M + m) * 4u)) : 1.0f) * acc[rt][k][i];
      red[((wv * RT + rt) * 16 + 4 * g + i) * 16 + r16] = -0.5f * v;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < RT * 256; e += blockDim.x) {
    const int rt = e >> 8, row = (e >> 4) & 15, col = e & 15;
    const int m = m0 + rt * 16 + row, b = a.b0 + col;
    if (m < a.M && b < a.B) {
      const float sum = sum_waves(red + (rt * 16 + row) * 16 + col, RT * 256, W);
      const size_t yi = (size_t)m * a.B + b;
      a.y[yi] = (a.accumulate ? a.y[yi] : 0.0f) + sum;
    }
  }
}

// ------------------------------------------------------------------ planning

bool mfma_eligible(int B, int xdt, bool colscale) {
  return B >= 4 && !colscale && (xdt == BSG_BF16 || xdt == BSG_F16);
}

static hipError_t dispatch_mfma(const ProdArgs& a, int RT, int KM, int XT, int VW, int nwg, int W, size_t lds,
                                hipStream_t st) {
  const int key = ((RT * 8 + KM) * 4 + XT) * 16 + VW;
  ProdPlan p{};
  p.nwg = nwg;
  p.W = W;
  p.lds = lds;
  if (a.np > 1) {
    switch (key) {
#define BSG_MF(RT_, KM_, XT_, VW_) \
  case ((RT_ * 8 + KM_) * 4 + XT_) * 16 + VW_: return launch_one(k_prod_mfma<RT_, KM_, XT_, VW_, 1>, p, a, st);
#define BSG_MF_VW(RT_, KM_, XT_) BSG_MF(RT_, KM_, XT_, 4) BSG_MF(RT_, KM_, XT_, 8)
#define BSG_MF_XT(RT_, KM_) BSG_MF_VW(RT_, KM_, 1) BSG_MF_VW(RT_, KM_, 2)
      BSG_MF_XT(1, 1) BSG_MF_XT(1, 2) BSG_MF_XT(1, 3) BSG_MF_XT(1, 4)
      BSG_MF_XT(2, 1) BSG_MF_XT(2, 2) BSG_MF_XT(2, 3) BSG_MF_XT(2, 4)
#undef BSG_MF_XT
#undef BSG_MF_VW
#undef BSG_MF
      default: return hipErrorInvalidConfiguration;
    }
  }
  switch (key) {
#define BSG_MF(RT_, KM_, XT_, VW_) \
  case ((RT_ * 8 + KM_) * 4 + XT_) * 16 + VW_: return launch_one(k_prod_mfma<RT_, KM_, XT_, VW_, 0>, p, a, st);
#define BSG_MF_VW(RT_, KM_, XT_) BSG_MF(RT_, KM_, XT_, 2) BSG_MF(RT_, KM_, XT_, 4) BSG_MF(RT_, KM_, XT_, 8)
#define BSG_MF_XT(RT_, KM_) BSG_MF_VW(RT_, KM_, 1) BSG_MF_VW(RT_, KM_, 2)
    BSG_MF_XT(1, 1) BSG_MF_XT(1, 2) BSG_MF_XT(1, 3) BSG_MF_XT(1, 4)
    BSG_MF_XT(2, 1) BSG_MF_XT(2, 2) BSG_MF_XT(2, 3) BSG_MF_XT(2, 4)
    // 2-byte x loads (odd B or x not 4-byte aligned): one row tile, at most
    // two bases a launch (the loads in flight take the registers)
    BSG_MF(1, 1, 1, 1) BSG_MF(1, 2, 1, 1) BSG_MF(1, 1, 2, 1) BSG_MF(1, 2, 2, 1)
#undef BSG_MF_XT
#undef BSG_MF_VW
#undef BSG_MF
    default: return hipErrorInvalidConfiguration;
  }
}

static int mf_env(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  const int r = std::atoi(v);
  return r > 0 ? r : dflt;
}

// x load width for this batch width and x address
static int mfma_vw(int B, const void* x) {
  const uintptr_t xa = (uintptr_t)x;
  return (B % 8 == 0 && xa % 16 == 0) ? 8 : (B % 4 == 0 && xa % 8 == 0) ? 4 : (B % 2 == 0 && xa % 4 == 0) ? 2 : 1;
}

bool mfma_multi_ok(int B, const void* x) { return mfma_vw(B, x) >= 4; }

// One launch per 16 batch columns and per group of up to 4 bases (2 with
// 2-byte x loads; later groups accumulate).  Row tiles per workgroup: 2 when
// that still gives at least 256 workgroups (x is then read once per 32
// rows), else 1.  Wavefronts: up to mfma_max_waves, each taking whole
// 4-step layout tiles.  With a0.np > 1 every launch covers the row tiles of
// all projections a0.proj[0 .. np) in turn (4- or 8-value x loads only).
hipError_t launch_prod_mfma(const ProdArgs& a0, hipStream_t st) {
  const int T4 = (a0.ND + 3) / 4;      // 4-step layout tiles
  const int XT = a0.xdt == BSG_BF16 ? 1 : 2;
  const int VW = mfma_vw(a0.B, a0.x);
  const bool multi = a0.np > 1;
  if (multi && VW < 4) return hipErrorInvalidConfiguration;
  int mt = a0.M;
  if (multi) {
    mt = 0;
    for (int i = 0; i < a0.np; ++i) mt += a0.proj[i].M;
  }
  const int RT = VW == 1 ? 1 : mf_env("BSG_MF_RT", (mt + 31) / 32 >= 256 ? 2 : 1) >= 2 ? 2 : 1;
  const int KG = VW == 1 ? 2 : 4;      // bases per launch
  int nwg = (a0.M + 16 * RT - 1) / (16 * RT);
  if (multi) {
    nwg = 0;
    for (int i = 0; i < a0.np; ++i) nwg += (a0.proj[i].M + 16 * RT - 1) / (16 * RT);
  }
  for (int k0 = 0; k0 < a0.K; k0 += KG) {
    const int KM = a0.K - k0 < KG ? a0.K - k0 : KG;
    const int wmax = std::min(mfma_max_waves(RT, KM, VW), mf_env("BSG_MF_W", 16));
    int W = T4 < wmax ? T4 : wmax;
    const int per = (T4 + W - 1) / W;  // tiles per wavefront
    W = (T4 + per - 1) / per;
    const size_t lds = (size_t)W * kXtBytes + (size_t)W * RT * 256 * 4;
    ProdArgs as = a0;
    as.bits = a0.bits + (size_t)k0 * a0.plane;
    as.alpha = a0.alpha ? a0.alpha + (size_t)k0 * a0.M : nullptr;
    as.K = KM;
    as.accumulate = k0 > 0 ? 1 : a0.accumulate;
    as.x_bytes = (uint32_t)((size_t)a0.N * a0.B * 2);
    as.cs_bytes = 0;
    as.al_bytes = a0.alpha ? (uint32_t)((size_t)KM * a0.M * 4) : 0u;
    as.W = W;
    as.NCH = per * 4;  // steps per wavefront
    if (multi) {
      int wg = 0;
      for (int i = 0; i < a0.np; ++i) {
        const ProjDesc& s0 = a0.proj[i];
        ProjDesc& d = as.proj[i];
        d.plane = plane_words(s0.M, a0.ND);
        d.bits = s0.bits + (size_t)k0 * d.plane;
        d.alpha = s0.alpha + (size_t)k0 * s0.M;
        d.al_bytes = (uint32_t)((size_t)KM * s0.M * 4);
        d.wg0 = wg;
        wg += (s0.M + 16 * RT - 1) / (16 * RT);
      }
    }
    for (int b0 = 0; b0 < a0.B; b0 += 16) {
      ProdArgs a = as;
      a.b0 = b0;
      const hipError_t e = dispatch_mfma(a, RT, KM, XT, VW, nwg, W, lds, st);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace bsg
