// Batched sign product on the matrix cores (gfx950), for B >= 4 batch
// columns of bf16 or fp16 activations, included by bsg_gemv_mfma.hip (per-row
// scales) and bsg_gemv_mfma_cg.hip (column scales, group-wise row scales):
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
//
// CG bit 0: fp16 column scales with fp16 x (FluxBin Sec. 3.1 decoupled
// scales).  The A values become +-c_k[n] instead of +-2: the column scale's
// own fp16 bits with the sign bit flipped for a set weight bit (one XOR in
// place of the OR), so the products with fp16 x stay exact; the scales of a
// tile's 128 columns are staged through the wavefront's LDS (4 bytes per
// lane per base) and read back 16 bytes per MFMA, like x.  CG bit 1:
// group-wise fp16 row scales (groups of g >= 128 columns, so a 128-column
// tile lies in one group): each tile's four MFMAs go to a fresh accumulator
// that is added times the group scales of the lane's four rows.
#pragma once
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
typedef __attribute__((address_space(3))) uint32_t lds_u32;

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

// A operand with column scales: the 8 fp16 scales of byte J's columns (cv,
// two per word, in column order) with the sign bit flipped where the weight
// bit is set: -c for a set bit, +c for a clear one.
template <int J>
__device__ inline uint4 a_operand_cs(uint32_t w, uint32_t msk, uint4 cv) {
  const u16x2 t = __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(0u, w, 0x0c000c00u | (J << 16) | J));
  const uint32_t c[4] = {cv.x, cv.y, cv.z, cv.w};
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u16x2 sh = t << u16x2{(unsigned short)(15 - 2 * i), (unsigned short)(14 - 2 * i)};
    d[i] = (__builtin_bit_cast(uint32_t, sh) & msk) ^ c[i];
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

constexpr int kXtRow = 136;                      // halves per batch row of a tile (128 + 8 pad)
constexpr uint32_t kXtBytes = 16 * kXtRow * 2;   // one 4-step tile of x in LDS

// Most wavefronts per workgroup: 16, or 8 where the accumulators, sign words
// and x loads in flight need more than 128 VGPRs (RT * KM >= 4; 2-byte
// loads: 32 per tile; 4-byte loads with RT * KM = 3; scales with
// RT * KM >= 3): up to 256, no spills.
constexpr int mfma_max_waves(int RT, int KM, int VW, int CG = 0) {
  return (RT * KM >= 4 || VW == 1 || (VW == 2 && RT * KM >= 3) || (CG && RT * KM >= 3)) ? 8 : 16;
}
// LDS bytes of one wavefront: its x tile, and with column scales its tile's
// scales (128 fp16 per base)
constexpr uint32_t mfma_wave_lds(int KM, int CG) { return kXtBytes + ((CG & 1) ? (uint32_t)KM * 256u : 0u); }

template <int RT, int KM, int CG = 0>
struct MfTile {
  uint32_t w[RT][KM];  // word g of the lane's row, per row tile and base
  uint32_t x[4][4];    // per step: 8 batch values of column 32 step + lane % 32
  uint32_t c[(CG & 1) ? KM : 1];             // column scales of columns 2 lane, 2 lane + 1 of the tile
  uint2 s[(CG & 2) ? RT : 1][(CG & 2) ? KM : 1];  // group scales of the lane's 4 rows
};

// XT: 1 bf16, 2 fp16 activations.  VW: batch values per x load (8, 4, 2 or
// 1: B % VW == 0 and x aligned to 2 VW bytes).  MP = 1: the fused launch of
// several projections (bs_gemv_multi).  CG: column scales (bit 0, fp16 x)
// and group-wise row scales (bit 1), as above.  EX bit 0: the tiles again
// with a.x2 in place of x, summed into the same result (the two
// bf16 halves of the low-rank expansion's activations); EX bit 1: instead of
// y, write the bf16 halves hi = bf16(w), lo = bf16(w - hi) of w = s[m] * y
// (s = a.split_scale fp16, outputs a.split_hi / a.split_lo, [M][B]).
template <int RT, int KM, int XT, int VW, int MP, int CG = 0, int EX = 0>
__global__ void __launch_bounds__(64 * mfma_max_waves(RT, KM, VW, CG)) k_prod_mfma(ProdArgs a) {
  asm volatile("" ::"s"(a.bits), "s"(a.alpha), "s"(a.x), "s"(a.y), "s"(a.plane), "s"(a.K), "s"(a.M), "s"(a.N),
               "s"(a.ND), "s"(a.B), "s"(a.b0), "s"(a.accumulate), "s"(a.NCH), "s"(a.x_bytes), "s"(a.al_bytes));
  static_assert(!(CG & 1) || XT == 2, "column scales need fp16 activations");
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
  const uint32_t xt = (uint32_t)(uintptr_t)lds + (uint32_t)wv * mfma_wave_lds(KM, CG);
  const uint32_t cb = xt + kXtBytes;  // column scales of the tile (CG bit 0): [base][128]
  uint32_t msk;
  asm volatile("s_mov_b32 %0, 0x80008000" : "=s"(msk));

  SignRows<KM> sr[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) sr[rt] = sign_rows<KM, 16 * RT>(a.bits, a.plane, a.K, a.ND, blk, m0 + rt * 16 + r16);
  const rsrc_t xs = make_rsrc(a.x, a.x_bytes);
  const rsrc_t csr = make_rsrc(a.colscale, (CG & 1) ? a.cs_bytes : 0);
  const rsrc_t gsr = make_rsrc(a.alpha, (CG & 2) ? a.al_bytes : 0);

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

  auto load_tile = [&](int t, MfTile<RT, KM, CG>& d, const rsrc_t& xr) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int k = 0; k < KM; ++k) d.w[rt][k] = ld32(sr[rt].r[k], (uint32_t)t * 1024u + sr[rt].row_off + (uint32_t)g * 4u);
    if (CG & 1) {
#pragma unroll
      for (int k = 0; k < KM; ++k) d.c[(CG & 1) ? k : 0] = ld32(csr, (uint32_t)(k * a.N + t * 128 + 2 * lane) * 2u);
    }
    if (CG & 2) {
      const int j = 4 * t / a.gsw;  // the tile's group (a.gsw >= 4 words)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int k = 0; k < KM; ++k)
          d.s[(CG & 2) ? rt : 0][(CG & 2) ? k : 0] =
              ld64(gsr, (uint32_t)((k * a.ngrp + j) * a.M + m0 + rt * 16 + 4 * g) * 2u);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t so = (uint32_t)(4 * t + j) * xstep;
#pragma unroll
      for (int q = 0; q < NL; ++q) {
        if (VW == 8) {
          const uint4 v = ld128(xr, xo[q] + so);
          d.x[j][0] = v.x;
          d.x[j][1] = v.y;
          d.x[j][2] = v.z;
          d.x[j][3] = v.w;
        } else if (VW == 4) {
          const uint2 v = ld64(xr, xo[q] + so);
          d.x[j][2 * q] = v.x;
          d.x[j][2 * q + 1] = v.y;
        } else if (VW == 2) {
          d.x[j][q] = ld32(xr, xo[q] + so);
        } else {
          const uint32_t h = ld16(xr, xo[q] + so);
          d.x[j][q >> 1] = (q & 1) ? (d.x[j][q >> 1] | (h << 16)) : h;
        }
      }
    }
  };

  auto run_tile = [&](const MfTile<RT, KM, CG>& d) {
    // transpose the tile's x block: row b of the LDS tile = batch column b
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t v = (d.x[j][i >> 1] >> (16 * (i & 1))) & 0xffffu;
        *(lds_u16*)(uintptr_t)(xt + (uint32_t)((bh * 8 + i) * kXtRow + j * 32 + nl) * 2u) = (uint16_t)v;
      }
    if (CG & 1) {
#pragma unroll
      for (int k = 0; k < KM; ++k) *(lds_u32*)(uintptr_t)(cb + (uint32_t)k * 256u + (uint32_t)lane * 4u) = d.c[(CG & 1) ? k : 0];
    }
    wave_sync();
    // k group g of MFMA j: columns 32 g + 8 j .. + 7 of the tile
    const uint32_t brow = xt + (uint32_t)(r16 * kXtRow + g * 32) * 2u;
    const uint4 bv0 = lds_u4(brow), bv1 = lds_u4(brow + 16u), bv2 = lds_u4(brow + 32u), bv3 = lds_u4(brow + 48u);
    if constexpr (CG == 0) {
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
    } else {
    // one base's column scales at a time (16 registers), shared by its row tiles
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      uint4 cv[4];
      if (CG & 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) cv[j] = lds_u4(cb + (uint32_t)k * 256u + (uint32_t)(32 * g + 8 * j) * 2u);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const uint32_t w = d.w[rt][k];
        f32x4 c4 = (CG & 2) ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[rt][k];
        if (CG & 1) {
          c4 = mfma_step<XT>(a_operand_cs<0>(w, msk, cv[0]), bv0, c4);
          c4 = mfma_step<XT>(a_operand_cs<1>(w, msk, cv[1]), bv1, c4);
          c4 = mfma_step<XT>(a_operand_cs<2>(w, msk, cv[2]), bv2, c4);
          c4 = mfma_step<XT>(a_operand_cs<3>(w, msk, cv[3]), bv3, c4);
        } else {
          c4 = mfma_step<XT>(a_operand<0>(w, msk), bv0, c4);
          c4 = mfma_step<XT>(a_operand<1>(w, msk), bv1, c4);
          c4 = mfma_step<XT>(a_operand<2>(w, msk), bv2, c4);
          c4 = mfma_step<XT>(a_operand<3>(w, msk), bv3, c4);
        }
        if (CG & 2) {
          const uint2 sv = d.s[(CG & 2) ? rt : 0][(CG & 2) ? k : 0];
          acc[rt][k][0] += f16_bits_to_float((uint16_t)(sv.x & 0xffffu)) * c4[0];
          acc[rt][k][1] += f16_bits_to_float((uint16_t)(sv.x >> 16)) * c4[1];
          acc[rt][k][2] += f16_bits_to_float((uint16_t)(sv.y & 0xffffu)) * c4[2];
          acc[rt][k][3] += f16_bits_to_float((uint16_t)(sv.y >> 16)) * c4[3];
        } else {
          acc[rt][k] = c4;
        }
      }
    }
    }
    wave_sync();  // the next tile's transpose overwrites the LDS tile
  };

  // tiles [tb, tb + NT) of this wavefront, two register sets in turn (no
  // copies between them: a copy would wait for the loads)
  const int NT = a.NCH >> 2;
  const int tb = wv * NT;
  MfTile<RT, KM, CG> ta, tc;
  if constexpr ((EX & 1) == 0) {
    load_tile(tb, ta, xs);
    int t = 0;
    for (; t + 2 <= NT; t += 2) {
      load_tile(tb + t + 1, tc, xs);
      run_tile(ta);
      load_tile(tb + min(t + 2, NT - 1), ta, xs);  // past the last tile: re-read it (a cache hit)
      run_tile(tc);
    }
    if (t < NT) run_tile(ta);
  } else {
    // 2 NT steps: the tiles with x, then the same sign tiles again with x2,
    // summed into the same accumulators
    const rsrc_t xs2 = make_rsrc(a.x2, a.x_bytes);
    auto load_v = [&](int v, MfTile<RT, KM, CG>& d) {
      const bool second = v >= NT;
      load_tile(tb + (second ? v - NT : v), d, second ? xs2 : xs);
    };
    const int NV = 2 * NT;
    load_v(0, ta);
    int v = 0;
    for (; v + 2 <= NV; v += 2) {
      load_v(v + 1, tc);
      run_tile(ta);
      load_v(min(v + 2, NV - 1), ta);
      run_tile(tc);
    }
    if (v < NV) run_tile(ta);
  }

  // row scales: lane holds C rows 4 g + i, batch column r16, of each row tile
  const rsrc_t als = make_rsrc(a.alpha, a.al_bytes);
  float* red = (float*)(lds + (size_t)W * mfma_wave_lds(KM, CG));  // [W][RT][16 rows][16 cols]
  // -1/2 undoes the +-2 of the A values; with column scales they are +-c
  constexpr float kOutScale = (CG & 1) ? -1.0f : -0.5f;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + rt * 16 + 4 * g + i;
      float v = 0.0f;
#pragma unroll
      for (int k = 0; k < KM; ++k)
        v += ((CG & 2) || !a.alpha ? 1.0f : __uint_as_float(ld32(als, (uint32_t)(k * a.M + m) * 4u))) * acc[rt][k][i];
      red[((wv * RT + rt) * 16 + 4 * g + i) * 16 + r16] = kOutScale * v;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < RT * 256; e += blockDim.x) {
    const int rt = e >> 8, row = (e >> 4) & 15, col = e & 15;
    const int m = m0 + rt * 16 + row, b = a.b0 + col;
    if (m < a.M && b < a.B) {
      const float sum = sum_waves(red + (rt * 16 + row) * 16 + col, RT * 256, W);
      const size_t yi = (size_t)m * a.B + b;
      if (EX & 2) {
        const float w = sum * f16_bits_to_float(a.split_scale[m]);
        const __bf16 hi = (__bf16)w;
        const __bf16 lo = (__bf16)(w - (float)hi);
        __builtin_memcpy(a.split_hi + yi, &hi, 2);
        __builtin_memcpy(a.split_lo + yi, &lo, 2);
      } else {
        a.y[yi] = (a.accumulate ? a.y[yi] : 0.0f) + sum;
      }
    }
  }
}

}  // namespace bsg
