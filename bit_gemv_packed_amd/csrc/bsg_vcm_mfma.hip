// Salient-column bases of the hybrid format on the matrix cores, for B >= 4
// columns of fp16 x (FluxBin Sec. 3.1 hybrid bases; Sec. 3.2 Virtual
// Columnar Mapping: the sparse salient columns are a dense physical matrix,
// read through an index list that gathers x and the scales):
//
//   y[m,b] += sum_k sum_j salpha_k[m][j] sum_{i < s} (2 sbit_k(m, js+i) - 1) sc_k[js+i] x[idx[js+i], b]
//
// It runs after the main product (which it accumulates onto), one launch per
// 16 batch columns.  A workgroup owns 16 or 32 rows.  Its prologue gathers
// x at the S salient columns for the launch's 16 batch columns into LDS,
// already transposed for the B operand ([batch column][S + 8 pad]), and the
// salient column scales [base][S]; every wavefront helps, with 8- or
// 16-byte loads of a row of x.  The wavefronts then split the 128-column
// tiles of the physical matrix.  The group row scale varies along the
// contraction (a group is s = 8, 16 or 32 physical columns, so one MFMA of
// 8 columns per lane lies in one group), so it is folded into the A values:
// A = +-fp16(c * salpha), the sign flipped for a set weight bit.  That
// product is the one rounding beyond fp32 sums (2^-11 relative per term).
#include <algorithm>

#include "bsg_prod_mfma.h"

namespace bsg {

typedef __attribute__((ext_vector_type(2))) _Float16 h2;

// A operand of MFMA J of a tile: the 8 columns of byte J of sign word w.
// The lane's GPW group scales (al, two per 32-bit value) hold the scale of
// these columns in slot J * GPW / 4; with column scales (CS) each value is
// fp16(c * scale), else the scale itself.
template <int J, int GPW, int CS>
__device__ inline uint4 a_operand_vcm(uint32_t w, uint32_t msk, uint4 c8, uint2 al) {
  constexpr int slot = J * GPW / 4;
  const uint32_t half = slot < 2 ? al.x : al.y;
  const uint32_t hb = (slot & 1) ? (half >> 16) : (half & 0xffffu);
  const uint32_t a2 = hb | (hb << 16);
  const u16x2 t = __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(0u, w, 0x0c000c00u | (J << 16) | J));
  const uint32_t c[4] = {c8.x, c8.y, c8.z, c8.w};
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u16x2 sh = t << u16x2{(unsigned short)(15 - 2 * i), (unsigned short)(14 - 2 * i)};
    const uint32_t v =
        CS ? __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, c[i]) * __builtin_bit_cast(h2, a2)) : a2;
    d[i] = v ^ (__builtin_bit_cast(uint32_t, sh) & msk);
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

// VW: batch values per x load in the gather (8: B % 8 == 0 and x 16-byte
// aligned; 4: B % 4 == 0 and x 8-byte aligned).
template <int RT, int KM, int GPW, int CS, int VW>
__global__ void __launch_bounds__(1024) k_vcm_mfma(ProdArgs a) {
  extern __shared__ __align__(16) char lds[];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const uint32_t blk = blockIdx.x;
  const int m0 = (int)(blk * 16 * RT);
  const int S = a.vs_S, nds = a.vs_nd;
  const int T4 = (nds + 3) / 4;  // 128-column tiles of the physical matrix
  const int SP = T4 * 128;       // columns with the padding of the last tile
  const int XR = SP + 8;         // halves per batch row of the LDS copy of x
  const uint32_t xb = (uint32_t)(uintptr_t)lds;
  const uint32_t cb = xb + (uint32_t)(16 * XR) * 2u;
  float* red = (float*)(lds + (size_t)16 * XR * 2 + (CS ? (size_t)KM * SP * 2 : 0));  // [W][RT][16][16]
  uint32_t msk;
  asm volatile("s_mov_b32 %0, 0x80008000" : "=s"(msk));

  // ---- gather (all wavefronts): x[idx[p]][b0 .. b0 + 15] -> LDS [b][p],
  // 0 for padding columns, indices outside [0, N) and batch columns >= B
  const rsrc_t xs = make_rsrc(a.x, a.x_bytes);
  const rsrc_t ir = make_rsrc(a.vs_idx, (size_t)S * 4);
  constexpr int NQ = 16 / VW;  // loads per column
  for (int e = threadIdx.x; e < SP * NQ; e += blockDim.x) {
    const int p = e / NQ, q = e % NQ;
    const uint32_t n = ld32(ir, (uint32_t)p * 4u);
    const int b = a.b0 + q * VW;
    const bool ok = p < S && n < (uint32_t)a.N && b < a.B;
    const uint32_t off = ok ? (n * (uint32_t)a.B + (uint32_t)b) * 2u : 0xffffffe0u;
    uint32_t v[VW / 2];
    if (VW == 8) {
      const uint4 t = ld128(xs, off);
      v[0] = t.x;
      v[1] = t.y;
      v[VW / 2 > 2 ? 2 : 0] = t.z;
      v[VW / 2 > 3 ? 3 : 0] = t.w;
    } else {
      const uint2 t = ld64(xs, off);
      v[0] = t.x;
      v[1] = t.y;
    }
#pragma unroll
    for (int i = 0; i < VW; ++i)
      *(lds_u16*)(uintptr_t)(xb + (uint32_t)((q * VW + i) * XR + p) * 2u) = (uint16_t)(v[i >> 1] >> (16 * (i & 1)));
  }
  if (CS) {
    const rsrc_t csr = make_rsrc(a.vs_cs, (size_t)a.K * S * 2);
    for (int e = threadIdx.x; e < KM * SP; e += blockDim.x) {
      const int k = e / SP, p = e % SP;
      const uint32_t h = p < S ? ld16(csr, (uint32_t)(k * S + p) * 2u) : 0u;
      *(lds_u16*)(uintptr_t)(cb + (uint32_t)e * 2u) = (uint16_t)h;
    }
  }
  __syncthreads();

  // ---- the wavefront's tiles
  SignRows<KM> sr[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
    sr[rt] = sign_rows<KM, 16 * RT>(a.vs_bits, a.vs_plane, a.K, nds, blk, m0 + rt * 16 + r16);
  const rsrc_t sar = make_rsrc(a.vs_alpha, (size_t)a.K * nds * a.M * GPW * 2);
  f32x4 acc[RT][KM];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int k = 0; k < KM; ++k) acc[rt][k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int t = wv; t < T4; t += W) {
    uint32_t wd[RT][KM];
    uint2 al[RT][KM];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        wd[rt][k] = ld32(sr[rt].r[k], (uint32_t)t * 1024u + sr[rt].row_off + (uint32_t)g * 4u);
        const uint32_t off = (uint32_t)(((k * nds + 4 * t + g) * a.M + m0 + rt * 16 + r16) * GPW) * 2u;
        al[rt][k] = GPW == 4 ? ld64(sar, off) : make_uint2(GPW == 2 ? ld32(sar, off) : ld16(sar, off), 0u);
      }
    // k group g of MFMA j: physical columns 128 t + 32 g + 8 j .. + 7
    const uint32_t brow = xb + (uint32_t)(r16 * XR + t * 128 + g * 32) * 2u;
    const uint4 bv0 = lds_u4(brow), bv1 = lds_u4(brow + 16u), bv2 = lds_u4(brow + 32u), bv3 = lds_u4(brow + 48u);
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      uint4 c8[4] = {};
      if (CS) {
        const uint32_t crow = cb + (uint32_t)(k * SP + t * 128 + g * 32) * 2u;
#pragma unroll
        for (int j = 0; j < 4; ++j) c8[j] = lds_u4(crow + 16u * j);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const uint32_t w = wd[rt][k];
        const uint2 s2 = al[rt][k];
        acc[rt][k] = mfma_step<2>(a_operand_vcm<0, GPW, CS>(w, msk, c8[0], s2), bv0, acc[rt][k]);
        acc[rt][k] = mfma_step<2>(a_operand_vcm<1, GPW, CS>(w, msk, c8[1], s2), bv1, acc[rt][k]);
        acc[rt][k] = mfma_step<2>(a_operand_vcm<2, GPW, CS>(w, msk, c8[2], s2), bv2, acc[rt][k]);
        acc[rt][k] = mfma_step<2>(a_operand_vcm<3, GPW, CS>(w, msk, c8[3], s2), bv3, acc[rt][k]);
      }
    }
  }

  // ---- the W partial tiles in a fixed order, added onto y (A = -c s for +1)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.0f;
#pragma unroll
      for (int k = 0; k < KM; ++k) v += acc[rt][k][i];
      red[((wv * RT + rt) * 16 + 4 * g + i) * 16 + r16] = -v;
    }
  __syncthreads();
  for (int e = threadIdx.x; e < RT * 256; e += blockDim.x) {
    const int rt = e >> 8, row = (e >> 4) & 15, col = e & 15;
    const int m = m0 + rt * 16 + row, b = a.b0 + col;
    if (m < a.M && b < a.B) {
      const float sum = sum_waves(red + (rt * 16 + row) * 16 + col, RT * 256, W);
      a.y[(size_t)m * a.B + b] += sum;
    }
  }
}

// LDS of one workgroup of W wavefronts and RT row tiles
static size_t vcm_lds(int S, int K, bool cs, int W, int RT) {
  const int T4 = ((S + 31) / 32 + 3) / 4, SP = T4 * 128;
  return (size_t)16 * (SP + 8) * 2 + (cs ? (size_t)K * SP * 2 : 0) + (size_t)W * RT * 256 * 4;
}

bool vcm_mfma_ok(int B, int xdt, const void* x, int K, int S, bool cs) {
  const uintptr_t xa = (uintptr_t)x;
  const bool vw = (B % 8 == 0 && xa % 16 == 0) || (B % 4 == 0 && xa % 8 == 0);
  return B >= 4 && xdt == BSG_F16 && vw && K >= 1 && K <= 4 && vcm_lds(S, K, cs, 16, 2) <= kMaxLds;
}

hipError_t launch_vcm_mfma(const ProdArgs& a0, hipStream_t st) {
  const int RT = (a0.M + 31) / 32 >= 256 ? 2 : 1;
  const bool cs = a0.vs_cs != nullptr;
  const int VW = (a0.B % 8 == 0 && (uintptr_t)a0.x % 16 == 0) ? 8 : 4;
  ProdPlan p{};
  p.nwg = (a0.M + 16 * RT - 1) / (16 * RT);
  p.W = 16;
  p.lds = vcm_lds(a0.vs_S, a0.K, cs, p.W, RT);
  if (p.lds > kMaxLds) return hipErrorInvalidConfiguration;
  ProdArgs as = a0;
  as.x_bytes = (uint32_t)((size_t)a0.N * a0.B * 2);
  const int key = (((RT * 8 + a0.K) * 8 + a0.vs_gpw) * 2 + (cs ? 1 : 0)) * 16 + VW;
  for (int b0 = 0; b0 < a0.B; b0 += 16) {
    ProdArgs a = as;
    a.b0 = b0;
    hipError_t e;
    switch (key) {
#define BSG_VCM(RT_, KM_, GPW_, CS_, VW_)                              \
  case (((RT_ * 8 + KM_) * 8 + GPW_) * 2 + CS_) * 16 + VW_:            \
    e = launch_one(k_vcm_mfma<RT_, KM_, GPW_, CS_, VW_>, p, a, st); \
    break;
#define BSG_VCM_VW(RT_, KM_, GPW_, CS_) BSG_VCM(RT_, KM_, GPW_, CS_, 4) BSG_VCM(RT_, KM_, GPW_, CS_, 8)
#define BSG_VCM_CS(RT_, KM_, GPW_) BSG_VCM_VW(RT_, KM_, GPW_, 0) BSG_VCM_VW(RT_, KM_, GPW_, 1)
#define BSG_VCM_G(RT_, KM_) BSG_VCM_CS(RT_, KM_, 1) BSG_VCM_CS(RT_, KM_, 2) BSG_VCM_CS(RT_, KM_, 4)
#define BSG_VCM_K(RT_) BSG_VCM_G(RT_, 1) BSG_VCM_G(RT_, 2) BSG_VCM_G(RT_, 3) BSG_VCM_G(RT_, 4)
      BSG_VCM_K(1) BSG_VCM_K(2)
#undef BSG_VCM_K
#undef BSG_VCM_G
#undef BSG_VCM_CS
#undef BSG_VCM_VW
#undef BSG_VCM
      default: return hipErrorInvalidConfiguration;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bsg
