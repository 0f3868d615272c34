// Batched sign product on the matrix cores (gfx950), for B >= 4 batch
// columns of bf16 or fp16 activations without column scales:
//
//   y[m,b] (= or +=) sum_k alpha_k[m] sum_n (2 bit_k(m,n) - 1) x[n,b]
//
// With several batch columns the product is a dense contraction, so it runs
// as v_mfma_f32_16x16x32_{bf16,f16}: A = 16 rows x 32 columns of +-1 signs,
// B = 32 columns x 16 batch columns of x, C = fp32 16 x 16.  Signs are
// exact in bf16 / fp16 and so are their products with x; the sums are fp32.
//
// A operand.  Lane l holds row l % 16 and 8 consecutive columns of the step,
// (l / 16) * 8 .. + 7: one byte of the row's sign word.  A 256-entry LDS
// table maps a byte to its 8 signs (16 bytes), so a lane gets its operand
// with one LDS read.
//
// B operand.  Lane l holds batch column l % 16 and the same 8 columns.  x is
// stored [N][B] (a batch row per column), so each wavefront transposes the
// 32 x 16 block of its step through a small LDS tile (8 two-byte writes and
// one 16-byte read per lane).  The product is linear in x, and the k order
// of A and B is the same, so any consistent split of the 32 columns works.
//
// Work decomposition.  A workgroup owns RT tiles of 16 complete rows (16 RT
// divides 64: all in one row block of the sign layout); its W wavefronts
// split the 32-column steps (NKS each, a multiple of 4 so that every
// wavefront starts at a 4-word layout tile: one 16-byte load per lane
// covers 4 steps of a row).  The W partial C tiles are summed through LDS in
// a fixed order: no atomics, deterministic.  Steps beyond N read zero sign
// words / zero x and add nothing.
#include "bsg_prod.h"

namespace bsg {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

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

constexpr uint32_t kLutBytes = 256 * 16;  // byte -> 8 signs
constexpr int kXtRow = 40;                // halves per batch row of a wavefront's x tile (32 + 8 pad)
constexpr uint32_t kXtBytes = 16 * kXtRow * 2;

// Most wavefronts per workgroup: 16, or 8 with RT * KM >= 4 accumulator and
// sign-word sets (up to 256 VGPRs, no spills).
constexpr int mfma_max_waves(int RT, int KM) { return RT * KM >= 4 ? 8 : 16; }

// XT: 1 bf16, 2 fp16 activations.  XV: 1 when B % 8 == 0 and x is 16-byte
// aligned (16-byte loads of 8 batch values), 0 otherwise (2-byte loads).
template <int RT, int KM, int XT, int XV>
__global__ void __launch_bounds__(64 * mfma_max_waves(RT, KM)) k_prod_mfma(ProdArgs a) {
  asm volatile("" ::"s"(a.bits), "s"(a.alpha), "s"(a.x), "s"(a.plane), "s"(a.K), "s"(a.M), "s"(a.N), "s"(a.ND),
               "s"(a.B), "s"(a.b0), "s"(a.NCH), "s"(a.x_bytes), "s"(a.al_bytes));
  extern __shared__ __align__(16) char lds[];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int m0 = blockIdx.x * 16 * RT;
  const uint32_t lut = (uint32_t)(uintptr_t)lds;
  const uint32_t xt = lut + kLutBytes + (uint32_t)wv * kXtBytes;

  // the sign table: entry e, element i = +1 if bit i of e is set, else -1
  {
    const uint32_t one = XT == 1 ? 0x3F80u : 0x3C00u;
    uint32_t* t = (uint32_t*)lds;
    for (int i = threadIdx.x; i < 1024; i += blockDim.x) {
      const int e = i >> 2, p = i & 3;
      const uint32_t lo = one | (((e >> (2 * p)) & 1) ? 0u : 0x8000u);
      const uint32_t hi = one | (((e >> (2 * p + 1)) & 1) ? 0u : 0x8000u);
      t[i] = lo | (hi << 16);
    }
  }
  __syncthreads();  // every wavefront reads the whole table

  SignRows<KM> sr[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) sr[rt] = sign_rows<KM, 16 * RT>(a.bits, a.plane, a.K, a.ND, m0 + rt * 16 + r16);
  const rsrc_t xs = make_rsrc(a.x, a.x_bytes);

  f32x4 acc[RT][KM];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int k = 0; k < KM; ++k) acc[rt][k] = f32x4{0.f, 0.f, 0.f, 0.f};

  // x of one step, for this lane's transpose writes: column n0 + lane % 32,
  // batch columns b0 + 8 (lane / 32) .. + 7
  const int nl = lane & 31, bh = lane >> 5;
  auto load_x = [&](int s, uint32_t (&xv)[4]) {
    const int n = s * 32 + nl;
    if (XV) {
      const uint4 v = ld128(xs, (uint32_t)(n * a.B + a.b0 + bh * 8) * 2u);  // 0 beyond N
      xv[0] = v.x;
      xv[1] = v.y;
      xv[2] = v.z;
      xv[3] = v.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = a.b0 + bh * 8 + 2 * i;
        const uint32_t lo = ld16(xs, (uint32_t)(n * a.B + min(b, a.B - 1)) * 2u);
        const uint32_t hi = ld16(xs, (uint32_t)(n * a.B + min(b + 1, a.B - 1)) * 2u);
        xv[i] = lo | (hi << 16);
      }
    }
    // batch columns beyond B are zero
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = a.b0 + bh * 8 + 2 * i;
      if (b >= a.B) xv[i] = 0u;
      else if (b + 1 >= a.B) xv[i] &= 0xffffu;
    }
  };

  const int s_begin = wv * a.NCH;  // NCH: steps per wavefront, a multiple of 4
  uint32_t xb[2][4];  // x of step j in xb[j % 2] (no register copies: a copy would wait for the load)
  load_x(s_begin, xb[0]);
  uint4 wcur[RT][KM], wnxt[RT][KM];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int k = 0; k < KM; ++k)
      wcur[rt][k] = ld128(sr[rt].r[k], (uint32_t)(s_begin >> 2) * 1024u + sr[rt].row_off);

  for (int s4 = 0; s4 < a.NCH; s4 += 4) {
    const int sb = s_begin + s4;  // first step of this layout tile
    // next tile's sign words (re-reads this tile after the last one: a cache hit)
    const int snext = s4 + 4 < a.NCH ? sb + 4 : sb;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int k = 0; k < KM; ++k)
        wnxt[rt][k] = ld128(sr[rt].r[k], (uint32_t)(snext >> 2) * 1024u + sr[rt].row_off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = sb + j;
      load_x(s4 + j + 1 < a.NCH ? s + 1 : s, xb[(j + 1) & 1]);
      // transpose the step's x block through this wavefront's tile
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t v = (xb[j & 1][i >> 1] >> (16 * (i & 1))) & 0xffffu;
        *(lds_u16*)(uintptr_t)(xt + (uint32_t)((bh * 8 + i) * kXtRow + nl) * 2u) = (uint16_t)v;
      }
      wave_sync();
      const uint4 bop = lds_u4(xt + (uint32_t)(r16 * kXtRow + g * 8) * 2u);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int k = 0; k < KM; ++k) {
          const uint32_t w = j == 0 ? wcur[rt][k].x : j == 1 ? wcur[rt][k].y : j == 2 ? wcur[rt][k].z : wcur[rt][k].w;
          const uint32_t byte = (w >> (8 * g)) & 0xffu;
          acc[rt][k] = mfma_step<XT>(lds_u4(lut + byte * 16u), bop, acc[rt][k]);
        }
      }
      wave_sync();  // the next step's transpose overwrites the tile
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int k = 0; k < KM; ++k) wcur[rt][k] = wnxt[rt][k];
  }

  // row scales: lane holds C rows 4 g + i, batch column r16, of each row tile
  const rsrc_t als = make_rsrc(a.alpha, a.al_bytes);
  float* red = (float*)(lds + kLutBytes + (size_t)W * kXtBytes);  // [W][RT][16 rows][16 cols]
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + rt * 16 + 4 * g + i;
      float t = 0.0f;
#pragma unroll
      for (int k = 0; k < KM; ++k)
        t += (a.alpha ? __uint_as_float(ld32(als, (uint32_t)(k * a.M + m) * 4u)) : 1.0f) * acc[rt][k][i];
      red[((wv * RT + rt) * 16 + 4 * g + i) * 16 + r16] = t;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < RT * 256; t += blockDim.x) {
    const int rt = t >> 8, row = (t >> 4) & 15, col = t & 15;
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

static hipError_t dispatch_mfma(const ProdArgs& a, int RT, int KM, int XT, int XV, int nwg, int W, size_t lds,
                                hipStream_t st) {
  const int key = ((RT * 16 + KM) * 4 + XT) * 2 + XV;
  ProdPlan p{};
  p.nwg = nwg;
  p.W = W;
  p.lds = lds;
  switch (key) {
#define BSG_MF(RT_, KM_, XT_, XV_) \
  case ((RT_ * 16 + KM_) * 4 + XT_) * 2 + XV_: return launch_one(k_prod_mfma<RT_, KM_, XT_, XV_>, p, a, st);
#define BSG_MF_XT(RT_, KM_) BSG_MF(RT_, KM_, 1, 0) BSG_MF(RT_, KM_, 1, 1) BSG_MF(RT_, KM_, 2, 0) BSG_MF(RT_, KM_, 2, 1)
    BSG_MF_XT(1, 1) BSG_MF_XT(1, 2) BSG_MF_XT(1, 3) BSG_MF_XT(1, 4)
    BSG_MF_XT(2, 1) BSG_MF_XT(2, 2) BSG_MF_XT(2, 3) BSG_MF_XT(2, 4)
#undef BSG_MF_XT
#undef BSG_MF
    default: return hipErrorInvalidConfiguration;
  }
}

// One launch per 16 batch columns and per group of up to 4 bases (later
// groups accumulate).  Row tiles per workgroup: 2 when that still gives at
// least 256 workgroups (x is then read once per 32 rows), else 1.
// Wavefronts: up to mfma_max_waves, each taking a multiple of 4 steps.
hipError_t launch_prod_mfma(const ProdArgs& a0, hipStream_t st) {
  const int RT = (a0.M + 31) / 32 >= 256 ? 2 : 1;
  const int NS = a0.ND;                // 32-column steps
  const int T4 = (NS + 3) / 4;         // 4-step layout tiles
  const int XT = a0.xdt == BSG_BF16 ? 1 : 2;
  const int XV = (a0.B % 8 == 0 && (((uintptr_t)a0.x) % 16) == 0) ? 1 : 0;
  const int nwg = (a0.M + 16 * RT - 1) / (16 * RT);
  for (int k0 = 0; k0 < a0.K; k0 += 4) {
    const int KM = a0.K - k0 < 4 ? a0.K - k0 : 4;
    const int wmax = mfma_max_waves(RT, KM);
    int W = T4 < wmax ? T4 : wmax;
    const int per = (T4 + W - 1) / W;  // tiles per wavefront
    W = (T4 + per - 1) / per;
    const size_t lds = kLutBytes + (size_t)W * kXtBytes + (size_t)W * RT * 256 * 4;
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
    for (int b0 = 0; b0 < a0.B; b0 += 16) {
      ProdArgs a = as;
      a.b0 = b0;
      const hipError_t e = dispatch_mfma(a, RT, KM, XT, XV, nwg, W, lds, st);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace bsg
