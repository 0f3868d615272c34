// Binary-base product kernel for gfx950 (float activations), included by
// bsg_gemv.hip (single products, fused projections) and bsg_gemv_gs.hip
// (group-wise row scales):
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
// its own LDS region, so the chunk loop has no workgroup barrier: the
// wavefronts drift apart and one's memory wait overlaps another's lookups
// (the only barrier precedes the final cross-wavefront sum).  Tables are
// laid out [step][quarter][16 entries] with 16 pad bytes
// after each step row: at every lookup the lanes of a quarter read one
// 64-byte table and the Q tables of one instruction occupy disjoint bank
// groups, and the pad staggers the tables that different lanes write at
// once across the banks, so neither reads nor writes conflict.
// Table addresses take one SDWA add per 4-bit slice: the sign word is
// rotated by 2 bits each way and masked once, after which byte j of the
// masked rotation is (slice value) * 4.  Per 32 weights: 2 rotates, 2 masks,
// 8 SDWA adds, 8 LDS reads and 8 fp32 adds.
#pragma once
#include "bsg_prod.h"

#include <cstdlib>
#include <type_traits>

namespace bsg {

// A float at an LDS byte address (the address already includes the base of
// the dynamic LDS block), read with the address in one VGPR.
typedef __attribute__((address_space(3))) const float lds_cf32;
__device__ __forceinline__ float lds_f32(uint32_t addr) { return *(lds_cf32*)(uintptr_t)addr; }

// The activations one sign product multiplies: resources of x [N][B] and
// of the column scales (size 0 when absent: their loads then read 0), and
// the shape.  The main operand is x with the bases' column scales; the fused
// low-rank expansion multiplies z = V x (fp32 [r][B]) with alpha_r as its
// column scales.
struct ActSrc {
  rsrc_t x, c;
  int N, B, b0, xdt;
  bool cs;
};
__device__ __forceinline__ ActSrc act_src(const ProdArgs& a) {
  ActSrc s;
  s.x = make_rsrc(a.x, a.x_bytes);
  s.c = make_rsrc(a.colscale, a.cs_bytes);
  s.N = a.N;
  s.B = a.B;
  s.b0 = a.b0;
  s.xdt = a.xdt;
  s.cs = a.colscale != nullptr;
  return s;
}
__device__ __forceinline__ ActSrc lr_src(const ProdArgs& a) {
  ActSrc s;
  s.x = make_rsrc(a.lr_z, (size_t)a.lr_r * a.B * 4);
  s.c = make_rsrc(a.lr_scale, (size_t)a.lr_r * 2);
  s.N = a.lr_r;
  s.B = a.B;
  s.b0 = a.b0;
  s.xdt = BSG_F32;
  s.cs = true;
  return s;
}

// Raw activation bits -> fp32 (fp32 bits, or a bf16 / fp16 pattern in the low half).
__device__ __forceinline__ float decode_x(uint32_t raw, int xdt) {
  const float h = f16_bits_to_float((uint16_t)raw);
  return xdt == BSG_F32 ? __uint_as_float(raw) : xdt == BSG_BF16 ? __uint_as_float(raw << 16) : h;
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
// 16-byte and column scales 8-byte aligned: one 8-byte load of x (kept
// packed) and one per base of scales.  XM = 0: any batch, dtype and
// alignment, two 16-bit loads per element (the second is the high half of
// an fp32 element, unused otherwise), 16-bit loads of the scales.  Columns at
// or beyond N read 0.
template <int KM, int BB, int XM>
__device__ __forceinline__ void fetch_act(const ProdArgs& a, const ActSrc& src, int n0, ActRaw<KM, BB>& r) {
  if (XM != 0) {
    const uint2 v = ld64(src.x, (uint32_t)n0 * 2u);
    r.x[0][0] = v.x;
    r.x[0][1] = v.y;
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (base_active<KM>(a, k)) r.c[k] = ld64(src.c, (uint32_t)(k * src.N + n0) * 2u);
  } else {
    const uint32_t esz = src.xdt == BSG_F32 ? 4u : 2u;
#pragma unroll
    for (int b = 0; b < BB; ++b) {
      const int bb = src.b0 + b < src.B ? src.b0 + b : src.B - 1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t off = (uint32_t)((n0 + j) * src.B + bb) * esz;
        const uint32_t lo = ld16(src.x, off), hi = ld16(src.x, off + 2);
        r.x[b][j] = esz == 4 ? (lo | (hi << 16)) : lo;
      }
    }
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (base_active<KM>(a, k)) {
        const uint32_t off = (uint32_t)(k * src.N + n0) * 2u;
        r.c[k] = make_uint2(ld16(src.c, off) | (ld16(src.c, off + 2) << 16),
                            ld16(src.c, off + 4) | (ld16(src.c, off + 6) << 16));
      }
    }
  }
}

// Tables of one chunk: the 16 signed sums of 4-column group g (columns
// n_lane .. n_lane + 3), for each of the KX column-scale sets and each batch
// column: entry e = sum_j (2 bit_j(e) - 1) c_j x_j (FluxBin Sec. 3.2: the
// column scale is folded in while the table is built).  Columns at or beyond
// N give a zero table.
template <int Q, int NWL, int KM, int BB, int XM>
__device__ __forceinline__ void build_tables(const ActSrc& s, const ActRaw<KM, BB>& act, int KX, int g, int n_lane,
                                    char* lds, uint32_t wbase_lds) {
  constexpr int STEPS = NWL * 8;          // groups per lane quarter
  constexpr uint32_t ROWB = Q * 64 + 16;  // bytes of one step row: Q tables + 16 pad bytes
  constexpr uint32_t REG = STEPS * ROWB;  // bytes of one (base, batch column) table set
  const int qq = g / STEPS, ii = g % STEPS;
  const bool inb = n_lane < s.N;
#pragma unroll
  for (int kx = 0; kx < KM; ++kx) {
    if (kx < KX) {
#pragma unroll
      for (int b = 0; b < BB; ++b) {
        float xv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t pk = act.x[0][j >> 1];  // XM != 0: two 16-bit values per word
          const float d = XM == 1   ? __uint_as_float((j & 1) ? (pk & 0xffff0000u) : (pk << 16))
                          : XM == 2 ? f16_bits_to_float((uint16_t)((j & 1) ? (pk >> 16) : pk))
                                    : decode_x(act.x[b][j], s.xdt);
          xv[j] = (inb && s.b0 + b < s.B) ? d : 0.0f;
        }
        if (s.cs) {
          xv[0] *= f16_bits_to_float((uint16_t)(act.c[kx].x & 0xffffu));
          xv[1] *= f16_bits_to_float((uint16_t)(act.c[kx].x >> 16));
          xv[2] *= f16_bits_to_float((uint16_t)(act.c[kx].y & 0xffffu));
          xv[3] *= f16_bits_to_float((uint16_t)(act.c[kx].y >> 16));
        }
        // bits 0,1 of e select the first pair's signed sum, bits 2,3 the second's
        const float p0 = xv[0] + xv[1], m0 = xv[0] - xv[1];
        const float p1 = xv[2] + xv[3], m1 = xv[2] - xv[3];
        const float hi[4] = {-p1, m1, -m1, p1};
        float4* dst =
            (float4*)(lds + wbase_lds + (uint32_t)(kx * BB + b) * REG + (uint32_t)ii * ROWB + (uint32_t)qq * 64);
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = make_float4(-p0 + hi[e], m0 + hi[e], -m0 + hi[e], p0 + hi[e]);
      }
    }
  }
}

// Lookups of one chunk: acc[k][b] += table entry of each 4-bit slice.  Words
// beyond ND are zero words (padding) or read 0 (beyond the row block) and
// their columns' tables are zero, so they add +-0 and need no guard.  Word j
// of every base is looked up together: 8K independent LDS reads in flight
// and K independent add chains.
template <int Q, int NWL, int KM, int BB>
__device__ __forceinline__ void lookup_chunk(const ProdArgs& a, const char* lds, uint32_t wbase_lds, bool cs, int q,
                                    const uint32_t (&cur)[KM][NWL], float (&acc)[KM][BB]) {
  constexpr uint32_t ROWB = Q * 64 + 16;             // bytes of one step row of tables
  constexpr uint32_t REG = NWL * 8 * ROWB;           // bytes of one (base, batch column) table set
  uint32_t lbase[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k)
    lbase[k] = (uint32_t)(uintptr_t)(lds + wbase_lds + (uint32_t)(cs ? k : 0) * BB * REG + (uint32_t)q * 64);
#pragma unroll
  for (int j = 0; j < NWL; ++j) {
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (base_active<KM>(a, k)) {
        const uint32_t word = cur[k][j];
        const uint32_t rl = __builtin_amdgcn_alignbit(word, word, 30) & 0x3c3c3c3cu;  // even slices * 4
        const uint32_t rr = __builtin_amdgcn_alignbit(word, word, 2) & 0x3c3c3c3cu;   // odd slices * 4
        uint32_t ad[8];
        ad[0] = byte_add<0>(lbase[k], rl);
        ad[1] = byte_add<0>(lbase[k], rr);
        ad[2] = byte_add<1>(lbase[k], rl);
        ad[3] = byte_add<1>(lbase[k], rr);
        ad[4] = byte_add<2>(lbase[k], rl);
        ad[5] = byte_add<2>(lbase[k], rr);
        ad[6] = byte_add<3>(lbase[k], rl);
        ad[7] = byte_add<3>(lbase[k], rr);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
#pragma unroll
          for (int b = 0; b < BB; ++b) acc[k][b] += lds_f32(ad[n] + (uint32_t)(j * 8 + n) * ROWB + (uint32_t)b * REG);
        }
      }
    }
    // finish word j's adds here: left free, the compiler sinks the add chains
    // to the end of the loop body and keeps every table entry of the chunk
    // live, which exhausts the registers
#pragma unroll
    for (int k = 0; k < KM; ++k)
#pragma unroll
      for (int b = 0; b < BB; ++b) asm volatile("" : "+v"(acc[k][b]));
  }
}

// Activations of one 4-column group of the salient matrix (FluxBin Sec. 3.2
// Virtual Columnar Mapping): physical columns p0 .. p0 + 3 read x at the
// logical columns idx[p0 + j] (an index outside [0, N) reads 0), with the
// salient column scales (8-byte aligned: one load per base); the raw form of
// fetch_act's generic path, one load per element.  iv: the four indices.
template <int KM, int BB>
__device__ __forceinline__ void fetch_gather(const ProdArgs& a, const ActSrc& src, uint4 iv, int n_true, int p0,
                                             ActRaw<KM, BB>& r) {
  const uint32_t id[4] = {iv.x, iv.y, iv.z, iv.w};
  const uint32_t esz = src.xdt == BSG_F32 ? 4u : 2u;
#pragma unroll
  for (int b = 0; b < BB; ++b) {
    const int bb = src.b0 + b < src.B ? src.b0 + b : src.B - 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t off = id[j] < (uint32_t)n_true ? (id[j] * (uint32_t)src.B + (uint32_t)bb) * esz : 0xfffffff0u;
      r.x[b][j] = esz == 4 ? ld32(src.x, off) : ld16(src.x, off);
    }
  }
#pragma unroll
  for (int k = 0; k < KM; ++k)
    if (base_active<KM>(a, k)) r.c[k] = ld64(src.c, (uint32_t)(k * src.N + p0) * 2u);
}

// Lookups of one salient chunk: like lookup_chunk, but each 4-bit slice's
// entry is scaled by the fp16 row scale of its group (GPW groups per word:
// slice n of a word lies in group n * GPW / 8), sc[k][j] holding word j's
// GPW scales (two per 32-bit value).
template <int Q, int NWL, int KM, int GPW>
__device__ __forceinline__ void lookup_chunk_scaled(const ProdArgs& a, const char* lds, uint32_t wbase_lds, bool cs,
                                                    int q, const uint32_t (&cur)[KM][NWL],
                                                    const uint2 (&sc)[KM][NWL], float (&acc)[KM]) {
  constexpr uint32_t ROWB = Q * 64 + 16;
  constexpr uint32_t REG = NWL * 8 * ROWB;
#pragma unroll
  for (int j = 0; j < NWL; ++j) {
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (base_active<KM>(a, k)) {
        const uint32_t lbase = (uint32_t)(uintptr_t)(lds + wbase_lds + (uint32_t)(cs ? k : 0) * REG + (uint32_t)q * 64);
        const uint32_t word = cur[k][j];
        const uint32_t rl = __builtin_amdgcn_alignbit(word, word, 30) & 0x3c3c3c3cu;
        const uint32_t rr = __builtin_amdgcn_alignbit(word, word, 2) & 0x3c3c3c3cu;
        const uint32_t ad[8] = {byte_add<0>(lbase, rl), byte_add<0>(lbase, rr), byte_add<1>(lbase, rl),
                                byte_add<1>(lbase, rr), byte_add<2>(lbase, rl), byte_add<2>(lbase, rr),
                                byte_add<3>(lbase, rl), byte_add<3>(lbase, rr)};
        float f[GPW];
#pragma unroll
        for (int t = 0; t < GPW; ++t) {
          const uint32_t w2 = t < 2 ? sc[k][j].x : sc[k][j].y;
          f[t] = f16_bits_to_float((uint16_t)((t & 1) ? (w2 >> 16) : w2));
        }
#pragma unroll
        for (int n = 0; n < 8; ++n)
          acc[k] = __builtin_fmaf(f[n * GPW / 8], lds_f32(ad[n] + (uint32_t)(j * 8 + n) * ROWB), acc[k]);
      }
    }
  }
}

// First index i in [0, n) with rows[i] >= key (n if none), rows ascending:
// a 64-way search, one probe per lane per round, so about log64(n) + 1
// dependent loads.  Uniform over the wavefront.
__device__ __forceinline__ int lower_bound_rows(rsrc_t rows, int n, int key, int lane) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int step = (hi - lo + 63) / 64;
    const int p = lo + (lane + 1) * step - 1;
    const bool ge = p >= hi || (int)ld32(rows, (uint32_t)p * 4u) >= key;
    const unsigned long long bal = __ballot(ge);
    const int f = bal ? __builtin_ctzll(bal) : 64;
    const int nlo = min(lo + f * step, hi);
    const int nhi = f < 64 ? min(lo + (f + 1) * step - 1, hi) : hi;
    lo = __builtin_amdgcn_readfirstlane(nlo);
    hi = __builtin_amdgcn_readfirstlane(nhi);
  }
  return lo;
}

// Register budget.  With one or two bases, one aligned 16-bit batch column
// and Q >= 2 the tables of a 16-wavefront workgroup take at most half the
// LDS, and the kernel is held to 64 VGPRs (8 wavefronts per SIMD) so that two
// such workgroups share a compute unit (the generic activation path needs
// more registers and is not held).  Instances with KM * BB >= 8 keep more
// sums in registers and run at most 8 wavefronts per workgroup.
// MP = 1: the fused launch of several projections (bs_gemv_multi); the
// single-product instances (MP = 0) carry none of its code.  GS >= 1: one row
// scale per group of a.gsw sign words (FluxBin Sec. 3.1, group-wise row
// scales): each lane's words of a chunk lie in one group, so the lane sums
// a chunk apart and adds it times its group's scales, which are loaded with
// the chunk's sign words (two chunks ahead, in three buffers).  GS = 2 adds
// the salient-column bases.
template <int Q, int NWL, int KM, int BB, int XM, int MP, int GS = 0>
__global__ void __launch_bounds__(64 * prod_max_waves(KM, BB, GS, XM), (KM <= 2 && BB == 1 && Q >= 2 && XM != 0 && !GS) ? 8 : 1)
    k_prod_f(ProdArgs a) {
  constexpr int RW = 64 / Q;
  constexpr int CW = Q * NWL;
  constexpr int G = CW * 8;             // 4-column groups per chunk
  constexpr int GPL = (G + 63) / 64;    // groups built per lane (lane, lane + 64)
  extern __shared__ __align__(16) char lds[];

  // every argument the prologue needs, in registers before anything else:
  // one batch of scalar loads and one wait, ahead of the first vector loads
  asm volatile("" ::"s"(a.bits), "s"(a.alpha), "s"(a.colscale), "s"(a.x), "s"(a.plane), "s"(a.K), "s"(a.M),
               "s"(a.N), "s"(a.ND), "s"(a.B), "s"(a.b0), "s"(a.xdt), "s"(a.NCH), "s"(a.wave_lds), "s"(a.x_bytes),
               "s"(a.cs_bytes), "s"(a.al_bytes));
  // fused launch: this workgroup's projection and its block within it
  uint32_t blk = blockIdx.x;
  if (MP) {
    // constant indices only (a computed index would copy the arguments to
    // scratch memory)
    ProjDesc d = a.proj[0];
#pragma unroll
    for (int i = 1; i < kMaxProj; ++i)
      if (i < a.np && (int)blockIdx.x >= a.proj[i].wg0) d = a.proj[i];
    a.bits = d.bits;
    a.alpha = d.alpha;
    a.colscale = d.colscale;
    a.y = d.y;
    a.plane = d.plane;
    a.M = d.M;
    a.al_bytes = d.al_bytes;
    a.cs_bytes = d.cs_bytes;
    blk = blockIdx.x - d.wg0;
  }
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wavefront index (uniform)
  const int q = lane / RW;
  const int r = lane % RW;
  const int m = (int)(blk * RW + r);
  const bool valid = m < a.M;
  // rows beyond M read padding; their sums are dropped
  const SignRows<KM> srows = sign_rows<KM, RW>(a.bits, a.plane, a.K, a.ND, blk, m);
  const ActSrc asrc = act_src(a);
  const rsrc_t alsrc = make_rsrc(a.alpha, a.al_bytes);
  const bool cs = a.colscale != nullptr;
  const int KX = cs ? a.K : 1;
  const uint32_t wbase_lds = (uint32_t)wv * a.wave_lds;
  // lane builds the tables of groups lane + 64 i (i < GPL) that exist
  auto grp = [&](int i) { return lane + 64 * i < G ? lane + 64 * i : 0; };

  float acc[KM][BB];
#pragma unroll
  for (int k = 0; k < KM; ++k)
#pragma unroll
    for (int b = 0; b < BB; ++b) acc[k][b] = 0.0f;

  // First chunk: activations and column scales, row scales, then the sign
  // words of the first two chunks, all in flight at once.  Loads complete in
  // issue order, so the table build (which needs only the activations) need
  // not wait for the sign words.  Sign words stay two chunks ahead of the
  // lookups, in three buffers used round-robin (the loop is unrolled by
  // three: a register copy between buffers would wait for the loads in
  // flight); activations stay one chunk ahead of the build.
  uint32_t wb0[KM][NWL], wb1[KM][NWL], wb2[KM][NWL];
  ActRaw<KM, BB> act[GPL];
  float al[KM];
  const int c0 = wv * a.NCH;  // this wavefront's first chunk
#pragma unroll
  for (int i = 0; i < GPL; ++i) fetch_act<KM, BB, XM>(a, asrc, c0 * CW * 32 + grp(i) * 4, act[i]);
#pragma unroll
  for (int k = 0; k < KM; ++k)
    if (!GS && base_active<KM>(a, k)) al[k] = __uint_as_float(ld32(alsrc, (uint32_t)(k * a.M + m) * 4u));
  // Prefetches past the wavefront's last chunk re-read that chunk (a cache
  // hit, no HBM traffic) instead of being skipped: unconditional loads keep
  // the compiler's load counting exact, so every wait is for the oldest load.
  const int clast = a.NCH - 1;
  // group scales of chunk cc (GS): the lane's group in it
  float ab0[KM], ab1[KM], ab2[KM];
  auto load_gscale = [&](int cc, float (&d)[KM]) {
    const int j = ((c0 + cc) * CW + q * NWL) / a.gsw;
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (base_active<KM>(a, k))
        d[k] = f16_bits_to_float((uint16_t)ld16(alsrc, (uint32_t)((k * a.ngrp + j) * a.M + m) * 2u));
  };
  load_chunk<KM, NWL>(a, srows, c0 * CW + q * NWL, wb0);
  if (GS) load_gscale(0, ab0);
  load_chunk<KM, NWL>(a, srows, (c0 + min(1, clast)) * CW + q * NWL, wb1);
  if (GS) load_gscale(min(1, clast), ab1);

  // Salient columns (GS = 2; FluxBin Sec. 3.1 hybrid bases, Sec. 3.2 Virtual
  // Columnar Mapping): K more bases over the dense physical matrix of the
  // gathered columns, after the main chunks.  Its chunks go round-robin
  // from wavefront 0: the first wavefronts start first (measured: 6.6 us
  // against 7.5 us at 4096 x 4096, s = 8, when they went to the last ones).
  // (Gathering the first salient chunk's activations here instead, behind
  // the main chunks' first loads, measured slower: the gather waits for the
  // index list and with it for every load issued before.)
  const int vc0 = wv;  // this wavefront's first salient chunk
  const int nds = a.vs_nd;
  const SignRows<KM> vrows = sign_rows<KM, RW>(a.vs_bits, a.vs_plane, a.K, nds, blk, m);
  ActSrc ss = asrc;
  ss.N = a.vs_S;
  ss.c = make_rsrc(a.vs_cs, a.vs_cs ? (size_t)a.K * a.vs_S * 2 : 0);
  ss.cs = a.vs_cs != nullptr;
  const rsrc_t ir = make_rsrc(a.vs_idx, (size_t)a.vs_S * 4);
  const rsrc_t sar = make_rsrc(a.vs_alpha, (size_t)a.K * nds * a.M * a.vs_gpw * 2);
  // the gathered activations, sign words and row scales of salient chunk cu
  auto salient_gather = [&](int cu, ActRaw<KM, BB>(&ga)[GPL]) {
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const int p0 = cu * CW * 32 + grp(i) * 4;
      fetch_gather<KM, BB>(a, ss, ld128(ir, (uint32_t)p0 * 4u), a.N, p0, ga[i]);
    }
  };
  auto salient_words = [&](int cu, uint32_t(&sw)[KM][NWL], uint2(&sc)[KM][NWL]) {
    load_chunk<KM, NWL>(a, vrows, cu * CW + q * NWL, sw);
    const int gpw = a.vs_gpw;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
#pragma unroll
      for (int j = 0; j < NWL; ++j) {
        if (base_active<KM>(a, k)) {
          const uint32_t off = (uint32_t)(((k * nds + cu * CW + q * NWL + j) * a.M + m) * gpw) * 2u;
          if (gpw == 4) sc[k][j] = ld64(sar, off);
          else if (gpw == 2) sc[k][j] = make_uint2(ld32(sar, off), 0u);
          else sc[k][j] = make_uint2(ld16(sar, off), 0u);
        }
      }
    }
  };

  // one chunk: build its tables, issue the next chunk's activations and the
  // sign words two chunks ahead (into `ahead`), look up `cur`
  auto chunk = [&](int c, const uint32_t(&cur)[KM][NWL], uint32_t(&ahead)[KM][NWL], const float(&gcur)[KM],
                   float(&gahead)[KM]) {
    const int cw0 = (c0 + c) * CW;  // first word of the chunk
#pragma unroll
    for (int i = 0; i < GPL; ++i)
      if (lane + 64 * i < G)
        build_tables<Q, NWL, KM, BB, XM>(asrc, act[i], KX, lane + 64 * i, cw0 * 32 + (lane + 64 * i) * 4, lds,
                                         wbase_lds);
#pragma unroll
    for (int i = 0; i < GPL; ++i)
      fetch_act<KM, BB, XM>(a, asrc, (c0 + min(c + 1, clast)) * CW * 32 + grp(i) * 4, act[i]);
    load_chunk<KM, NWL>(a, srows, (c0 + min(c + 2, clast)) * CW + q * NWL, ahead);
    if (GS) load_gscale(min(c + 2, clast), gahead);
    wave_sync();  // the tables are private to this wavefront
    if (GS) {
      float cacc[KM][BB];
#pragma unroll
      for (int k = 0; k < KM; ++k)
#pragma unroll
        for (int b = 0; b < BB; ++b) cacc[k][b] = 0.0f;
      lookup_chunk<Q, NWL, KM, BB>(a, lds, wbase_lds, cs, q, cur, cacc);
#pragma unroll
      for (int k = 0; k < KM; ++k)
#pragma unroll
        for (int b = 0; b < BB; ++b) acc[k][b] += gcur[k] * cacc[k][b];
    } else {
      lookup_chunk<Q, NWL, KM, BB>(a, lds, wbase_lds, cs, q, cur, acc);
    }
    wave_sync();  // the next chunk's tables overwrite these
  };
  // No branch inside the loop body: the compiler's load counting at the
  // back edge stays exact.  The last one or two chunks run after it.
  int c = 0;
  for (; c + 3 <= a.NCH; c += 3) {
    chunk(c, wb0, wb2, ab0, ab2);
    chunk(c + 1, wb1, wb0, ab1, ab0);
    chunk(c + 2, wb2, wb1, ab2, ab1);
  }
  if (c < a.NCH) chunk(c, wb0, wb2, ab0, ab2);
  if (c + 1 < a.NCH) chunk(c + 1, wb1, wb0, ab1, ab0);

  // ---- row scales
  float tot[BB];
#pragma unroll
  for (int b = 0; b < BB; ++b) tot[b] = 0.0f;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (base_active<KM>(a, k)) {
      const float alk = (GS || !a.alpha) ? 1.0f : al[k];  // group scales are in acc already
#pragma unroll
      for (int b = 0; b < BB; ++b) tot[b] += alk * acc[k][b];
    }
  }

  // ---- fused binary low-rank expansion: y += U (alpha_r (.) z), the same
  // sign product over the r ranks (BiLoCo, "The core idea"); the chunks of
  // U's r/32 words per row go round-robin over the wavefronts
  if (a.lr_bits) {
    const ActSrc ls = lr_src(a);
    const int ndu = a.lr_r / 32;
    const SignRows<1> urows = sign_rows<1, RW>(a.lr_bits, a.lr_plane, 1, ndu, blk, m);
    const int tu = (pad_words(ndu) + CW - 1) / CW;
    float lacc[1][BB];
#pragma unroll
    for (int b = 0; b < BB; ++b) lacc[0][b] = 0.0f;
    for (int cu = wv; cu < tu; cu += a.W) {
      ActRaw<1, BB> la[GPL];
      uint32_t uw[1][NWL];
#pragma unroll
      for (int i = 0; i < GPL; ++i) fetch_act<1, BB, 0>(a, ls, cu * CW * 32 + grp(i) * 4, la[i]);
      load_chunk<1, NWL>(a, urows, cu * CW + q * NWL, uw);
      wave_sync();  // earlier lookups of this wavefront's tables are done
#pragma unroll
      for (int i = 0; i < GPL; ++i)
        if (lane + 64 * i < G)
          build_tables<Q, NWL, 1, BB, 0>(ls, la[i], 1, lane + 64 * i, cu * CW * 32 + (lane + 64 * i) * 4, lds,
                                         wbase_lds);
      wave_sync();
      lookup_chunk<Q, NWL, 1, BB>(a, lds, wbase_lds, true, q, uw, lacc);
    }
#pragma unroll
    for (int b = 0; b < BB; ++b) tot[b] += lacc[0][b];
  }

  // ---- the salient chunks (GS = 2)
  if (GS == 2) {
    const int KS = ss.cs ? a.K : 1;
    const int ts = (nds + CW - 1) / CW;
    float sacc[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k) sacc[k] = 0.0f;
    auto pass = [&](auto gpw_c) {
      constexpr int GPW = decltype(gpw_c)::value;
      for (int cu = vc0; cu < ts; cu += a.W) {
        ActRaw<KM, BB> ga[GPL];
        uint32_t sw[KM][NWL];
        uint2 sc[KM][NWL];
        salient_words(cu, sw, sc);
        salient_gather(cu, ga);
        wave_sync();  // earlier lookups of this wavefront's tables are done
#pragma unroll
        for (int i = 0; i < GPL; ++i)
          if (lane + 64 * i < G)
            build_tables<Q, NWL, KM, BB, 0>(ss, ga[i], KS, lane + 64 * i, cu * CW * 32 + (lane + 64 * i) * 4, lds,
                                            wbase_lds);
        wave_sync();
        lookup_chunk_scaled<Q, NWL, KM, GPW>(a, lds, wbase_lds, ss.cs, q, sw, sc, sacc);
      }
    };
    if (a.vs_gpw == 4) pass(std::integral_constant<int, 4>());
    else if (a.vs_gpw == 2) pass(std::integral_constant<int, 2>());
    else pass(std::integral_constant<int, 1>());
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (base_active<KM>(a, k)) tot[0] += sacc[k];
  }

  // ---- fused protected rows: y[rows[i]] += s_i (q_i . x) (BiSCo-LLM,
  // "Sensitivity Protection"); each of the workgroup's protected rows is
  // split into shares of 1024 columns over its first wavefronts (one round
  // of loads for N <= 1024 W; the first wavefronts start first), and the
  // shares meet in the workgroup's final sum of wavefront partials
  if (a.sal_n > 0) {
    const rsrc_t rs = make_rsrc(a.sal_rows, (size_t)a.sal_n * 4);
    const rsrc_t qs = make_rsrc(a.sal_q, (size_t)a.sal_n * a.N);
    const rsrc_t ss = make_rsrc(a.sal_s, (size_t)a.sal_n * 2);
    const int m0 = (int)(blk * RW);
    const int i0 = lower_bound_rows(rs, a.sal_n, m0, lane);
    const int i1 = lower_bound_rows(rs, a.sal_n, m0 + RW, lane);
    // shares of 1024 columns (one load per lane), or 1024 times the fewest
    // rounds that reach N over W wavefronts: the first wavefronts take them
    const int span = 1024 * ((a.N + 1024 * a.W - 1) / (1024 * a.W));
    const int c1 = min(a.N, (wv + 1) * span);
    for (int i = i0; i < i1; ++i) {
      const int rr = __builtin_amdgcn_readfirstlane((int)ld32(rs, (uint32_t)i * 4u)) - m0;
      float dot[BB];
#pragma unroll
      for (int b = 0; b < BB; ++b) dot[b] = 0.0f;
      for (int n0 = wv * span + lane * 16; n0 < c1; n0 += 1024) {
        const uint4 qv = ld128(qs, (uint32_t)((size_t)i * a.N + n0));
        const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
        if (XM != 0) {  // 16 aligned 16-bit activations: two 16-byte loads
          const uint4 x0 = ld128(asrc.x, (uint32_t)n0 * 2u), x1 = ld128(asrc.x, (uint32_t)n0 * 2u + 16u);
          const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const uint32_t pk = xw[j >> 1];
            const float xv = XM == 1 ? __uint_as_float((j & 1) ? (pk & 0xffff0000u) : (pk << 16))
                                     : f16_bits_to_float((uint16_t)((j & 1) ? (pk >> 16) : pk));
            const float qf = (float)(int8_t)(qw[j >> 2] >> (8 * (j & 3)));
            dot[0] = __builtin_fmaf(qf, xv, dot[0]);
          }
        } else {
#pragma unroll
          for (int b = 0; b < BB; ++b) {
            const int bb = a.b0 + b < a.B ? a.b0 + b : a.B - 1;
            const uint32_t esz = a.xdt == BSG_F32 ? 4u : 2u;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const uint32_t off = (uint32_t)((n0 + j) * a.B + bb) * esz;
              const uint32_t lo = ld16(asrc.x, off), hi = ld16(asrc.x, off + 2);
              const float xv = decode_x(esz == 4 ? (lo | (hi << 16)) : lo, a.xdt);
              const float qf = (float)(int8_t)(qw[j >> 2] >> (8 * (j & 3)));
              dot[b] = __builtin_fmaf(qf, xv, dot[b]);
            }
          }
        }
      }
      const float sv = f16_bits_to_float((uint16_t)ld16(ss, (uint32_t)i * 2u));
#pragma unroll
      for (int b = 0; b < BB; ++b) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) dot[b] += __shfl_xor(dot[b], o);
        if (r == rr && q == 0 && a.b0 + b < a.B) tot[b] += sv * dot[b];
      }
    }
  }

  // ---- the Q lanes of a row, then the W wavefronts, in a fixed order
#pragma unroll
  for (int b = 0; b < BB; ++b) {
    if (!valid) tot[b] = 0.0f;
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
    const int mm = (int)(blk * RW + rr);
    if (mm < a.M && a.b0 + b < a.B) {
      const float s = sum_waves(red + rr * BB + b, RW * BB, a.W);
      const size_t yi = (size_t)mm * a.B + a.b0 + b;
      a.y[yi] = (a.accumulate ? a.y[yi] : 0.0f) + s;
    }
  }
}

}  // namespace bsg
