// Internal declarations shared by the libbsg translation units (device code
// for gfx950 and the host-side launchers).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bsg.h"

namespace bsg {

constexpr int kRowBlock = 64;   // rows per layout tile = lanes per wavefront
constexpr int kGroupWords = 4;  // words per layout tile (one 16-byte load per lane)
constexpr int kMaxK = 8;
constexpr int kMaxB = 64;
constexpr int kMaxFitRank = 2048;  // binlr_fit: the r x r refit is solved on the host
constexpr size_t kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950

// Words of one base in the device layout: M*ND rounded up to 64 words.
// Device layout (documented in bsg.h): rows padded to a multiple of 64,
// words per row to a multiple of 4, whole 64 x 4-word tiles.
__host__ __device__ inline int pad_rows(int M) { return (M + 63) & ~63; }
__host__ __device__ inline int pad_words(int ND) { return (ND + 3) & ~3; }
__host__ __device__ inline size_t plane_words(int M, int ND) { return (size_t)pad_rows(M) * (size_t)pad_words(ND); }

// Device-layout word offset of logical word w of row m of base k.
__host__ __device__ inline size_t layout_offset(int M, int ND, size_t plane, int k, int m, int w) {
  (void)M;
  return (size_t)k * plane + (size_t)(m >> 6) * 64 * (size_t)pad_words(ND) + (size_t)(w >> 2) * 256 +
         (size_t)(m & 63) * 4 + (size_t)(w & 3);
}

// bf16 / fp16 bit patterns -> fp32 (exact).
__device__ inline float bf16_bits_to_float(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ inline float f16_bits_to_float(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return (float)v;
}

__device__ inline float load_x(const void* x, int dt, size_t i) {
  if (dt == BSG_F32) return ((const float*)x)[i];
  if (dt == BSG_BF16) return bf16_bits_to_float(((const uint16_t*)x)[i]);
  return f16_bits_to_float(((const uint16_t*)x)[i]);
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Launch plan of the sign products (bsg_gemv.hip).  A workgroup owns RW =
// 64/Q full rows; Q lanes of a wavefront share a row and each covers 1/Q of
// the wavefront's column chunk; W wavefronts split the input dimension into
// chunks of CW = Q*NWL sign words, NCH chunks each.  No reduction crosses
// workgroups.
struct ProdPlan {
  int Q;       // lanes per row: 1, 2 or 4
  int NWL;     // sign words per lane per chunk and base
  int KM;      // bases unrolled: K itself for K <= 4, else 8
  int XM;      // float kernel activation path: 0 generic, 1 / 2 one aligned bf16 / fp16 batch column
  int BB;      // batch columns per launch
  int CW;      // words per chunk (Q * NWL)
  int RW;      // rows per workgroup (64 / Q)
  int W;       // wavefronts per workgroup
  int NCH;     // chunks per wavefront
  int nwg;     // workgroups
  int nlaunch; // launches over batch chunks of BB columns
  size_t wave_lds;  // LDS bytes per wavefront (tables or bit planes)
  size_t lds;       // LDS bytes per workgroup
};

// gsw > 0: group-wise row scales with groups of gsw sign words (one batch
// column per launch, lanes kept inside a group).
ProdPlan plan_prod(int K, int M, int N, int B, bool colscale, bool int8_mode, int gsw = 0);

// One projection of a fused launch (bs_gemv_multi): its own weights, scales
// and output, the first workgroup of its row blocks in the grid.
constexpr int kMaxProj = 8;
struct ProjDesc {
  const uint32_t* bits;
  const float* alpha;
  const uint16_t* colscale;
  float* y;
  size_t plane;
  int M, wg0;
  uint32_t al_bytes, cs_bytes;
};

struct ProdArgs {
  // Read by the prologue of every product kernel: kept together at the front
  // so that they arrive in one batch of scalar loads.
  const uint32_t* bits;
  const float* alpha;        // fp32 [K][M], or NULL
  const uint16_t* colscale;  // fp16 [K][N], or NULL
  const void* x;             // [N][B] of dtype xdt (float path)
  float* y;                  // [M][B] or NULL (int8 path)
  size_t plane;
  int K, M, N, ND;
  int B, b0, xdt, accumulate;
  int W, NCH;
  uint32_t wave_lds;
  // operand sizes in bytes (0 for an absent operand), set by the launcher so
  // that the kernel prologue has no branches
  uint32_t x_bytes, cs_bytes, al_bytes;
  int xvec;                  // x 16-byte and colscale 8-byte aligned: vector loads
  int gsw, ngrp;             // group-wise row scales (fp16 [K][ngrp][M] at alpha): words per group, groups
  // Salient columns of the group-wise path (FluxBin VCM; NULL vs_bits when
  // absent): K bases over vs_S physical columns p, column p reading x[vs_idx[p]];
  // fp16 row scales word-grouped, vs_gpw per sign word: (k, w, m, t) at
  // ((k * vs_nd + w) * M + m) * vs_gpw + t; fp16 column scales [K][vs_S]
  const uint32_t* vs_bits;
  size_t vs_plane;
  const int32_t* vs_idx;
  const uint16_t* vs_alpha;
  const uint16_t* vs_cs;
  int vs_S, vs_nd, vs_gpw;
  // int8 path
  const int8_t* xq;          // [N][B]
  const float* sx;           // [B]
  int32_t* acc;              // [K][M][B] or NULL
  // Fused terms of bsg_linear (float path; NULL / 0 when absent):
  //   y += U (lr_scale (.) lr_z)        binary low-rank expansion, z = V x precomputed
  //   y[sal_rows[i]] += sal_s[i] * (sal_q[i] . x)   protected int8 rows
  const uint32_t* lr_bits;   // U: device layout, M x lr_r signs, or NULL
  size_t lr_plane;
  const float* lr_z;         // [lr_r][B]
  const uint16_t* lr_scale;  // fp16 [lr_r]
  int lr_r;                  // rank, a multiple of 32
  int sal_n;                 // protected rows (0: none)
  const int32_t* sal_rows;   // [sal_n], ascending
  const int8_t* sal_q;       // [sal_n][N]
  const uint16_t* sal_s;     // fp16 [sal_n]
  // Fused launch of np > 1 projections sharing x (float path, bases only):
  // workgroup w works for the last projection p with proj[p].wg0 <= w.
  int np;
  ProjDesc proj[kMaxProj];
  // Batched low-rank expansion on the matrix cores (NULL when unused): a
  // second activation array summed into the same product, and the split
  // output hi/lo = bf16 halves of split_scale[m] * y[m][b]
  const void* x2;
  uint16_t* split_hi;
  uint16_t* split_lo;
  const uint16_t* split_scale;
};

hipError_t launch_prod_f(const ProdArgs& a, const ProdPlan& p, hipStream_t s);
// One launch over a.np > 1 projections (a.proj) sharing x (bsg_gemv.hip).
hipError_t launch_prod_multi(const ProdArgs& a, hipStream_t s);
// Group-wise row scales (bsg_gemv_gs.hip): a.gsw, a.ngrp set, alpha fp16 [K][ngrp][M];
// optional salient columns (a.vs_*).
hipError_t launch_prod_grouped(const ProdArgs& a, hipStream_t s);
// Batched product on the matrix cores (bsg_gemv_mfma.hip): B >= 4 columns of
// bf16 / fp16 x, no column scales.
bool mfma_eligible(int B, int xdt, bool colscale);
hipError_t launch_prod_mfma(const ProdArgs& a, hipStream_t s);
// The matrix-core path can fuse projections (a.np > 1) for this B and x.
bool mfma_multi_ok(int B, const void* x);
// The matrix-core path takes column scales (fp16 x) and group-wise row scales
// (a.gsw words per group, >= 4) for this B, x and M.
bool mfma_cg_ok(int B, int xdt, const void* x, bool colscale, int gsw, int M);
// Salient-column bases (a.vs_*) on the matrix cores after the main product
// (bsg_vcm_mfma.hip): fp16 x, B >= 4, K <= 4, the gathered x within the LDS.
bool vcm_mfma_ok(int B, int xdt, const void* x, int K, int S, bool cs);
hipError_t launch_vcm_mfma(const ProdArgs& a, hipStream_t s);
hipError_t launch_prod_i8(const ProdArgs& a, const ProdPlan& p, hipStream_t s);

}  // namespace bsg
