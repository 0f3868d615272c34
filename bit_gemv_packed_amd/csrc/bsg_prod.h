// Device helpers shared by the float and int8 sign-product kernels, and the
// set of kernel instances the launch planner may choose.
#pragma once

#include "bsg_internal.h"

#include <mutex>
#include <unordered_set>

namespace bsg {

// (byte J of v) + base in one VALU instruction (SDWA operand select).
template <int J>
__device__ inline uint32_t byte_add(uint32_t base, uint32_t v);
#define BSG_BYTE_ADD(J)                                                                                  \
  template <>                                                                                            \
  __device__ inline uint32_t byte_add<J>(uint32_t base, uint32_t v) {                                    \
    uint32_t r;                                                                                          \
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_" #J \
        : "=v"(r)                                                                                        \
        : "v"(base), "v"(v));                                                                            \
    return r;                                                                                            \
  }
BSG_BYTE_ADD(0)
BSG_BYTE_ADD(1)
BSG_BYTE_ADD(2)
BSG_BYTE_ADD(3)
#undef BSG_BYTE_ADD

// Kernels are instantiated for the exact number of bases K = KM when K <= 4
// (no per-base branch) and for KM = 8 covering K = 5..8 (guarded).
template <int KM>
__device__ inline bool base_active(const ProdArgs& a, int k) {
  return KM <= 4 || k < a.K;
}

// Buffer resources.  Operands are read with buffer loads: a 128-bit
// descriptor in scalar registers (base, size in bytes) plus a 32-bit byte
// offset per lane.  That halves the address registers of 64-bit pointers,
// and a read at or beyond the size returns 0 without touching memory (a
// descriptor of size 0 for an absent operand reads all zeros).  Word 3 of
// the descriptor is the gfx9 raw-buffer setting (32-bit data format).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t make_rsrc(const void* p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}
__device__ inline uint32_t ld32(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0); }
__device__ inline uint2 ld64(rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v[0], v[1]);
}
__device__ inline uint4 ld128(rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ inline uint32_t ld16(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0); }
__device__ inline uint32_t ld8(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0); }

// The sign words of one workgroup: all its rows lie in one 64-row block
// (RW divides 64), so each base's block is one resource, uniform over the
// workgroup: 64 rows x NDP words (padded layout, bsg.h).  Row blocks hold
// zero words in their padding rows and words, so rows beyond M and words
// beyond ND need no guard; words beyond NDP are out of range and read 0.
template <int KM>
struct SignRows {
  rsrc_t r[KM];
  uint32_t row_off;  // byte offset of this lane's row in a tile: (m % 64) * 16
};
// rb: the (uniform) 64-row block, m: this lane's row in it
template <int KM>
__device__ inline SignRows<KM> sign_rows_in(const uint32_t* bits, size_t plane, int K, int ND, int rb, int m) {
  SignRows<KM> s;
  const size_t blk = (size_t)64 * pad_words(ND);  // words of one row block
  s.row_off = (uint32_t)(m & 63) * 16u;
#pragma unroll
  for (int k = 0; k < KM; ++k)
    s.r[k] = make_rsrc(bits + (size_t)(k < K ? k : 0) * plane + (size_t)rb * blk, blk * 4);
  return s;
}
// workgroup blk (uniform) owns rows [blk RW, blk RW + RW)
template <int KM, int RW>
__device__ inline SignRows<KM> sign_rows(const uint32_t* bits, size_t plane, int K, int ND, uint32_t blk, int m) {
  return sign_rows_in<KM>(bits, plane, K, ND, (int)(blk * RW) >> 6, m);
}

// Sign words of one chunk: NWL consecutive logical words [w0, w0 + NWL) of
// the lane's row for every base k < K (w0 is a multiple of min(NWL, 4)):
// 4-, 8- or 16-byte loads at tile (w0 / 4) * 1 KiB + row * 16 + (w0 % 4) * 4.
template <int KM, int NWL>
__device__ inline void load_chunk(const ProdArgs& a, const SignRows<KM>& s, int w0, uint32_t (&wd)[KM][NWL]) {
  constexpr int PW = NWL < 4 ? NWL : 4;  // words per load
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (base_active<KM>(a, k)) {
#pragma unroll
      for (int g = 0; g < NWL / PW; ++g) {
        const int wf = w0 + g * PW;
        const uint32_t off = (uint32_t)(wf >> 2) * 1024u + s.row_off + (uint32_t)(wf & 3) * 4u;
        if (PW == 4) {
          const uint4 v = ld128(s.r[k], off);
          wd[k][g * 4 + 0] = v.x;
          wd[k][g * 4 + 1] = v.y;
          wd[k][g * 4 + 2] = v.z;
          wd[k][g * 4 + 3] = v.w;
        } else if (PW == 2) {
          const uint2 v = ld64(s.r[k], off);
          wd[k][g * 2 + 0] = v.x;
          wd[k][g * 2 + 1] = v.y;
        } else {
          wd[k][g] = ld32(s.r[k], off);
        }
      }
    }
  }
}

// Orders this wavefront's LDS writes before its later LDS reads (and reads
// before later writes) across its lanes; no workgroup barrier.
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Most wavefronts per workgroup of an instance: 16, or 8 where KM * BB >= 8
// partial sums (and as many sign-word sets) live in registers, or four bases
// carry group scales as well, or three do with the generic activation path
// (XM = 0; XM < 0: not yet chosen), so that the kernel has up to 256 VGPRs
// and does not spill.
constexpr int prod_max_waves(int KM, int BB, int GS = 0, int XM = -1) {
  return (KM * BB >= 8 || (GS && KM >= 4) || (GS && KM >= 3 && XM == 0)) ? 8 : 16;
}

// Sum of the W <= 16 per-wavefront partials p[0], p[stride], ... read from
// LDS all at once (straight-line), added in a fixed order.
template <typename T>
__device__ inline T sum_waves(const T* p, int stride, int W) {
  T v[16];
#pragma unroll
  for (int w = 0; w < 16; ++w) v[w] = p[(w < W ? w : W - 1) * stride];  // in-bounds read, then mask
#pragma unroll
  for (int w = 0; w < 16; ++w) v[w] = w < W ? v[w] : T(0);
#pragma unroll
  for (int h = 8; h >= 1; h >>= 1)
#pragma unroll
    for (int w = 0; w < h; ++w) v[w] += v[w + h];
  return v[0];
}

// Workgroups of more than 32 KiB of LDS: the kernel's limit is raised once
// per kernel (the set of raised kernels is shared by all threads).
inline hipError_t allow_large_lds(const void* kern) {
  static std::mutex mu;
  static std::unordered_set<const void*> raised;
  std::lock_guard<std::mutex> lock(mu);
  if (raised.count(kern)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
  if (e == hipSuccess) raised.insert(kern);
  return e;
}

template <typename Kern>
inline hipError_t launch_one(Kern kern, const ProdPlan& p, const ProdArgs& a, hipStream_t st) {
  if (p.lds > 32768) {
    const hipError_t e = allow_large_lds((const void*)kern);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(p.nwg), dim3(64 * p.W), p.lds, st, a);
  return hipGetLastError();
}

// Every kernel instance the planner may choose.  One batch column: 8-word
// chunks for K <= 2, and for K <= 4 with Q >= 2 and no column scales, 4-word
// chunks otherwise; XM = 1 / 2 select the aligned bf16 / fp16 single-column
// activation path of the float kernel.  Several batch columns: 4-word
// chunks, generic activation path.
#define BSG_PROD_XM(X, Q, NWL, KM) X(Q, NWL, KM, 1, 0) X(Q, NWL, KM, 1, 1) X(Q, NWL, KM, 1, 2)
#define BSG_PROD_F_ONE_COLUMN(X)                                                                             \
  BSG_PROD_XM(X, 4, 2, 1) BSG_PROD_XM(X, 4, 2, 2) BSG_PROD_XM(X, 2, 4, 1) BSG_PROD_XM(X, 2, 4, 2)            \
  BSG_PROD_XM(X, 1, 8, 1) BSG_PROD_XM(X, 1, 8, 2) BSG_PROD_XM(X, 4, 2, 3) BSG_PROD_XM(X, 4, 2, 4)            \
  BSG_PROD_XM(X, 4, 1, 8) BSG_PROD_XM(X, 2, 4, 3) BSG_PROD_XM(X, 2, 4, 4) BSG_PROD_XM(X, 2, 2, 8)            \
  BSG_PROD_XM(X, 1, 4, 3) BSG_PROD_XM(X, 1, 4, 4) BSG_PROD_XM(X, 1, 4, 8) BSG_PROD_XM(X, 4, 1, 3)            \
  BSG_PROD_XM(X, 4, 1, 4) BSG_PROD_XM(X, 2, 2, 3) BSG_PROD_XM(X, 2, 2, 4)
#define BSG_PROD_F_INSTANCES(X) BSG_PROD_F_ONE_COLUMN(X) BSG_PROD_MULTI_B(X, 2) BSG_PROD_I8_MULTI_B(X, 4)
#define BSG_PROD_I8_INSTANCES(X)                                                                       \
  X(4, 2, 1, 1, 0) X(4, 2, 2, 1, 0) X(2, 4, 1, 1, 0) X(2, 4, 2, 1, 0) X(1, 8, 1, 1, 0) X(1, 8, 2, 1, 0) \
  X(4, 1, 3, 1, 0) X(4, 1, 4, 1, 0) X(4, 1, 8, 1, 0) X(2, 2, 3, 1, 0) X(2, 2, 4, 1, 0) X(2, 2, 8, 1, 0) \
  X(1, 4, 3, 1, 0) X(1, 4, 4, 1, 0) X(1, 4, 8, 1, 0) BSG_PROD_I8_MULTI_B(X, 2) BSG_PROD_I8_MULTI_B(X, 4)
// Several batch columns with K <= 4 (float: K > 4 takes at most two batch
// columns per launch; int8: one, as 8 plane counters per base and column
// would not fit in registers)
#define BSG_PROD_I8_MULTI_B(X, BB)                                                                     \
  X(4, 1, 1, BB, 0) X(4, 1, 2, BB, 0) X(4, 1, 3, BB, 0) X(4, 1, 4, BB, 0)                              \
  X(2, 2, 1, BB, 0) X(2, 2, 2, BB, 0) X(2, 2, 3, BB, 0) X(2, 2, 4, BB, 0)                              \
  X(1, 4, 1, BB, 0) X(1, 4, 2, BB, 0) X(1, 4, 3, BB, 0) X(1, 4, 4, BB, 0)
#define BSG_PROD_MULTI_B(X, BB)                                                                        \
  X(4, 1, 1, BB, 0) X(4, 1, 2, BB, 0) X(4, 1, 3, BB, 0) X(4, 1, 4, BB, 0) X(4, 1, 8, BB, 0)            \
  X(2, 2, 1, BB, 0) X(2, 2, 2, BB, 0) X(2, 2, 3, BB, 0) X(2, 2, 4, BB, 0) X(2, 2, 8, BB, 0)            \
  X(1, 4, 1, BB, 0) X(1, 4, 2, BB, 0) X(1, 4, 3, BB, 0) X(1, 4, 4, BB, 0) X(1, 4, 8, BB, 0)

constexpr int prod_key(int Q, int NWL, int KM, int BB, int XM) {
  return (((Q * 16 + NWL) * 16 + KM) * 16 + BB) * 4 + XM;
}

}  // namespace bsg
