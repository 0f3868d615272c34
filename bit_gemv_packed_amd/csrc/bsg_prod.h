// Device helpers shared by the float and int8 sign-product kernels, and the
// set of kernel instances the launch planner may choose.
#pragma once

#include "bsg_internal.h"

#include <atomic>

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

// Sign words of one chunk: NWL consecutive logical words [w0, w0 + NWL) of
// row m for every base k < K (w0 is a multiple of min(NWL, 4)).
//
// load_chunk_full: every word of the chunk lies in a complete 4-word layout
// tile (the caller checks this once per wavefront); straight-line 4/8/16-byte
// loads, all in flight together.  m must be a valid row (callers clamp rows
// beyond M to M-1 and discard their sums).
template <int KM, int NWL>
__device__ inline void load_chunk_full(const ProdArgs& a, int m, int w0, uint32_t (&wd)[KM][NWL]) {
  const int rb = m >> 6, rt = m & 63;
  const int h = min(64, a.M - rb * 64);
  constexpr int PW = NWL < 4 ? NWL : 4;  // words per load
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (base_active<KM>(a, k)) {
      const uint32_t* base = a.bits + (size_t)k * a.plane + (size_t)rb * 64 * a.ND;
#pragma unroll
      for (int g = 0; g < NWL / PW; ++g) {
        const int wf = w0 + g * PW;
        const uint32_t* p = base + (size_t)(wf >> 2) * 4 * h + rt * 4 + (wf & 3);
        if (PW == 4) {
          const uint4 v = *(const uint4*)p;
          wd[k][g * 4 + 0] = v.x;
          wd[k][g * 4 + 1] = v.y;
          wd[k][g * 4 + 2] = v.z;
          wd[k][g * 4 + 3] = v.w;
        } else if (PW == 2) {
          const uint2 v = *(const uint2*)p;
          wd[k][g * 2 + 0] = v.x;
          wd[k][g * 2 + 1] = v.y;
        } else {
          wd[k][g] = p[0];
        }
      }
    }
  }
}

// load_chunk_any: the last, ragged chunk; one guarded load per word, words at
// or beyond ND read as 0 (their lookups are skipped).
template <int KM, int NWL>
__device__ inline void load_chunk_any(const ProdArgs& a, int m, int w0, uint32_t (&wd)[KM][NWL]) {
  const int rb = m >> 6, rt = m & 63;
  const int h = min(64, a.M - rb * 64);
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (base_active<KM>(a, k)) {
      const uint32_t* base = a.bits + (size_t)k * a.plane + (size_t)rb * 64 * a.ND;
#pragma unroll
      for (int j = 0; j < NWL; ++j) {
        const int w = w0 + j;
        const int g4 = w >> 2;
        const int wg = min(4, a.ND - 4 * g4);
        wd[k][j] = w < a.ND ? base[(size_t)g4 * 4 * h + rt * wg + (w & 3)] : 0u;
      }
    }
  }
}

// Loads the sign words of chunk [cw0, cw0 + CW) for this lane (quarter q);
// `full` must be uniform across the wavefront.
template <int KM, int NWL>
__device__ inline void load_chunk(const ProdArgs& a, bool full, int m, int w0, uint32_t (&wd)[KM][NWL]) {
  if (full)
    load_chunk_full<KM, NWL>(a, m, w0, wd);
  else
    load_chunk_any<KM, NWL>(a, m, w0, wd);
}

template <typename Kern>
inline hipError_t launch_one(Kern kern, const ProdPlan& p, const ProdArgs& a, hipStream_t st) {
  static std::atomic<int> raised{0};
  if (p.lds > 65536 && !raised.load(std::memory_order_relaxed)) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    if (e != hipSuccess) return e;
    raised.store(1, std::memory_order_relaxed);
  }
  hipLaunchKernelGGL(kern, dim3(p.nwg), dim3(64 * p.W), p.lds, st, a);
  return hipGetLastError();
}

// Every kernel instance the planner may choose.  One batch column: 8-word
// chunks for K <= 2, 4-word chunks otherwise; XM = 1 / 2 select the aligned
// bf16 / fp16 single-column activation path of the float kernel.  Several
// batch columns: 4-word chunks, generic activation path.
#define BSG_PROD_XM(X, Q, NWL, KM) X(Q, NWL, KM, 1, 0) X(Q, NWL, KM, 1, 1) X(Q, NWL, KM, 1, 2)
#define BSG_PROD_F_INSTANCES(X)                                                                              \
  BSG_PROD_XM(X, 4, 2, 1) BSG_PROD_XM(X, 4, 2, 2) BSG_PROD_XM(X, 2, 4, 1) BSG_PROD_XM(X, 2, 4, 2)            \
  BSG_PROD_XM(X, 1, 8, 1) BSG_PROD_XM(X, 1, 8, 2) BSG_PROD_XM(X, 4, 1, 3) BSG_PROD_XM(X, 4, 1, 4)            \
  BSG_PROD_XM(X, 4, 1, 8) BSG_PROD_XM(X, 2, 2, 3) BSG_PROD_XM(X, 2, 2, 4) BSG_PROD_XM(X, 2, 2, 8)            \
  BSG_PROD_XM(X, 1, 4, 3) BSG_PROD_XM(X, 1, 4, 4) BSG_PROD_XM(X, 1, 4, 8) BSG_PROD_MULTI_B(X, 2)             \
  BSG_PROD_MULTI_B(X, 4)
#define BSG_PROD_I8_INSTANCES(X)                                                                       \
  X(4, 2, 1, 1, 0) X(4, 2, 2, 1, 0) X(2, 4, 1, 1, 0) X(2, 4, 2, 1, 0) X(1, 8, 1, 1, 0) X(1, 8, 2, 1, 0) \
  X(4, 1, 3, 1, 0) X(4, 1, 4, 1, 0) X(4, 1, 8, 1, 0) X(2, 2, 3, 1, 0) X(2, 2, 4, 1, 0) X(2, 2, 8, 1, 0) \
  X(1, 4, 3, 1, 0) X(1, 4, 4, 1, 0) X(1, 4, 8, 1, 0) BSG_PROD_MULTI_B(X, 2) BSG_PROD_MULTI_B(X, 4)
#define BSG_PROD_MULTI_B(X, BB)                                                                        \
  X(4, 1, 1, BB, 0) X(4, 1, 2, BB, 0) X(4, 1, 3, BB, 0) X(4, 1, 4, BB, 0) X(4, 1, 8, BB, 0)            \
  X(2, 2, 1, BB, 0) X(2, 2, 2, BB, 0) X(2, 2, 3, BB, 0) X(2, 2, 4, BB, 0) X(2, 2, 8, BB, 0)            \
  X(1, 4, 1, BB, 0) X(1, 4, 2, BB, 0) X(1, 4, 3, BB, 0) X(1, 4, 4, BB, 0) X(1, 4, 8, BB, 0)

constexpr int prod_key(int Q, int NWL, int KM, int BB, int XM) {
  return (((Q * 16 + NWL) * 16 + KM) * 16 + BB) * 4 + XM;
}

}  // namespace bsg
