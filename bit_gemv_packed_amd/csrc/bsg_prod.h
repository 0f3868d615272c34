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

// Loads NWL consecutive logical words [w0, w0 + NWL) of row m, base k, from
// the device layout (w0 is a multiple of min(NWL, 4)).  Words at or beyond ND
// read as 0; callers never use them.
template <int NWL>
__device__ inline void load_row_words(const ProdArgs& a, int k, int m, int w0, uint32_t* out) {
  const int rb = m >> 6, rt = m & 63;
  const int h = min(64, a.M - rb * 64);
  const uint32_t* base = a.bits + (size_t)k * a.plane + (size_t)rb * 64 * a.ND;
  constexpr int PW = NWL < 4 ? NWL : 4;  // words per piece
#pragma unroll
  for (int g = 0; g < NWL / PW; ++g) {
    const int wf = w0 + g * PW;
    const int g4 = wf >> 2;
    const int j0 = wf & 3;
    const int wg = min(4, a.ND - 4 * g4);  // words in this layout tile
    const uint32_t* tile = base + (size_t)g4 * 4 * h;
    if (wf < a.ND && wg == 4) {
      const uint32_t* p = tile + rt * 4 + j0;
      if (PW == 4) {
        const uint4 v = *(const uint4*)p;
        out[g * 4 + 0] = v.x;
        out[g * 4 + 1] = v.y;
        out[g * 4 + 2] = v.z;
        out[g * 4 + 3] = v.w;
      } else if (PW == 2) {
        const uint2 v = *(const uint2*)p;
        out[g * PW + 0] = v.x;
        out[g * PW + 1] = v.y;
      } else {
        out[g * PW] = p[0];
      }
    } else {
#pragma unroll
      for (int j = 0; j < PW; ++j) {
        const int jj = j0 + j;
        out[g * PW + j] = (wf + j < a.ND && jj < wg) ? tile[rt * wg + jj] : 0u;
      }
    }
  }
}

template <int KM, int NWL>
__device__ inline void load_chunk(const ProdArgs& a, bool valid, int m, int w0, uint32_t (&wd)[KM][NWL]) {
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (k < a.K && valid) load_row_words<NWL>(a, k, m, w0, wd[k]);
  }
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

// Every (Q, NWL, KM, BB) the planner may choose: BB = 1 with 8-word chunks
// (KM <= 4, at most 2 table sets) or 4-word chunks, and BB = 2, 4 with
// 4-word chunks.
#define BSG_PROD_INSTANCES(X)                                                          \
  X(4, 2, 2, 1) X(4, 2, 4, 1) X(2, 4, 2, 1) X(2, 4, 4, 1) X(1, 8, 2, 1) X(1, 8, 4, 1) \
  X(4, 1, 4, 1) X(4, 1, 8, 1) X(2, 2, 4, 1) X(2, 2, 8, 1) X(1, 4, 4, 1) X(1, 4, 8, 1) \
  X(4, 1, 2, 2) X(4, 1, 4, 2) X(4, 1, 8, 2) X(2, 2, 2, 2) X(2, 2, 4, 2) X(2, 2, 8, 2) \
  X(1, 4, 2, 2) X(1, 4, 4, 2) X(1, 4, 8, 2)                                           \
  X(4, 1, 2, 4) X(4, 1, 4, 4) X(4, 1, 8, 4) X(2, 2, 2, 4) X(2, 2, 4, 4) X(2, 2, 8, 4) \
  X(1, 4, 2, 4) X(1, 4, 4, 4) X(1, 4, 8, 4)

constexpr int prod_key(int Q, int NWL, int KM, int BB) { return ((Q * 16 + NWL) * 16 + KM) * 16 + BB; }

}  // namespace bsg
