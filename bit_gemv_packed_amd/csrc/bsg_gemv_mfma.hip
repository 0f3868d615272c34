// Planner and dispatch of the batched sign product on the matrix cores
// (kernel in bsg_prod_mfma.h).
#include <algorithm>
#include <cstdlib>

#include "bsg_prod_mfma.h"

namespace bsg {

// ------------------------------------------------------------------ planning

bool mfma_eligible(int B, int xdt, bool colscale) {
  return B >= 4 && !colscale && (xdt == BSG_BF16 || xdt == BSG_F16);
}

// Instances with column or group scales (bsg_gemv_mfma_cg.hip), and the
// one-base instances of the batched low-rank expansion (bsg_gemv_mfma_ex.hip).
hipError_t dispatch_mfma_cg(const ProdArgs& a, int RT, int KM, int XT, int VW, int CG, const ProdPlan& p,
                            hipStream_t st);
hipError_t dispatch_mfma_ex(const ProdArgs& a, int RT, int XT, int VW, int EX, const ProdPlan& p, hipStream_t st);

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

// Column scales (fp16 x only: the A values are the scales' own fp16 bits)
// and group-wise row scales (g >= 128, M % 4 == 0: four rows' scales in one
// 8-byte load) on the matrix cores: 4- or 8-value x loads.
bool mfma_cg_ok(int B, int xdt, const void* x, bool colscale, int gsw, int M) {
  if (B < 4 || (xdt != BSG_BF16 && xdt != BSG_F16) || mfma_vw(B, x) < 4) return false;
  if (colscale && xdt != BSG_F16) return false;
  if (gsw && (gsw < 4 || M % 4 != 0)) return false;
  return true;
}

// One launch per 16 batch columns and per group of up to 4 bases (2 with
// 2-byte x loads; later groups accumulate).  Row tiles per workgroup: 2 when
// one would give more than 256 workgroups (x is then read once per 32
// rows, in one round of workgroups where M < 8192: at B = 16, 5120 x 5120,
// K = 3 takes 12.6 against 17.0 us, 6144 x 4096 9.3 against 12.2 us), else
// 1 (4096 x 4096: 7.4 against 9.3 us).  Wavefronts: up to mfma_max_waves, each taking whole
// 4-step layout tiles.  With a0.np > 1 every launch covers the row tiles of
// all projections a0.proj[0 .. np) in turn (4- or 8-value x loads only).
hipError_t launch_prod_mfma(const ProdArgs& a0, hipStream_t st) {
  const int T4 = (a0.ND + 3) / 4;      // 4-step layout tiles
  const int XT = a0.xdt == BSG_BF16 ? 1 : 2;
  const int VW = mfma_vw(a0.B, a0.x);
  const bool multi = a0.np > 1;
  const int CG = (a0.colscale ? 1 : 0) | (a0.gsw ? 2 : 0);
  const int EX = (a0.x2 ? 1 : 0) | (a0.split_hi ? 2 : 0);
  if (multi && VW < 4) return hipErrorInvalidConfiguration;
  if (EX && (multi || CG || a0.K != 1)) return hipErrorInvalidConfiguration;
  if (CG && (multi || !mfma_cg_ok(a0.B, a0.xdt, a0.x, a0.colscale != nullptr, a0.gsw, a0.M)))
    return hipErrorInvalidConfiguration;
  int mt = a0.M;
  if (multi) {
    mt = 0;
    for (int i = 0; i < a0.np; ++i) mt += a0.proj[i].M;
  }
  const int RT = VW == 1 ? 1 : mf_env("BSG_MF_RT", (mt + 15) / 16 > 256 ? 2 : 1) >= 2 ? 2 : 1;
  const int KG = VW == 1 ? 2 : 4;      // bases per launch
  int nwg = (a0.M + 16 * RT - 1) / (16 * RT);
  if (multi) {
    nwg = 0;
    for (int i = 0; i < a0.np; ++i) nwg += (a0.proj[i].M + 16 * RT - 1) / (16 * RT);
  }
  for (int k0 = 0; k0 < a0.K; k0 += KG) {
    const int KM = a0.K - k0 < KG ? a0.K - k0 : KG;
    const int wmax = std::min(mfma_max_waves(RT, KM, VW, CG), mf_env("BSG_MF_W", 16));
    int W = T4 < wmax ? T4 : wmax;
    const int per = (T4 + W - 1) / W;  // tiles per wavefront
    W = (T4 + per - 1) / per;
    const size_t lds = (size_t)W * mfma_wave_lds(KM, CG) + (size_t)W * RT * 256 * 4;
    ProdArgs as = a0;
    as.bits = a0.bits + (size_t)k0 * a0.plane;
    as.K = KM;
    as.accumulate = k0 > 0 ? 1 : a0.accumulate;
    as.x_bytes = (uint32_t)((size_t)a0.N * a0.B * 2);
    if (CG & 2) {  // fp16 group scales [K][ngrp][M]
      as.alpha = (const float*)(const void*)((const uint16_t*)(const void*)a0.alpha + (size_t)k0 * a0.ngrp * a0.M);
      as.al_bytes = (uint32_t)((size_t)KM * a0.ngrp * a0.M * 2);
    } else {
      as.alpha = a0.alpha ? a0.alpha + (size_t)k0 * a0.M : nullptr;
      as.al_bytes = a0.alpha ? (uint32_t)((size_t)KM * a0.M * 4) : 0u;
    }
    as.colscale = a0.colscale ? a0.colscale + (size_t)k0 * a0.N : nullptr;
    as.cs_bytes = a0.colscale ? (uint32_t)((size_t)KM * a0.N * 2) : 0u;
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
      hipError_t e;
      if (CG || EX) {
        ProdPlan p{};
        p.nwg = nwg;
        p.W = W;
        p.lds = lds;
        e = CG ? dispatch_mfma_cg(a, RT, KM, XT, VW, CG, p, st) : dispatch_mfma_ex(a, RT, XT, VW, EX, p, st);
      } else {
        e = dispatch_mfma(a, RT, KM, XT, VW, nwg, W, lds, st);
      }
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace bsg
