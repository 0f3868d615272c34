// Binary-base product with group-wise row scales (FluxBin Sec. 3.1: one row
// scale per weight group; g = 128 in its Kb-g128 configurations; App. C.2:
// scales stored in fp16), optionally with the salient-column bases of its
// hybrid configurations read through the Virtual Columnar Mapping (Sec. 3.2):
//
//   y[m,b] (= or +=) sum_k sum_j alpha_k[m][j] sum_{n in group j} (2 bit_k(m,n) - 1) c_k[n] x[n,b]
//                  + sum_k sum_j salpha_k[m][j] sum_{i < s} (2 sbit_k(m, js+i) - 1) sc_k[js+i] x[idx[js+i],b]
//
// The table kernel of bsg_prod_f.h with GS = 1: every lane sums its words of
// a chunk apart (they lie in one group) and adds that sum times its group's
// scale; the salient chunks follow the main ones.  One batch column per
// launch.
#include "bsg_prod_f.h"

namespace bsg {

// Every (Q, NWL, KM) the grouped planner may choose (K <= 4, one batch
// column, NWL <= the words of a group).
#define BSG_PROD_GS_INSTANCES(X)                                                                              \
  BSG_PROD_XM(X, 4, 2, 1) BSG_PROD_XM(X, 4, 2, 2) BSG_PROD_XM(X, 2, 4, 1) BSG_PROD_XM(X, 2, 4, 2)            \
  BSG_PROD_XM(X, 1, 8, 1) BSG_PROD_XM(X, 1, 8, 2) BSG_PROD_XM(X, 4, 2, 3) BSG_PROD_XM(X, 4, 2, 4)            \
  BSG_PROD_XM(X, 2, 4, 3) BSG_PROD_XM(X, 2, 4, 4) BSG_PROD_XM(X, 4, 1, 3) BSG_PROD_XM(X, 4, 1, 4)            \
  BSG_PROD_XM(X, 2, 2, 3) BSG_PROD_XM(X, 2, 2, 4) BSG_PROD_XM(X, 1, 4, 3) BSG_PROD_XM(X, 1, 4, 4)

// GS = 2: with the salient-column bases; np > 1: fused projections (MP = 1)
static hipError_t dispatch_gs(const ProdArgs& a, const ProdPlan& p, hipStream_t st) {
  const bool sal = a.vs_bits != nullptr;
  if (a.np > 1) {
    if (sal) return hipErrorInvalidConfiguration;
    switch (prod_key(p.Q, p.NWL, p.KM, p.BB, p.XM)) {
#define BSG_CASE(Q, NWL, KM, BB, XM) \
  case prod_key(Q, NWL, KM, BB, XM): return launch_one(k_prod_f<Q, NWL, KM, BB, XM, 1, 1>, p, a, st);
      BSG_PROD_GS_INSTANCES(BSG_CASE)
#undef BSG_CASE
      default: return hipErrorInvalidConfiguration;
    }
  }
  switch (prod_key(p.Q, p.NWL, p.KM, p.BB, p.XM)) {
#define BSG_CASE(Q, NWL, KM, BB, XM)                                                           \
  case prod_key(Q, NWL, KM, BB, XM):                                                           \
    return sal ? launch_one(k_prod_f<Q, NWL, KM, BB, XM, 0, 2>, p, a, st)                      \
               : launch_one(k_prod_f<Q, NWL, KM, BB, XM, 0, 1>, p, a, st);
    BSG_PROD_GS_INSTANCES(BSG_CASE)
#undef BSG_CASE
    default: return hipErrorInvalidConfiguration;
  }
}

hipError_t launch_prod_grouped(const ProdArgs& a0, hipStream_t st) {
  const bool multi = a0.np > 1;
  int mt = a0.M;
  if (multi) {
    mt = 0;
    for (int i = 0; i < a0.np; ++i) mt += a0.proj[i].M;
  }
  // the tables per wavefront depend on the column scales (one set per base)
  const bool cs = multi ? a0.proj[0].colscale != nullptr : a0.colscale != nullptr;
  ProdPlan p = plan_prod(a0.K, mt, a0.N, a0.B, cs, false, a0.gsw);
  if (p.KM > 4 || p.BB != 1 || (multi && a0.B != 1)) return hipErrorInvalidConfiguration;
  ProdArgs as = a0;
  if (multi) {
    // every projection's row blocks in one grid; the kernel prologue reads
    // the first projection's operands before it switches to its own
    int wg = 0;
    for (int i = 0; i < as.np; ++i) {
      ProjDesc& d = as.proj[i];
      d.plane = plane_words(d.M, as.ND);
      d.wg0 = wg;
      d.al_bytes = (uint32_t)((size_t)as.K * as.ngrp * d.M * 2);
      d.cs_bytes = d.colscale ? (uint32_t)((size_t)as.K * as.N * 2) : 0u;
      wg += (d.M + p.RW - 1) / p.RW;
    }
    p.nwg = wg;
    as.bits = as.proj[0].bits;
    as.alpha = as.proj[0].alpha;
    as.colscale = as.proj[0].colscale;
    as.y = as.proj[0].y;
    as.plane = as.proj[0].plane;
    as.M = as.proj[0].M;
  }
  as.x_bytes = (uint32_t)((size_t)a0.N * a0.B * (a0.xdt == BSG_F32 ? 4 : 2));
  as.cs_bytes = as.colscale ? (uint32_t)((size_t)a0.K * a0.N * 2) : 0u;
  as.al_bytes = (uint32_t)((size_t)as.K * as.M * as.ngrp * 2);
  p.XM = (a0.B == 1 && a0.xvec && a0.xdt != BSG_F32) ? (a0.xdt == BSG_BF16 ? 1 : 2) : 0;
  // the instance for this XM may allow fewer wavefronts than the plan took
  const int wmax = prod_max_waves(p.KM, p.BB, a0.vs_bits ? 2 : 1, p.XM);
  if (p.W > wmax) {
    const int T = (a0.ND + p.CW - 1) / p.CW;
    const size_t per_wave = p.lds / p.W;
    p.NCH = (T + wmax - 1) / wmax;
    p.W = (T + p.NCH - 1) / p.NCH;  // no wavefront without chunks
    p.lds = per_wave * p.W;
  }
  for (int c = 0; c < p.nlaunch; ++c) {
    ProdArgs a = as;
    a.b0 = c;
    a.W = p.W;
    a.NCH = p.NCH;
    a.wave_lds = (uint32_t)p.wave_lds;
    const hipError_t e = dispatch_gs(a, p, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bsg
