// Binary-base product for gfx950 (float activations): planning and launch of
// the table kernel of bsg_prod_f.h for single products and fused projections.
#include "bsg_prod_f.h"

#include <cstdlib>

namespace bsg {

// ------------------------------------------------------------------ planning

static int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  const int r = std::atoi(v);
  return r > 0 ? r : dflt;
}

ProdPlan plan_prod(int K, int M, int N, int B, bool colscale, bool i8, int gsw) {
  ProdPlan p{};
  const int ND = N / 32;
  p.KM = K <= 4 ? K : 8;
  p.BB = (B <= 1 || gsw > 0 || (i8 && p.KM == 8)) ? 1 : (B <= 2 || p.KM == 8) ? 2 : 4;
  p.nlaunch = (B + p.BB - 1) / p.BB;
  // Lanes per row: the fewest that still give at least 256 workgroups
  // (one per compute unit) -- except for very tall matrices (>= 256 row
  // blocks of 64), which run 2 lanes per row (measured fastest on
  // 28672 x 8192).
  // The int8 product at one batch column builds its bit planes once per
  // workgroup for all its rows, so it takes the fewest lanes that give 192
  // workgroups (measured: 14336 x 4096 at 1 lane per row, 224 workgroups,
  // 8.9 us against 11.6 us at 2 lanes; 4096 x 4096 best at 4 lanes).
  const int forceQ = env_int("BSG_Q", 0);
  const bool tall = M >= 64 * 256;
  const int minwg = (i8 && B == 1) ? 192 : 256;
  if (forceQ == 1 || forceQ == 2 || forceQ == 4) {
    p.Q = forceQ;
  } else if (tall && !(i8 && B == 1)) {
    p.Q = 2;
  } else {
    p.Q = 4;
    for (int qq = 1; qq <= 4; qq *= 2) {
      if ((M + 64 / qq - 1) / (64 / qq) >= minwg) {
        p.Q = qq;
        break;
      }
    }
    // 4 lanes per row with more than 256 workgroups (4096 < M < 8192): 2
    // lanes, one round of workgroups with 32 rows each, measured faster
    // than 16 rows in more than one round (5120 x 13824: 10.5 against
    // 11.6 us; 5120 x 5120, K = 3: 7.55 against 7.73 us)
    if (p.Q == 4 && !i8 && (M + 15) / 16 > 256) p.Q = 2;
  }
  p.RW = 64 / p.Q;
  const int KX = (colscale && !i8) ? K : 1;
  // 8-word chunks (256 columns) for one batch column and K <= 2, and for
  // K <= 4 with 2 or 4 lanes per row and one table set (no column scales);
  // 4-word chunks otherwise (smaller tables and register sets)
  p.CW = (p.BB == 1 && (p.KM <= 2 || (!i8 && p.KM <= 4 && p.Q >= 2 && KX == 1))) ? 8 : 4;
  // group-wise row scales: a lane's words must lie in one group of gsw words
  // (gsw and NWL are powers of two): more lanes per row where needed
  while (gsw > 0 && p.CW / p.Q > gsw && p.Q < 4) p.Q *= 2;
  p.RW = 64 / p.Q;
  p.NWL = p.CW / p.Q;
  p.wave_lds = i8 ? (size_t)p.CW * p.BB * 12 * 4 : (size_t)KX * p.BB * (p.NWL * 8) * (p.Q * 64 + 16);
  const int T = (ND + p.CW - 1) / p.CW;  // chunks
  int W = env_int("BSG_WAVES", 16);
  const int wmax = prod_max_waves(p.KM, p.BB, gsw > 0);
  W = W > wmax ? wmax : W;
  W = W > T ? T : W;
  const size_t red_per_wave = (size_t)p.RW * p.BB * 4 * (i8 ? p.KM : 1);
  while (W > 1 && (size_t)W * (p.wave_lds + red_per_wave) > kMaxLds) --W;
  p.W = W < 1 ? 1 : W;
  p.NCH = (T + p.W - 1) / p.W;
  // no wavefront without chunks: with T = 20 chunks, 10 wavefronts of 2
  // chunks measured 7.7 us against 11.5 us for 16 wavefronts of which 6 idle
  // (5120 x 5120, K = 3)
  p.W = (T + p.NCH - 1) / p.NCH;
  p.nwg = (M + p.RW - 1) / p.RW;
  // More workgroups than compute units, and so much LDS per workgroup that
  // only one fits on a compute unit: half the wavefronts (twice the chunks
  // each) let two share one, so the grid runs in half the rounds (14336 x
  // 4096 with column scales: 8.7 us against 10.1 us).
  const size_t per_wave = p.wave_lds + red_per_wave;
  if (p.nwg > 256 && p.W >= 2 && (size_t)p.W * per_wave > kMaxLds / 2 && !env_int("BSG_WAVES", 0)) {
    const int nch = (T + p.W / 2 - 1) / (p.W / 2);
    const int w2 = (T + nch - 1) / nch;
    if ((size_t)w2 * per_wave <= kMaxLds / 2) {
      p.NCH = nch;
      p.W = w2;
    }
  }
  p.lds = (size_t)p.W * per_wave;
  return p;
}

static hipError_t dispatch_f(const ProdArgs& a, const ProdPlan& p, hipStream_t st) {
  if (a.np > 1) {
    if (p.BB != 1) return hipErrorInvalidConfiguration;
    switch (prod_key(p.Q, p.NWL, p.KM, p.BB, p.XM)) {
#define BSG_CASE(Q, NWL, KM, BB, XM) \
  case prod_key(Q, NWL, KM, BB, XM): return launch_one(k_prod_f<Q, NWL, KM, BB, XM, 1>, p, a, st);
      BSG_PROD_F_ONE_COLUMN(BSG_CASE)
#undef BSG_CASE
      default: return hipErrorInvalidConfiguration;
    }
  }
  switch (prod_key(p.Q, p.NWL, p.KM, p.BB, p.XM)) {
#define BSG_CASE(Q, NWL, KM, BB, XM) \
  case prod_key(Q, NWL, KM, BB, XM): return launch_one(k_prod_f<Q, NWL, KM, BB, XM, 0>, p, a, st);
    BSG_PROD_F_INSTANCES(BSG_CASE)
#undef BSG_CASE
    default: return hipErrorInvalidConfiguration;
  }
}

// Fused launch over the projections a0.proj[0 .. a0.np) (same K, N, x and
// column-scale presence; one batch column): one grid, the row blocks of each
// projection in turn, planned for their total rows.
hipError_t launch_prod_multi(const ProdArgs& a0, hipStream_t st) {
  int mt = 0;
  for (int i = 0; i < a0.np; ++i) mt += a0.proj[i].M;
  ProdPlan p = plan_prod(a0.K, mt, a0.N, a0.B, a0.proj[0].colscale != nullptr, false);
  ProdArgs a = a0;
  int wg = 0;
  for (int i = 0; i < a.np; ++i) {
    ProjDesc& d = a.proj[i];
    d.plane = plane_words(d.M, a.ND);
    d.wg0 = wg;
    d.al_bytes = (uint32_t)((size_t)a.K * d.M * 4);
    d.cs_bytes = d.colscale ? (uint32_t)((size_t)a.K * a.N * 2) : 0u;
    wg += (d.M + p.RW - 1) / p.RW;
  }
  p.nwg = wg;
  // the kernel prologue reads these before it switches to its projection
  a.bits = a.proj[0].bits;
  a.alpha = a.proj[0].alpha;
  a.colscale = a.proj[0].colscale;
  a.y = a.proj[0].y;
  a.plane = a.proj[0].plane;
  a.M = a.proj[0].M;
  return launch_prod_f(a, p, st);
}

hipError_t launch_prod_f(const ProdArgs& a0, const ProdPlan& p0, hipStream_t st) {
  ProdPlan p = p0;
  ProdArgs as = a0;
  as.x_bytes = (uint32_t)((size_t)a0.N * a0.B * (a0.xdt == BSG_F32 ? 4 : 2));
  as.cs_bytes = a0.colscale ? (uint32_t)((size_t)a0.K * a0.N * 2) : 0u;
  as.al_bytes = a0.alpha ? (uint32_t)((size_t)a0.K * a0.M * 4) : 0u;
  p.XM = (a0.B == 1 && a0.xvec && a0.xdt != BSG_F32) ? (a0.xdt == BSG_BF16 ? 1 : 2) : 0;
  for (int c = 0; c < p.nlaunch; ++c) {
    ProdArgs a = as;
    a.b0 = c * p.BB;
    a.W = p.W;
    a.NCH = p.NCH;
    a.wave_lds = (uint32_t)p.wave_lds;
    const hipError_t e = dispatch_f(a, p, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bsg
