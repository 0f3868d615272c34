// Instances of the batched matrix-core product (bsg_prod_mfma.h) with fp16
// column scales (fp16 x) and / or group-wise fp16 row scales (FluxBin Sec.
// 3.1: decoupled row and column scales, one row scale per group of columns).
#include "bsg_prod_mfma.h"

namespace bsg {

hipError_t dispatch_mfma_cg(const ProdArgs& a, int RT, int KM, int XT, int VW, int CG, const ProdPlan& p,
                            hipStream_t st) {
  const int key = (((RT * 8 + KM) * 4 + XT) * 16 + VW) * 4 + CG;
  switch (key) {
#define BSG_MF(RT_, KM_, XT_, VW_, CG_)                  \
  case (((RT_ * 8 + KM_) * 4 + XT_) * 16 + VW_) * 4 + CG_: \
    return launch_one(k_prod_mfma<RT_, KM_, XT_, VW_, 0, CG_>, p, a, st);
#define BSG_MF_VW(RT_, KM_, XT_, CG_) BSG_MF(RT_, KM_, XT_, 4, CG_) BSG_MF(RT_, KM_, XT_, 8, CG_)
#define BSG_MF_K(RT_, XT_, CG_) \
  BSG_MF_VW(RT_, 1, XT_, CG_) BSG_MF_VW(RT_, 2, XT_, CG_) BSG_MF_VW(RT_, 3, XT_, CG_) BSG_MF_VW(RT_, 4, XT_, CG_)
#define BSG_MF_RT(XT_, CG_) BSG_MF_K(1, XT_, CG_) BSG_MF_K(2, XT_, CG_)
    // column scales: fp16 x only; group scales: bf16 or fp16 x
    BSG_MF_RT(2, 1) BSG_MF_RT(1, 2) BSG_MF_RT(2, 2) BSG_MF_RT(2, 3)
#undef BSG_MF_RT
#undef BSG_MF_K
#undef BSG_MF_VW
#undef BSG_MF
    default: return hipErrorInvalidConfiguration;
  }
}

}  // namespace bsg
