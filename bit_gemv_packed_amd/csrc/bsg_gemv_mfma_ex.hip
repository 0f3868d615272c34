// One-base instances of the batched matrix-core product for the low-rank
// expansion of bsg_linear and binlr_apply (bsg_prod_mfma.h, EX): z' = V x
// written as the bf16 halves of alpha_r (.) z' (EX = 2), and U times the
// sum of the two halves in one launch (EX = 1).
#include "bsg_prod_mfma.h"

namespace bsg {

hipError_t dispatch_mfma_ex(const ProdArgs& a, int RT, int XT, int VW, int EX, const ProdPlan& p, hipStream_t st) {
  const int key = ((RT * 4 + XT) * 16 + VW) * 4 + EX;
  switch (key) {
#define BSG_MF(RT_, XT_, VW_, EX_)           \
  case ((RT_ * 4 + XT_) * 16 + VW_) * 4 + EX_: \
    return launch_one(k_prod_mfma<RT_, 1, XT_, VW_, 0, 0, EX_>, p, a, st);
#define BSG_MF_VW(RT_, XT_, EX_) BSG_MF(RT_, XT_, 2, EX_) BSG_MF(RT_, XT_, 4, EX_) BSG_MF(RT_, XT_, 8, EX_)
#define BSG_MF_XT(RT_, EX_) BSG_MF_VW(RT_, 1, EX_) BSG_MF_VW(RT_, 2, EX_)
    BSG_MF_XT(1, 1) BSG_MF_XT(2, 1) BSG_MF_XT(1, 2) BSG_MF_XT(2, 2)
    // 2-byte x loads: one row tile
    BSG_MF(1, 1, 1, 1) BSG_MF(1, 2, 1, 1) BSG_MF(1, 1, 1, 2) BSG_MF(1, 2, 1, 2)
#undef BSG_MF_XT
#undef BSG_MF_VW
#undef BSG_MF
    default: return hipErrorInvalidConfiguration;
  }
}

}  // namespace bsg
