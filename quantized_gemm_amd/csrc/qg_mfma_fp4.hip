// MFMA-bound GEMM instantiations: e2m1 weights with UE8M0 block scales.
#include "qg_mfma_kernel.h"

namespace qg {

bool mfma_fp4(const MfmaArgs& a, const MfmaTile& t, int wp, int af, int of, int stype, bool zero, bool moe,
              hipStream_t st) {
  if (wp == WP_FP4 && af == A_BF16 && of == O_BF16 && stype == S_UE8M0 && zero == false)
    return launch_mfma_variant<WP_FP4, A_BF16, O_BF16, S_UE8M0, false>(a, t, moe, st);
  if (wp == WP_FP4 && af == A_F16 && of == O_F16 && stype == S_UE8M0 && zero == false)
    return launch_mfma_variant<WP_FP4, A_F16, O_F16, S_UE8M0, false>(a, t, moe, st);
  // e4m3 activations (W4A8 MXFP4): scaled fp8 x fp4 MFMAs
  if (wp == WP_FP4 && af == A_FP8 && of == O_BF16 && stype == S_UE8M0 && zero == false)
    return launch_mfma_variant<WP_FP4, A_FP8, O_BF16, S_UE8M0, false>(a, t, moe, st);
  if (wp == WP_FP4 && af == A_FP8 && of == O_F16 && stype == S_UE8M0 && zero == false)
    return launch_mfma_variant<WP_FP4, A_FP8, O_F16, S_UE8M0, false>(a, t, moe, st);
  // e2m1 activations (W4A4 MXFP4): scaled fp4 x fp4 MFMAs
  if (wp == WP_FP4 && af == A_FP4 && of == O_BF16 && stype == S_UE8M0 && zero == false)
    return launch_mfma_variant<WP_FP4, A_FP4, O_BF16, S_UE8M0, false>(a, t, moe, st);
  if (wp == WP_FP4 && af == A_FP4 && of == O_F16 && stype == S_UE8M0 && zero == false)
    return launch_mfma_variant<WP_FP4, A_FP4, O_F16, S_UE8M0, false>(a, t, moe, st);
  return false;
}

}  // namespace qg
