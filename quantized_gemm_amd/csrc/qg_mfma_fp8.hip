// MFMA-bound GEMM instantiations: e4m3 weights with e4m3 activations.
#include "qg_mfma_kernel.h"

namespace qg {

bool mfma_fp8(const MfmaArgs& a, const MfmaTile& t, int wp, int af, int of, int stype, bool zero, bool moe,
              hipStream_t st) {
  if (wp == WP_FP8 && af == A_FP8 && of == O_BF16 && stype == S_F32 && zero == false)
    return launch_mfma_variant<WP_FP8, A_FP8, O_BF16, S_F32, false>(a, t, moe, st);
  if (wp == WP_FP8 && af == A_FP8 && of == O_F16 && stype == S_F32 && zero == false)
    return launch_mfma_variant<WP_FP8, A_FP8, O_F16, S_F32, false>(a, t, moe, st);
  return false;
}

}  // namespace qg
