// MFMA-bound GEMM instantiations: int4 / uint4 weights with f16 / bf16 activations.
#include "qg_mfma_kernel.h"

namespace qg {

bool mfma_int4(const MfmaArgs& a, const MfmaTile& t, int wp, int af, int of, int stype, bool zero, bool moe,
               hipStream_t st) {
  if (wp == WP_INT4_MAGIC && af == A_F16 && of == O_F16 && stype == S_F16 && zero == false)
    return launch_mfma_variant<WP_INT4_MAGIC, A_F16, O_F16, S_F16, false>(a, t, moe, st);
  if (wp == WP_INT4_MAGIC && af == A_BF16 && of == O_BF16 && stype == S_BF16 && zero == false)
    return launch_mfma_variant<WP_INT4_MAGIC, A_BF16, O_BF16, S_BF16, false>(a, t, moe, st);
  if (wp == WP_INT4_MAGIC && af == A_BF16 && of == O_BF16 && stype == S_BF16 && zero == true)
    return launch_mfma_variant<WP_INT4_MAGIC, A_BF16, O_BF16, S_BF16, true>(a, t, moe, st);
  if (wp == WP_INT4_MAGIC && af == A_F16 && of == O_F16 && stype == S_F16 && zero == true)
    return launch_mfma_variant<WP_INT4_MAGIC, A_F16, O_F16, S_F16, true>(a, t, moe, st);
  return false;
}

}  // namespace qg
