// MFMA-bound GEMM instantiations: W4A8 layers (two's complement int4 in QUAD order, group
// scales) on the 16-bit path, with the e4m3 activations widened to bf16 beforehand and the
// per-token scale applied in the epilogue.
#include "qg_mfma_kernel.h"

namespace qg {

bool mfma_int4q(const MfmaArgs& a, const MfmaTile& t, int wp, int af, int of, int stype, bool zero, bool moe,
                hipStream_t st) {
  if (wp != WP_INT4Q_MAGIC || af != A_BF16 || zero) return false;
  if (of == O_BF16 && stype == S_BF16) return launch_mfma_variant<WP_INT4Q_MAGIC, A_BF16, O_BF16, S_BF16, false>(a, t, moe, st);
  if (of == O_F16 && stype == S_F16) return launch_mfma_variant<WP_INT4Q_MAGIC, A_BF16, O_F16, S_F16, false>(a, t, moe, st);
  return false;
}

}  // namespace qg
