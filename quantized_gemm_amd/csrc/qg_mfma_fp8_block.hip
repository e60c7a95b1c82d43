// MFMA-bound GEMM instantiations: block-scaled W8A8, e4m3 weights with one float32 scale per
// 128 x 128 block of (output channel, K) and e4m3 activations with one float32 scale per
// (row, 128-wide K group) ("Humming" wiki article, "Quantization representation": block scales
// share one scale across both matrix dimensions).  Neither scale is a power of two, so the
// matrix cores' block exponents cannot carry them: the MFMA kernel computes each 128-wide K
// step's product from zero and promotes it, acc += (sa[row, step] * sw[n / 128, step]) * P
// (its BLK path).  Split-K partials are scaled already; the reduction only adds them.
#include "qg_mfma_kernel.h"

namespace qg {

bool mfma_fp8_block(const MfmaArgs& a, const MfmaTile& t, int wp, int af, int of, int stype, bool zero, bool moe,
                    hipStream_t st) {
  if (wp != WP_FP8_BLOCK || af != A_FP8 || stype != S_F32 || zero) return false;
  if (of == O_BF16) return launch_mfma_variant<WP_FP8_BLOCK, A_FP8, O_BF16, S_F32, false>(a, t, moe, st);
  if (of == O_F16) return launch_mfma_variant<WP_FP8_BLOCK, A_FP8, O_F16, S_F32, false>(a, t, moe, st);
  return false;
}

}  // namespace qg
