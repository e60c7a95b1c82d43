// MFMA-bound GEMM instantiations: W4A8 layers, two's complement int4 weights (QUAD nibble
// order) with bf16 / f16 group scales, converted to e4m3 inside the kernel and multiplied
// with e4m3 activations on the fp8 MFMAs; each 128-wide K step is one scale group, its
// products promoted by the group scale, and the per-token activation scale is applied in
// the epilogue (or the split-K reduction).
//
// "Humming: Fast, Flexible Kernels for Quantized Inference", the W4A8 paragraph on GPUs
// without native FP4, and "Ant Group's Humming ...", *Coverage reaches beyond standard PTX
// types*: 4-bit weights are stored as such and converted inside the kernel into the
// format the matrix cores multiply; every int4 value is an e4m3 value, so the conversion
// is exact.
#include "qg_mfma_kernel.h"

namespace qg {

bool mfma_w4a8(const MfmaArgs& a, const MfmaTile& t, int wp, int af, int of, int stype, bool zero, bool moe,
               hipStream_t st) {
  if (wp != WP_INT4Q_FP8 || af != A_FP8 || zero) return false;
  if (of == O_BF16 && stype == S_BF16) return launch_mfma_variant<WP_INT4Q_FP8, A_FP8, O_BF16, S_BF16, false>(a, t, moe, st);
  if (of == O_F16 && stype == S_F16) return launch_mfma_variant<WP_INT4Q_FP8, A_FP8, O_F16, S_F16, false>(a, t, moe, st);
  return false;
}

}  // namespace qg
