// Weight-streaming GEMM instantiations: e2m1 weights with UE8M0 block scales.
#include "qg_stream_kernel.h"

namespace qg {

bool stream_fp4(const StreamArgs& a, const StreamTile& t, int wp, int af, int of, int stype, bool zero, bool moe,
                hipStream_t st) {
  if (wp == WP_FP4 && af == A_BF16 && of == O_BF16 && stype == S_UE8M0 && zero == false)
    return launch_stream_variant<WP_FP4, A_BF16, O_BF16, S_UE8M0, false>(a, t, moe, st);
  if (wp == WP_FP4 && af == A_F16 && of == O_F16 && stype == S_UE8M0 && zero == false)
    return launch_stream_variant<WP_FP4, A_F16, O_F16, S_UE8M0, false>(a, t, moe, st);
  // e4m3 activations (W4A8 MXFP4): scaled fp8 x fp4 MFMAs
  if (wp == WP_FP4 && af == A_FP8 && of == O_BF16 && stype == S_UE8M0 && zero == false)
    return launch_stream_variant<WP_FP4, A_FP8, O_BF16, S_UE8M0, false>(a, t, moe, st);
  if (wp == WP_FP4 && af == A_FP8 && of == O_F16 && stype == S_UE8M0 && zero == false)
    return launch_stream_variant<WP_FP4, A_FP8, O_F16, S_UE8M0, false>(a, t, moe, st);
  return false;
}

}  // namespace qg
