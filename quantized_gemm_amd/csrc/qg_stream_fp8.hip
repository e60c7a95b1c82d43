// Weight-streaming GEMM instantiations: e4m3 weights with e4m3 activations.
#include "qg_stream_kernel.h"

namespace qg {

bool stream_fp8(const StreamArgs& a, const StreamTile& t, int wp, int af, int of, int stype, bool zero, bool moe,
                hipStream_t st) {
  if (wp == WP_FP8 && af == A_FP8 && of == O_BF16 && stype == S_F32 && zero == false)
    return launch_stream_variant<WP_FP8, A_FP8, O_BF16, S_F32, false>(a, t, moe, st);
  if (wp == WP_FP8 && af == A_FP8 && of == O_F16 && stype == S_F32 && zero == false)
    return launch_stream_variant<WP_FP8, A_FP8, O_F16, S_F32, false>(a, t, moe, st);
  // block-scaled e4m3 (128 x 128 weight blocks, per-(row, 128-K) activation scales)
  if (wp == WP_FP8_BLOCK && af == A_FP8 && of == O_BF16 && stype == S_F32 && zero == false)
    return launch_stream_variant<WP_FP8_BLOCK, A_FP8, O_BF16, S_F32, false>(a, t, moe, st);
  if (wp == WP_FP8_BLOCK && af == A_FP8 && of == O_F16 && stype == S_F32 && zero == false)
    return launch_stream_variant<WP_FP8_BLOCK, A_FP8, O_F16, S_F32, false>(a, t, moe, st);
  return false;
}

}  // namespace qg
