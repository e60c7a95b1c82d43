// Weight-streaming GEMM instantiations: int4 weights (QUAD layout) with e4m3 activations, run as bf16.
#include "qg_stream_kernel.h"

namespace qg {

bool stream_int4q(const StreamArgs& a, const StreamTile& t, int wp, int af, int of, int stype, bool zero, bool moe,
                  hipStream_t st) {
  if (wp == WP_INT4Q_MAGIC && af == A_FP8 && of == O_BF16 && stype == S_BF16 && zero == false)
    return launch_stream_variant<WP_INT4Q_MAGIC, A_FP8, O_BF16, S_BF16, false>(a, t, moe, st);
  if (wp == WP_INT4Q_MAGIC && af == A_FP8 && of == O_F16 && stype == S_F16 && zero == false)
    return launch_stream_variant<WP_INT4Q_MAGIC, A_FP8, O_F16, S_F16, false>(a, t, moe, st);
  return false;
}

}  // namespace qg
