// Dispatch of the GEMM kernels to their per-format instantiation units.
#include "qg_kernels.h"

namespace qg {

bool stream_int4(const StreamArgs&, const StreamTile&, int, int, int, int, bool, bool, hipStream_t);
bool stream_int4q(const StreamArgs&, const StreamTile&, int, int, int, int, bool, bool, hipStream_t);
bool stream_fp4(const StreamArgs&, const StreamTile&, int, int, int, int, bool, bool, hipStream_t);
bool stream_fp8(const StreamArgs&, const StreamTile&, int, int, int, int, bool, bool, hipStream_t);

bool launch_stream_gemm(const StreamArgs& a, const StreamTile& t, int wp, int af, int of, int stype, bool zero,
                        bool moe, hipStream_t st) {
  if (stream_int4(a, t, wp, af, of, stype, zero, moe, st)) return true;
  if (stream_int4q(a, t, wp, af, of, stype, zero, moe, st)) return true;
  if (stream_fp4(a, t, wp, af, of, stype, zero, moe, st)) return true;
  if (stream_fp8(a, t, wp, af, of, stype, zero, moe, st)) return true;
  return false;
}

bool mfma_int4(const MfmaArgs&, const MfmaTile&, int, int, int, int, bool, bool, hipStream_t);
bool mfma_fp4(const MfmaArgs&, const MfmaTile&, int, int, int, int, bool, bool, hipStream_t);
bool mfma_fp8(const MfmaArgs&, const MfmaTile&, int, int, int, int, bool, bool, hipStream_t);
bool mfma_w4a8(const MfmaArgs&, const MfmaTile&, int, int, int, int, bool, bool, hipStream_t);
bool mfma_fp8_block(const MfmaArgs&, const MfmaTile&, int, int, int, int, bool, bool, hipStream_t);

bool launch_mfma_gemm(const MfmaArgs& a, const MfmaTile& t, int wp, int af, int of, int stype, bool zero, bool moe,
                      hipStream_t st) {
  if (mfma_int4(a, t, wp, af, of, stype, zero, moe, st)) return true;
  if (mfma_fp4(a, t, wp, af, of, stype, zero, moe, st)) return true;
  if (mfma_fp8(a, t, wp, af, of, stype, zero, moe, st)) return true;
  if (mfma_w4a8(a, t, wp, af, of, stype, zero, moe, st)) return true;
  if (mfma_fp8_block(a, t, wp, af, of, stype, zero, moe, st)) return true;
  return false;
}

}  // namespace qg
