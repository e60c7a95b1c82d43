// Reduction of split-K partial sums: y[m][n] = out(sum_s part[s][m][n] * w_scale[n] * x_scale[m]).
//
// Used when a dense GEMM has too few output tiles to occupy the GPU and K is split over
// workgroups ("Humming" wiki article, "Device and workload selection": the selector picks
// tiles and split-K by M).  Deterministic: slices are added in order.  Each thread owns 8
// consecutive columns of one row (two 16-byte loads per slice, one 16-byte store).
#include "qg_device.h"
#include "qg_kernels.h"

namespace qg {

template <int OF, bool WS, bool XS>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int ksplit, int64_t m, int n,
                                                           const float* __restrict__ w_scale,
                                                           const float* __restrict__ x_scale, uint16_t* __restrict__ y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int n8 = n >> 3;
  if (idx >= m * n8) return;
  const int64_t row = idx / n8;
  const int col = (int)(idx - row * n8) * 8;
  const int64_t slab = m * (int64_t)n;
  const float* p = part + row * n + col;
  f32x4 v0 = *(const f32x4*)p, v1 = *(const f32x4*)(p + 4);
  for (int s = 1; s < ksplit; ++s) {
    const f32x4 u0 = *(const f32x4*)(p + s * slab), u1 = *(const f32x4*)(p + s * slab + 4);
    v0 += u0;
    v1 += u1;
  }
  float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
  if constexpr (WS) {
    const f32x4 w0 = *(const f32x4*)(w_scale + col), w1 = *(const f32x4*)(w_scale + col + 4);
    for (int j = 0; j < 4; ++j) { v[j] *= w0[j]; v[4 + j] *= w1[j]; }
  }
  if constexpr (XS) {
    const float xs = x_scale[row];
    for (int j = 0; j < 8; ++j) v[j] *= xs;
  }
  u32x4 o;
  for (int j = 0; j < 4; ++j) o[j] = (uint32_t)f32_to_out<OF>(v[2 * j]) | ((uint32_t)f32_to_out<OF>(v[2 * j + 1]) << 16);
  *(u32x4*)(y + row * n + col) = o;
}

bool launch_split_reduce(const MfmaArgs& a, bool w_scale, bool x_scale, int of, hipStream_t st) {
  const int64_t items = a.m * (a.n / 8);
  const dim3 grid((unsigned)((items + 255) / 256));
  const float* ws = w_scale ? (const float*)a.s : nullptr;
  uint16_t* y = (uint16_t*)a.y;
#define QG_RED(OF_, WS_, XS_)                                                                                 \
  if (of == OF_ && w_scale == WS_ && x_scale == XS_) {                                                        \
    hipLaunchKernelGGL((split_reduce_kernel<OF_, WS_, XS_>), grid, dim3(256), 0, st, a.part, a.ksplit, a.m, a.n, \
                       ws, a.x_scale, y);                                                                     \
    return true;                                                                                              \
  }
  QG_RED(O_BF16, false, false) QG_RED(O_BF16, true, false) QG_RED(O_BF16, false, true) QG_RED(O_BF16, true, true)
  QG_RED(O_F16, false, false) QG_RED(O_F16, true, false) QG_RED(O_F16, false, true) QG_RED(O_F16, true, true)
#undef QG_RED
  return false;
}

}  // namespace qg
