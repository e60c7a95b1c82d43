// Reduction of split-K partial sums: y[m][n] = out(sum_s part[s][m][n] * w_scale[n] * x_scale[m]).
//
// Used when a dense GEMM has too few output tiles to occupy the GPU and K is split over
// workgroups ("Humming" wiki article, "Device and workload selection": the selector picks
// tiles and split-K by M).  Deterministic: slices are added in order.
#include "qg_device.h"
#include "qg_kernels.h"

namespace qg {

// KS slices (2, 4 or 8) as a compile-time count: every thread issues all of its slices'
// loads before adding any (a runtime loop waits for one load round trip per slice).  Each
// thread owns 4 consecutive columns of one row (one 16-byte load per slice, one 8-byte store).
template <int OF, bool WS, bool XS, int KS>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int64_t m, int n,
                                                           const float* __restrict__ w_scale,
                                                           const float* __restrict__ x_scale, uint16_t* __restrict__ y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int n4 = n >> 2;
  if (idx >= m * n4) return;
  const int64_t row = idx / n4;
  const int col = (int)(idx - row * n4) * 4;
  const int64_t slab = m * (int64_t)n;
  const float* p = part + row * n + col;
  f32x4 u[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) u[s] = __builtin_nontemporal_load((const f32x4*)(p + s * slab));
  f32x4 v = u[0];
#pragma unroll
  for (int s = 1; s < KS; ++s) v += u[s];
  if constexpr (WS) v *= *(const f32x4*)(w_scale + col);
  if constexpr (XS) v *= x_scale[row];
  u32x2 o;
  o[0] = (uint32_t)f32_to_out<OF>(v[0]) | ((uint32_t)f32_to_out<OF>(v[1]) << 16);
  o[1] = (uint32_t)f32_to_out<OF>(v[2]) | ((uint32_t)f32_to_out<OF>(v[3]) << 16);
  *(u32x2*)(y + row * n + col) = o;
}

template <int OF, bool WS, bool XS>
static bool launch_red(const MfmaArgs& a, dim3 grid, const float* ws, uint16_t* y, hipStream_t st) {
  switch (a.ksplit) {
    case 2: hipLaunchKernelGGL((split_reduce_kernel<OF, WS, XS, 2>), grid, dim3(256), 0, st, a.part, a.m, a.n, ws, a.x_scale, y); return true;
    case 4: hipLaunchKernelGGL((split_reduce_kernel<OF, WS, XS, 4>), grid, dim3(256), 0, st, a.part, a.m, a.n, ws, a.x_scale, y); return true;
    case 8: hipLaunchKernelGGL((split_reduce_kernel<OF, WS, XS, 8>), grid, dim3(256), 0, st, a.part, a.m, a.n, ws, a.x_scale, y); return true;
    default: return false;
  }
}

bool launch_split_reduce(const MfmaArgs& a, bool w_scale, bool x_scale, int of, hipStream_t st) {
  const int64_t items = a.m * (a.n / 4);
  const dim3 grid((unsigned)((items + 255) / 256));
  const float* ws = w_scale ? (const float*)a.s : nullptr;
  uint16_t* y = (uint16_t*)a.y;
#define QG_RED(OF_, WS_, XS_) \
  if (of == OF_ && w_scale == WS_ && x_scale == XS_) return launch_red<OF_, WS_, XS_>(a, grid, ws, y, st);
  QG_RED(O_BF16, false, false) QG_RED(O_BF16, true, false) QG_RED(O_BF16, false, true) QG_RED(O_BF16, true, true)
  QG_RED(O_F16, false, false) QG_RED(O_F16, true, false) QG_RED(O_F16, false, true) QG_RED(O_F16, true, true)
#undef QG_RED
  return false;
}

}  // namespace qg
