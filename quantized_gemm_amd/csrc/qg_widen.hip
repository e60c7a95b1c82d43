// e4m3 activations -> bf16, exactly (every e4m3 value is a bf16 value), for W4A8 layers
// run on the 16-bit MFMA path: the int4 weights decode exactly to bf16 there too, and the
// per-token activation scale is applied in that kernel's epilogue, so the product is the
// same as multiplying e4m3 by int4 converted to e4m3.  Running the W4A8 product in bf16
// is this library's own reading: the pages fix the operand types (int4 weights converted
// to FP8 inside the kernel), not the MFMA that multiplies them, and both routes compute the
// same exact products.  Each thread widens 16 codes (16 bytes in, 32 out).
#include "qg_device.h"
#include "qg_kernels.h"

namespace qg {

__global__ __launch_bounds__(256) void widen_e4m3_bf16_kernel(const uint8_t* __restrict__ x, uint16_t* __restrict__ y,
                                                              int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const u32x4 v = *(const u32x4*)(x + 16 * i);
  u32x4 o0, o1;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    o0[2 * d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[d], 1.0f, false));
    o0[2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[d], 1.0f, true));
    o1[2 * d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[2 + d], 1.0f, false));
    o1[2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[2 + d], 1.0f, true));
  }
  *(u32x4*)(y + 16 * i) = o0;
  *(u32x4*)(y + 16 * i + 8) = o1;
}

void launch_widen_e4m3_bf16(const void* x, void* y, int64_t elems, hipStream_t st) {
  const int64_t n16 = elems / 16;
  hipLaunchKernelGGL(widen_e4m3_bf16_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, st,
                     (const uint8_t*)x, (uint16_t*)y, n16);
}

}  // namespace qg
