// The steps of an MoE layer around its two grouped products.  The pages time an MoE
// layer as its gate/up product plus its down product ("Humming: Fast, Flexible Kernels
// for Quantized Inference", benchmark paragraph; "Humming" wiki article, "Reported
// performance"); what joins them is this library's reading:
//
//  * SwiGLU on each (token, slot) row of the gate/up output [gate | up]:
//    act = silu(gate) * up, silu(g) = g / (1 + e^-g), in float32; written as f16/bf16, or
//    quantized per row to e4m3 (scale = max|row| / 448, 1 for an all-zero row; RNE after
//    clamping to +-448) when the down product takes FP8 activations.
//  * The down product is the grouped GEMM itself with one input row per slot.
//  * Combine: out[t] = sum_j w[t, j] * y[t * topk + j] over the slots routed inside
//    [0, E), float32 in slot order, one rounding at the end.
//  * Per-token e4m3 quantization of 16-bit activations (the input of a W4A8 product), the
//    same row quantizer without the SwiGLU.
//
// All three are HBM-bound streams: 16-byte loads and stores, 8 elements per thread-piece,
// consecutive lanes on consecutive pieces of a row.  The per-row e4m3 quantization reduces a
// row's absmax within one wave for rows up to 2048 wide, within a workgroup beyond.
#include "qg_device.h"
#include "qg_kernels.h"

namespace qg {

namespace {

template <int T>   // O_F16 / O_BF16
__device__ __forceinline__ float to_f32(uint32_t bits16) {
  if constexpr (T == O_BF16) return bf16_bits_to_f32(bits16);
  else return f16_bits_to_f32(bits16);
}

template <int T>
__device__ __forceinline__ void unpack8(const u32x4 v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = to_f32<T>(v[i] & 0xFFFFu);
    f[2 * i + 1] = to_f32<T>(v[i] >> 16);
  }
}

template <int T>
__device__ __forceinline__ u32x4 pack8(const float* f) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = (uint32_t)f32_to_out<T>(f[2 * i]) | ((uint32_t)f32_to_out<T>(f[2 * i + 1]) << 16);
  return o;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

template <int IN>
__device__ __forceinline__ void swiglu8(const uint16_t* row, int64_t inter, int64_t c8, float* act) {
  float g[8], u[8];
  unpack8<IN>(ldg16(row + 8 * c8), g);
  unpack8<IN>(ldg16(row + inter + 8 * c8), u);
#pragma unroll
  for (int i = 0; i < 8; ++i) act[i] = silu(g[i]) * u[i];
}

// One thread per 8 outputs of a row.
template <int IN, int OUT>
__global__ __launch_bounds__(256) void swiglu_kernel(const uint16_t* __restrict__ gu, int64_t rows, int64_t inter,
                                                     uint16_t* __restrict__ out) {
  const int64_t per_row = inter >> 3;
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= rows * per_row) return;
  const int64_t r = p / per_row, c8 = p - r * per_row;
  float act[8];
  swiglu8<IN>(gu + r * 2 * inter, inter, c8, act);
  *(u32x4*)(out + r * inter + 8 * c8) = pack8<OUT>(act);
}

// SwiGLU -> MXFP4, one thread per 32 outputs of a row: the activations are computed exactly as
// swiglu_kernel does, rounded to bfloat16 (the 16-bit SwiGLU output), then encoded, so the
// result equals swiglu_kernel followed by the MXFP4 row quantizer bit for bit.
template <int IN>
__global__ __launch_bounds__(256) void swiglu_e2m1_kernel(const uint16_t* __restrict__ gu, int64_t rows, int64_t inter,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t per_row = inter >> 5;
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= rows * per_row) return;
  const int64_t r = p / per_row, blk = p - r * per_row;
  float act[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) swiglu8<IN>(gu + r * 2 * inter, inter, 4 * blk + q, act + 8 * q);
#pragma unroll
  for (int i = 0; i < 32; ++i) act[i] = bf16_bits_to_f32(f32_to_out<O_BF16>(act[i]));
  u32x4 packed;
  const uint32_t e8 = mxfp4_encode32(act, packed);
  *(u32x4*)(codes + r * (inter >> 1) + 16 * blk) = packed;
  scales[p] = (uint8_t)e8;
}

// One workgroup of 256 threads per row; each thread keeps up to kSwigluE4m3Pieces pieces of 8
// activations in registers while the row's absmax is reduced, then quantizes them.
constexpr int kSwigluE4m3Pieces = 4;   // inter <= 256 * 4 * 8 = 8192

template <int IN, bool SILU>
__global__ __launch_bounds__(256) void swiglu_e4m3_kernel(const uint16_t* __restrict__ gu, int64_t inter,
                                                          uint8_t* __restrict__ codes, float* __restrict__ scale) {
  __shared__ float s_wmax[4];
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const int64_t per_row = inter >> 3;
  const uint16_t* row = gu + r * (SILU ? 2 : 1) * inter;
  float act[kSwigluE4m3Pieces][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kSwigluE4m3Pieces; ++i) {
    const int64_t c8 = tid + 256 * i;
    if (c8 < per_row) {
      if constexpr (SILU) swiglu8<IN>(row, inter, c8, act[i]);
      else unpack8<IN>(ldg16(row + 8 * c8), act[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(act[i][e]));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((tid & 63) == 0) s_wmax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_wmax[0], s_wmax[1]), fmaxf(s_wmax[2], s_wmax[3]));
  const float sc = amax == 0.0f ? 1.0f : amax / 448.0f;     // correctly rounded division
  if (tid == 0) scale[r] = sc;
#pragma unroll
  for (int i = 0; i < kSwigluE4m3Pieces; ++i) {
    const int64_t c8 = tid + 256 * i;
    if (c8 < per_row) {
      uint32_t w[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float q[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = fminf(fmaxf(act[i][4 * h + e] / sc, -448.0f), 448.0f);
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);   // bytes 0, 1
        v = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], v, true);        // bytes 2, 3
        w[h] = (uint32_t)v;
      }
      u32x2 o;
      o[0] = w[0];
      o[1] = w[1];
      *(u32x2*)(codes + r * inter + 8 * c8) = o;
    }
  }
}

// Rows up to kSwigluWaveRow wide: one wave per row (four rows per workgroup), the absmax
// reduced with wave shuffles only; every lane keeps up to four pieces in registers.
constexpr int kSwigluWaveRow = 64 * 4 * 8;

// SILU: the row is [gate | up] and its SwiGLU is quantized; else the row itself (per-token
// quantization of 16-bit activations).
template <int IN, bool SILU>
__global__ __launch_bounds__(256) void swiglu_e4m3_wave_kernel(const uint16_t* __restrict__ gu, int64_t rows,
                                                               int64_t inter, uint8_t* __restrict__ codes,
                                                               float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;                       // whole waves leave together
  const int64_t per_row = inter >> 3;
  const uint16_t* row = gu + r * (SILU ? 2 : 1) * inter;
  float act[4][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t c8 = lane + 64 * i;
    if (c8 < per_row) {
      if constexpr (SILU) swiglu8<IN>(row, inter, c8, act[i]);
      else unpack8<IN>(ldg16(row + 8 * c8), act[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(act[i][e]));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float sc = amax == 0.0f ? 1.0f : amax / 448.0f;     // correctly rounded division
  if (lane == 0) scale[r] = sc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t c8 = lane + 64 * i;
    if (c8 < per_row) {
      u32x2 o;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float q[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = fminf(fmaxf(act[i][4 * h + e] / sc, -448.0f), 448.0f);
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], v, true);
        o[h] = (uint32_t)v;
      }
      *(u32x2*)(codes + r * inter + 8 * c8) = o;
    }
  }
}

// One thread per 8 outputs of a token.  Slots go in groups of 8 with every row load of a
// group in flight at once: a dropped slot's row exists (it is only unwritten), so it is read
// like the others and discarded with a select, never multiplied (it may hold NaN).
template <int T>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y, const float* __restrict__ w,
                                                      const int32_t* __restrict__ ids, int64_t tokens, int topk,
                                                      int experts, int64_t n, uint16_t* __restrict__ out) {
  constexpr int G = 8;
  const int64_t per_row = n >> 3;
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= tokens * per_row) return;
  const int64_t t = p / per_row, c8 = p - t * per_row;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < topk; j0 += G) {
    u32x4 v[G];
    bool ok[G];
    float wj[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int j = j0 + u;
      const int64_t f = t * topk + (j < topk ? j : topk - 1);
      const int e = ids[f];
      ok[u] = j < topk && e >= 0 && e < experts;
      wj[u] = w[f];
      v[u] = ldg16(y + f * n + 8 * c8);
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      float vv[8];
      unpack8<T>(v[u], vv);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = ok[u] ? __builtin_fmaf(wj[u], vv[i], acc[i]) : acc[i];
    }
  }
  *(u32x4*)(out + t * n + 8 * c8) = pack8<T>(acc);
}

}  // namespace

template <bool SILU>
static bool launch_rows_e4m3(const uint16_t* g, int64_t rows, int64_t inter, int in_t, void* out, float* out_scale,
                             hipStream_t st) {
  if (inter > 256 * kSwigluE4m3Pieces * 8) return false;
  if (inter <= kSwigluWaveRow) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (in_t == O_BF16)
      hipLaunchKernelGGL((swiglu_e4m3_wave_kernel<O_BF16, SILU>), grid, dim3(256), 0, st, g, rows, inter, (uint8_t*)out,
                         out_scale);
    else
      hipLaunchKernelGGL((swiglu_e4m3_wave_kernel<O_F16, SILU>), grid, dim3(256), 0, st, g, rows, inter, (uint8_t*)out,
                         out_scale);
    return true;
  }
  const dim3 grid((unsigned)rows);
  if (in_t == O_BF16)
    hipLaunchKernelGGL((swiglu_e4m3_kernel<O_BF16, SILU>), grid, dim3(256), 0, st, g, inter, (uint8_t*)out, out_scale);
  else
    hipLaunchKernelGGL((swiglu_e4m3_kernel<O_F16, SILU>), grid, dim3(256), 0, st, g, inter, (uint8_t*)out, out_scale);
  return true;
}

bool launch_swiglu(const void* gu, int64_t rows, int64_t inter, int in_t, int out_t, void* out, void* out_scale,
                   hipStream_t st) {
  const uint16_t* g = (const uint16_t*)gu;
  if (out_t == A_FP8) return launch_rows_e4m3<true>(g, rows, inter, in_t, out, (float*)out_scale, st);
  if (out_t == A_FP4) {
    const dim3 grid4((unsigned)((rows * (inter >> 5) + 255) / 256));
    uint8_t* c = (uint8_t*)out;
    uint8_t* e = (uint8_t*)out_scale;
    if (in_t == O_BF16) hipLaunchKernelGGL((swiglu_e2m1_kernel<O_BF16>), grid4, dim3(256), 0, st, g, rows, inter, c, e);
    else if (in_t == O_F16) hipLaunchKernelGGL((swiglu_e2m1_kernel<O_F16>), grid4, dim3(256), 0, st, g, rows, inter, c, e);
    else return false;
    return true;
  }
  const int64_t pieces = rows * (inter >> 3);
  const dim3 grid((unsigned)((pieces + 255) / 256));
  uint16_t* o = (uint16_t*)out;
  if (in_t == O_BF16 && out_t == A_BF16) hipLaunchKernelGGL((swiglu_kernel<O_BF16, O_BF16>), grid, dim3(256), 0, st, g, rows, inter, o);
  else if (in_t == O_BF16 && out_t == A_F16) hipLaunchKernelGGL((swiglu_kernel<O_BF16, O_F16>), grid, dim3(256), 0, st, g, rows, inter, o);
  else if (in_t == O_F16 && out_t == A_BF16) hipLaunchKernelGGL((swiglu_kernel<O_F16, O_BF16>), grid, dim3(256), 0, st, g, rows, inter, o);
  else if (in_t == O_F16 && out_t == A_F16) hipLaunchKernelGGL((swiglu_kernel<O_F16, O_F16>), grid, dim3(256), 0, st, g, rows, inter, o);
  else return false;
  return true;
}

bool launch_quant_rows_e4m3(const void* x, int64_t rows, int64_t k, int in_t, void* codes, float* scale,
                            hipStream_t st) {
  return launch_rows_e4m3<false>((const uint16_t*)x, rows, k, in_t, codes, scale, st);
}

bool launch_combine(const void* y, const float* w, const int32_t* ids, int64_t tokens, int topk, int experts, int64_t n,
                    int dtype, void* out, hipStream_t st) {
  const int64_t pieces = tokens * (n >> 3);
  const dim3 grid((unsigned)((pieces + 255) / 256));
  const uint16_t* yy = (const uint16_t*)y;
  uint16_t* o = (uint16_t*)out;
  if (dtype == O_BF16) hipLaunchKernelGGL(combine_kernel<O_BF16>, grid, dim3(256), 0, st, yy, w, ids, tokens, topk, experts, n, o);
  else if (dtype == O_F16) hipLaunchKernelGGL(combine_kernel<O_F16>, grid, dim3(256), 0, st, yy, w, ids, tokens, topk, experts, n, o);
  else return false;
  return true;
}

}  // namespace qg
