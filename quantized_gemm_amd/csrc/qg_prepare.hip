// Offline weight transform ("transform()": validate, then repack weights, scales and
// zero points into the layout the kernels read -- "Humming: Fast, Flexible Kernels for
// Quantized Inference", standard-format paragraphs; "Humming" wiki article,
// "Quantization representation") and the read-back used to check it.
//
// Every output element has exactly one writer and is a pure bit permutation of the
// input, so the prepared image is deterministic and bit-exact.
#include "qg_device.h"
#include "qg_kernels.h"

namespace qg {

// Nibble position p of a prepared word holds element ORDER[p] of the 8 consecutive k.
__constant__ uint8_t kOrders[3][8] = {
    {0, 1, 2, 3, 4, 5, 6, 7},   // natural (e2m1)
    {0, 2, 4, 6, 1, 3, 5, 7},   // pair (int4/uint4 with 16-bit activations)
    {0, 4, 1, 5, 2, 6, 3, 7}};  // quad (int4 converted to e4m3)

// One thread per 16-byte W unit.
__global__ void repack_w_kernel(RepackArgs a) {
  const int nb_count = a.n >> 4;
  const int64_t kun = a.w4 ? (a.k >> 5) : (a.k >> 4);
  const int64_t units = (int64_t)a.experts * nb_count * kun * 16;
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= units) return;
  const int c = (int)(u & 15);
  int64_t rest = u >> 4;
  const int64_t ku = rest % kun;
  rest /= kun;
  const int nb = (int)(rest % nb_count);
  const int e = (int)(rest / nb_count);
  const int64_t n = (int64_t)nb * 16 + c;
  const int64_t row_bytes = a.w4 ? (a.k >> 1) : a.k;
  const uint8_t* src = (const uint8_t*)a.w + ((int64_t)e * a.n + n) * row_bytes + ku * 16;
  u32x4 v = *(const u32x4*)src;
  if (a.w4) {
    const uint8_t* ord = kOrders[a.order];
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t word = 0;
#pragma unroll
      for (int p = 0; p < 8; ++p) word |= ((v[j] >> (4 * ord[p])) & 0xFu) << (4 * p);
      o[j] = a.bias8 ? (word ^ 0x88888888u) : word;
    }
    v = o;
  }
  *(u32x4*)(a.out_w + (u << 4)) = v;
}

// Elements of a region padded to its 256-byte boundary (the bytes up to it are written too,
// as zeros, so the prepared image is fully defined).
inline int64_t padded_elems(int64_t elems, int bytes) { return (elems * bytes + 255) / 256 * 256 / bytes; }

// One thread per scale element: [e][nb][g][c] <- [e][nb*16 + c][g]; block scales
// (s_plain elements, 4 bytes each) are copied as they are; then zeros up to the region's end.
__global__ void repack_s_kernel(RepackArgs a, int64_t padded) {
  const int nb_count = a.n >> 4;
  const int64_t total = a.s_plain > 0 ? a.s_plain : (int64_t)a.experts * a.n * a.groups;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= padded) return;
  if (i >= total) {
    const int eb = a.s_plain > 0 ? 4 : a.s_bytes;
    if (eb == 1) a.out_s[i] = 0;
    else if (eb == 2) ((uint16_t*)a.out_s)[i] = 0;
    else ((uint32_t*)a.out_s)[i] = 0;
    return;
  }
  if (a.s_plain > 0) {
    ((uint32_t*)a.out_s)[i] = ((const uint32_t*)a.s)[i];
    return;
  }
  const int c = (int)(i & 15);
  int64_t rest = i >> 4;
  const int g = (int)(rest % a.groups);
  rest /= a.groups;
  const int nb = (int)(rest % nb_count);
  const int e = (int)(rest / nb_count);
  const int64_t src = ((int64_t)e * a.n + (int64_t)nb * 16 + c) * a.groups + g;
  if (a.s_bytes == 1) a.out_s[i] = ((const uint8_t*)a.s)[src];
  else if (a.s_bytes == 2) ((uint16_t*)a.out_s)[i] = ((const uint16_t*)a.s)[src];
  else ((uint32_t*)a.out_s)[i] = ((const uint32_t*)a.s)[src];
}

// One thread per zero-point word: 8 columns of one (e, nb, g); then zeros up to the region's end.
__global__ void repack_z_kernel(RepackArgs a, int64_t padded) {
  const int nb_count = a.n >> 4;
  const int64_t total = (int64_t)a.experts * nb_count * a.groups * 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= padded) return;
  if (i >= total) {
    a.out_z[i] = 0u;
    return;
  }
  const int half = (int)(i & 1);
  int64_t rest = i >> 1;
  const int g = (int)(rest % a.groups);
  rest /= a.groups;
  const int nb = (int)(rest % nb_count);
  const int e = (int)(rest / nb_count);
  uint32_t word = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int64_t n = (int64_t)nb * 16 + half * 8 + p;
    word |= (uint32_t)(a.z[((int64_t)e * a.n + n) * a.groups + g] & 0xF) << (4 * p);
  }
  a.out_z[i] = word;
}

void launch_repack(const RepackArgs& a, hipStream_t st) {
  const int64_t kun = a.w4 ? (a.k >> 5) : (a.k >> 4);
  const int64_t units = (int64_t)a.experts * (a.n >> 4) * kun * 16;
  hipLaunchKernelGGL(repack_w_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, st, a);
  // (W regions are whole multiples of 256 bytes: n % 64 == 0 and k % 128 == 0)
  const int64_t ns = a.s_plain > 0 ? padded_elems(a.s_plain, 4)
                                   : padded_elems((int64_t)a.experts * a.n * a.groups, a.s_bytes);
  hipLaunchKernelGGL(repack_s_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, st, a, ns);
  if (a.z) {
    const int64_t nz = padded_elems((int64_t)a.experts * (a.n >> 4) * a.groups * 2, 4);
    hipLaunchKernelGGL(repack_z_kernel, dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, st, a, nz);
  }
}

// ---- read-back through the kernels' own unpack routines ---------------------------
// One thread per (n, 32-k unit) (4-bit) or (n, 16-k unit) (e4m3).
template <int WP, int AF, int ST>
__global__ void dequant_kernel(DequantArgs a) {
  const int64_t kun = (WP == WP_FP8) ? (a.k >> 4) : (a.k >> 5);
  const int64_t total = (int64_t)a.n * kun;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t n = i / kun;
  const int64_t ku = i % kun;
  const int nb = (int)(n >> 4), c = (int)(n & 15);
  const u32x4 v = *(const u32x4*)(a.w + ((((int64_t)nb * kun + ku) * 16 + c) << 4));
  float* out = a.out + n * a.k + ku * ((WP == WP_FP8) ? 16 : 32);
  if constexpr (WP == WP_FP8) {
    const float sw = ((const float*)a.s)[n];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[j], 1.0f, false);
      const auto f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[j], 1.0f, true);
      out[4 * j + 0] = f0[0] * sw;
      out[4 * j + 1] = f0[1] * sw;
      out[4 * j + 2] = f1[0] * sw;
      out[4 * j + 3] = f1[1] * sw;
    }
    return;
  } else {
    const int64_t k0 = ku * 32;
    const int grp = (WP == WP_FP4) ? (int)ku : (a.group == 0 ? 0 : (int)(k0 / a.group));
    const int64_t sidx = ((int64_t)nb * a.groups + grp) * 16 + c;
    const float s = scale_to_f32<ST>(a.s, sidx);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float e8[8];
      if constexpr (WP == WP_FP4) {
        const u32x4 b = fp4_to_16<AF>(v[j], s);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          e8[2 * q] = (AF == A_F16) ? f16_bits_to_f32(b[q] & 0xFFFF) : bf16_bits_to_f32(b[q] & 0xFFFF);
          e8[2 * q + 1] = (AF == A_F16) ? f16_bits_to_f32(b[q] >> 16) : bf16_bits_to_f32(b[q] >> 16);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) out[8 * j + q] = e8[q];
      } else if constexpr (WP == WP_INT4Q_FP8) {
        const u32x2 b = int4q_to_e4m3(v[j]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const auto f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(b[h], 1.0f, false);
          const auto f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(b[h], 1.0f, true);
          out[8 * j + 4 * h + 0] = f0[0] * s;
          out[8 * j + 4 * h + 1] = f0[1] * s;
          out[8 * j + 4 * h + 2] = f1[0] * s;
          out[8 * j + 4 * h + 3] = f1[1] * s;
        }
      } else {
        // magic decode: 1 + u/2^p -> u; then (u - z) * s
        constexpr int MAF = (AF == A_FP8) ? A_BF16 : AF;
        constexpr float inv = MagicConst<MAF>::kInvStep;
        float z = 8.0f;
        if (a.zero) {
          const uint32_t zw = a.z[(((int64_t)nb * a.groups + grp) << 1) + (c >> 3)];
          z = (float)((zw >> ((c & 7) * 4)) & 0xF);
        }
        uint32_t wj = v[j];
        if constexpr (WP == WP_INT4Q_MAGIC) wj ^= 0x88888888u;
        const u32x4 b = magic4<MAF>(wj);
        // element order of dword q: PAIR -> (2q, 2q+1); QUAD -> (0,2) (4,6) (1,3) (5,7)
        constexpr int lo[4] = {WP == WP_INT4Q_MAGIC ? 0 : 0, WP == WP_INT4Q_MAGIC ? 4 : 2,
                               WP == WP_INT4Q_MAGIC ? 1 : 4, WP == WP_INT4Q_MAGIC ? 5 : 6};
        constexpr int hi[4] = {WP == WP_INT4Q_MAGIC ? 2 : 1, WP == WP_INT4Q_MAGIC ? 6 : 3,
                               WP == WP_INT4Q_MAGIC ? 3 : 5, WP == WP_INT4Q_MAGIC ? 7 : 7};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float vlo = (MAF == A_F16) ? f16_bits_to_f32(b[q] & 0xFFFF) : bf16_bits_to_f32(b[q] & 0xFFFF);
          const float vhi = (MAF == A_F16) ? f16_bits_to_f32(b[q] >> 16) : bf16_bits_to_f32(b[q] >> 16);
          e8[lo[q]] = (vlo - 1.0f) * inv;
          e8[hi[q]] = (vhi - 1.0f) * inv;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) out[8 * j + q] = (e8[q] - z) * s;
      }
    }
  }
}

void launch_dequant(const DequantArgs& a, hipStream_t st) {
  const int64_t kun = (a.wp == WP_FP8) ? (a.k >> 4) : (a.k >> 5);
  const int64_t total = (int64_t)a.n * kun;
  dim3 grid((unsigned)((total + 255) / 256)), block(256);
#define QG_DQ(WP_, AF_, ST_) \
  if (a.wp == WP_ && a.af == AF_ && a.stype == ST_) { hipLaunchKernelGGL((dequant_kernel<WP_, AF_, ST_>), grid, block, 0, st, a); return; }
  QG_DQ(WP_INT4_MAGIC, A_F16, S_F16)
  QG_DQ(WP_INT4_MAGIC, A_F16, S_BF16)
  QG_DQ(WP_INT4_MAGIC, A_BF16, S_BF16)
  QG_DQ(WP_INT4_MAGIC, A_BF16, S_F16)
  QG_DQ(WP_INT4Q_MAGIC, A_FP8, S_BF16)
  QG_DQ(WP_INT4Q_MAGIC, A_FP8, S_F16)
  QG_DQ(WP_INT4Q_FP8, A_FP8, S_BF16)
  QG_DQ(WP_INT4Q_FP8, A_FP8, S_F16)
  QG_DQ(WP_FP4, A_BF16, S_UE8M0)
  QG_DQ(WP_FP4, A_F16, S_UE8M0)
  QG_DQ(WP_FP8, A_FP8, S_F32)
#undef QG_DQ
}

}  // namespace qg
