// Device-side building blocks for the gfx950 quantized GEMM kernels: vector types,
// MFMA wrappers, bit-unpack / dequant routines for the prepared layout, loads.
//
// Prepared layout (format version 1; the offline transform of "Humming: Fast, Flexible
// Kernels for Quantized Inference", standard-format paragraph, which reorders weights,
// scales and zero points into the order the kernel reads them):
//   W: 16-byte units [e][n/16][k/KU][n%16], KU = 32 (4-bit) or 16 (e4m3).  A 4-bit unit is
//      four u32 words; word j holds k = 8j..8j+7 of the unit, nibble position p holding
//      element ORDER[p]:  PAIR {0,2,4,6,1,3,5,7} (int4/uint4 with f16/bf16 activations;
//      int4 stored biased, q + 8), QUAD {0,4,1,5,2,6,3,7} (int4 for the e4m3 conversion,
//      two's complement), NATURAL (e2m1).
//   S: [e][n/16][group][n%16] scale elements.  Z: [e][n/16][group] two u32 words of
//      16 nibbles (column c at word c/8, nibble c%8).
// One 16-byte unit is exactly what one lane loads, so every kernel reads the weight
// stream with 16-byte, fully coalesced loads whatever its tile shape.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Formats (template tags) ---------------------------------------------------------
enum : int { A_F16 = 1, A_BF16 = 2, A_FP8 = 3, A_FP4 = 4 };
enum : int { O_F16 = 1, O_BF16 = 2 };
enum : int { S_F16 = 1, S_BF16 = 2, S_F32 = 3, S_UE8M0 = 4 };
// Weight paths of the kernels.
enum : int {
  WP_INT4_MAGIC = 1,   // int4/uint4 (PAIR order) -> 16-bit operand 1 + u/2^p, zero/scale applied per group
  WP_INT4Q_MAGIC = 2,  // int4 (QUAD order, two's complement) -> 16-bit operand, A permuted to match
  WP_FP4 = 3,          // e2m1 -> bf16/f16 with the UE8M0 block scale folded in
  WP_FP8 = 4,          // e4m3 used as is, fp8 MFMA
  WP_INT4Q_FP8 = 5,    // int4 (QUAD) -> e4m3 by table, fp8 MFMA, group scale per 128-k MFMA
  WP_FP8_BLOCK = 6     // e4m3 with 128 x 128 block scales x e4m3 with (row, 128-k) scales, promoted per step
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// A stored 16-bit or UE8M0 scale (its bits, zero-extended) -> fp32.
template <int ST>
__device__ __forceinline__ float scale_bits_to_f32(uint32_t b) {
  static_assert(ST != S_F32, "fp32 scales are read as floats");
  if constexpr (ST == S_F16) return f16_bits_to_f32(b);
  else if constexpr (ST == S_BF16) return bf16_bits_to_f32(b);
  else {
    // 2^(e-127); e == 0 is the subnormal 2^-127, e == 255 is NaN.
    return b == 0 ? __uint_as_float(0x00400000u) : (b == 255 ? __uint_as_float(0x7fc00000u) : __uint_as_float(b << 23));
  }
}

template <int ST>
__device__ __forceinline__ float scale_to_f32(const void* base, int64_t idx) {
  if constexpr (ST == S_F32) return ((const float*)base)[idx];
  else if constexpr (ST == S_UE8M0) return scale_bits_to_f32<ST>(((const uint8_t*)base)[idx]);
  else return scale_bits_to_f32<ST>(((const uint16_t*)base)[idx]);
}

// Two floats -> packed 16-bit pair (round to nearest even), low half = lo.
template <int AF>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (AF == A_F16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
}

// Output conversion (round to nearest even).
template <int OF>
__device__ __forceinline__ uint16_t f32_to_out(float v) {
  if constexpr (OF == O_BF16) return __builtin_bit_cast(uint16_t, (__bf16)v);
  else return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// ---- 4-bit unpack ------------------------------------------------------------------
// Magic-number decode: OR a nibble into the mantissa of 1.0.  bf16: 1 + u/128
// (0x3F80 | u), f16: 1 + u/1024 (0x3C00 | u); both exact.  Dword q of the result holds
// the nibbles at positions q (low half) and q+4 (high half) of the word.
// The compiler selects one v_and_or_b32 for (x & mask) | bits when neither constant is a
// literal (VOP3 takes no literal operand on this GPU and reads at most one SGPR), so the
// mask is pinned in a VGPR and the OR-ed bits in an SGPR by empty asm statements; with
// literals it emits v_and + v_or.  The instruction itself stays compiler-generated, so its
// hazards against the MFMAs that read the result are tracked (a hand-written v_and_or_b32 in
// inline asm is invisible to that tracking).
template <int AF>
__device__ __forceinline__ u32x4 magic4(uint32_t w) {
  constexpr uint32_t M = (AF == A_F16) ? 0x3C003C00u : 0x3F803F80u;
  uint32_t mask = 0x000F000Fu, bits = M;
  asm("" : "+v"(mask));
  asm("" : "+s"(bits));
  u32x4 r;
  r[0] = (w & mask) | bits;
  r[1] = ((w >> 4) & mask) | bits;
  r[2] = ((w >> 8) & mask) | bits;
  r[3] = ((w >> 12) & mask) | bits;
  return r;
}
template <int AF> struct MagicConst;
template <> struct MagicConst<A_BF16> { static constexpr float kInvStep = 128.0f; };
template <> struct MagicConst<A_F16> { static constexpr float kInvStep = 1024.0f; };
// fp8 activations on the 16-bit path are converted to bf16.
template <> struct MagicConst<A_FP8> { static constexpr float kInvStep = 128.0f; };

// e2m1 x 2^e -> 8 bf16 (natural order): one conversion per byte (two elements).
template <int AF>
__device__ __forceinline__ u32x4 fp4_to_16(uint32_t w, float scale) {
  u32x4 r;
  if constexpr (AF == A_F16) {
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 0));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 1));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 2));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 3));
  } else {
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  }
  return r;
}

// int4 (two's complement, QUAD order) -> 8 e4m3 bytes in k order (2 dwords).
// Table lookup with v_perm_b32: the low 3 bits of a code index two 8-entry tables
// (q = 0..7 and q = -8..-1) held in register pairs, and a third v_perm picks, byte by
// byte, the entry of the table that the code's bit 3 names (selector byte i + 4 * bit 3).
// The nibbles are taken in place: bit 3 of byte i's low (high) nibble moved to bit 2 by a
// shift of 1 (5).  Six or seven operations per 4 weights.  Every int4 value is an exact
// e4m3 value, so the conversion is lossless.
template <int SH>   // 0: the low nibble of each byte, 4: the high nibble
__device__ __forceinline__ uint32_t int4x4_to_e4m3(uint32_t w) {
  const uint32_t idx = (w >> SH) & 0x07070707u;
  const uint32_t pos = __builtin_amdgcn_perm(0x4E4C4A48u, 0x44403800u, idx);
  const uint32_t neg = __builtin_amdgcn_perm(0xB8C0C4C8u, 0xCACCCED0u, idx);
  const uint32_t sel = ((w >> (SH + 1)) & 0x04040404u) | 0x03020100u;
  return __builtin_amdgcn_perm(neg, pos, sel);
}
__device__ __forceinline__ u32x2 int4q_to_e4m3(uint32_t w) {
  u32x2 r;
  r[0] = int4x4_to_e4m3<0>(w);   // positions 0,2,4,6 = elements 0..3
  r[1] = int4x4_to_e4m3<4>(w);   // positions 1,3,5,7 = elements 4..7
  return r;
}

// 8 consecutive e4m3 activations (2 dwords) -> 8 bf16 in the element order the QUAD
// magic decode produces: (0,2) (4,6) (1,3) (5,7).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16_quad(uint32_t e0, uint32_t e1) {
  const uint32_t g0 = __builtin_amdgcn_perm(e1, e0, 0x03010200u);  // f0 f2 f1 f3
  const uint32_t g1 = __builtin_amdgcn_perm(e1, e0, 0x07050604u);  // f4 f6 f5 f7
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(g0, 1.0f, false));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(g0, 1.0f, true));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(g1, 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(g1, 1.0f, true));
  return r;
}
// 8 consecutive 16-bit activations (4 dwords, natural order) -> QUAD element order.
__device__ __forceinline__ u32x4 a16_to_quad(u32x4 d) {
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(d[1], d[0], 0x05040100u);  // a0 a2
  r[2] = __builtin_amdgcn_perm(d[1], d[0], 0x07060302u);  // a1 a3
  r[1] = __builtin_amdgcn_perm(d[3], d[2], 0x05040100u);  // a4 a6
  r[3] = __builtin_amdgcn_perm(d[3], d[2], 0x07060302u);  // a5 a7
  return r;
}

// ---- MFMA wrappers -----------------------------------------------------------------
template <int AF>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (AF == A_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// e4m3 x e4m3, 16x16x128 with neutral block scales (E8M0 127 = 1.0).
__device__ __forceinline__ f32x4 mfma16x16x128_fp8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// e4m3 activations x e2m1 weights (format code 4) with the weights' UE8M0 block scale:
// each lane passes the biased exponent of the 32 K it holds of its column (sb); the
// activation operand's scale is neutral.  The e2m1 operand uses the low 4 dwords of b.
__device__ __forceinline__ f32x4 mfma16x16x128_fp8_fp4(i32x8 a, i32x8 b, int sb, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, 127, 0, sb);
}

// MXFP4 encoding of 32 finite values (the OCP Microscaling conversion): shared exponent
// E = floor(log2 amax) - 2 clamped to [-127, 127] (-127 for an all-zero block), codes = the
// e2m1 value nearest to v / 2^E, ties to the even code, magnitudes above 6 giving 6, negative
// only when not zero.  The scaling by 2^-E is exact and each comparison is against an e2m1
// midpoint, so no rounding enters.  Returns the UE8M0 byte E + 127; codes packed 8 per word,
// element 2j in the low nibble of byte j.
__device__ __forceinline__ uint32_t mxfp4_encode32(const float* v, u32x4& packed) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // amax = f * 2^e with f in [0.5, 1): floor(log2 amax) = e - 1
  const int e = amax > 0.f ? max(-127, min(127, __builtin_amdgcn_frexp_expf(amax) - 3)) : -127;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t word = 0;
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const float q = __builtin_ldexpf(v[8 * j + h], -e);
      const float m = fabsf(q);
      uint32_t c = (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) + (uint32_t)(m >= 1.75f) +
                   (uint32_t)(m > 2.5f) + (uint32_t)(m >= 3.5f) + (uint32_t)(m > 5.0f);
      if (q < 0.f && c != 0) c |= 8u;
      word |= c << (4 * h);
    }
    packed[j] = word;
  }
  return (uint32_t)(e + 127);
}

// e2m1 x e2m1 with E8M0 block exponents for both operands (format code 4 for A and B)
__device__ __forceinline__ f32x4 mfma16x16x128_fp4_fp4(i32x8 a, i32x8 b, int sa, int sb, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}

__device__ __forceinline__ f32x16 mfma32x32x64_fp4_fp4(i32x8 a, i32x8 b, int sa, int sb, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}
// The same with the scale bytes taken from byte J of each scale word (the instruction's
// byte select: four steps' or quarters' exponents share one register)
template <int J>
__device__ __forceinline__ f32x16 mfma32x32x64_fp4_fp4_b(i32x8 a, i32x8 b, int sa, int sb, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, J, sa, J, sb);
}
__device__ __forceinline__ f32x16 mfma32x32x64_fp4_fp4_byte(int j, i32x8 a, i32x8 b, int sa, int sb, f32x16 c) {
  switch (j) {
    case 0: return mfma32x32x64_fp4_fp4_b<0>(a, b, sa, sb, c);
    case 1: return mfma32x32x64_fp4_fp4_b<1>(a, b, sa, sb, c);
    case 2: return mfma32x32x64_fp4_fp4_b<2>(a, b, sa, sb, c);
    default: return mfma32x32x64_fp4_fp4_b<3>(a, b, sa, sb, c);
  }
}

template <int AF>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (AF == A_F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ f32x16 mfma32x32x64_fp8_fp4(i32x8 a, i32x8 b, int sb, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 4, 0, 127, 0, sb);
}
template <int J>
__device__ __forceinline__ f32x16 mfma32x32x64_fp8_fp4_b(i32x8 a, i32x8 b, int sb, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 4, 0, 127, J, sb);
}
__device__ __forceinline__ f32x16 mfma32x32x64_fp8_fp4_byte(int j, i32x8 a, i32x8 b, int sb, f32x16 c) {
  switch (j) {
    case 0: return mfma32x32x64_fp8_fp4_b<0>(a, b, sb, c);
    case 1: return mfma32x32x64_fp8_fp4_b<1>(a, b, sb, c);
    case 2: return mfma32x32x64_fp8_fp4_b<2>(a, b, sb, c);
    default: return mfma32x32x64_fp8_fp4_b<3>(a, b, sb, c);
  }
}

// ---- loads -------------------------------------------------------------------------
// Raw buffer loads: an offset at or beyond the resource's size returns zeros without
// touching memory, which keeps predicated loads branch-free (so the compiler can
// count outstanding loads exactly and wait only for the ones an instruction needs).
constexpr int kOOB = 0x7FFFFFF0;     // an offset past every resource this library builds
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x4 bload16_stream(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);   // nt: streamed once
}
// An empty asm that takes a 32x32 accumulator in VGPRs: the value must be computed
// before this point (device-only, so that no host pass sees a 512-bit register operand).
__device__ __forceinline__ void keep_in_vgprs(const f32x16& v) { asm volatile("" ::"v"(v)); }

// 16 bytes per lane from a buffer straight into LDS: lane l writes lds + 16 l (lds is
// wave-uniform); an out-of-range offset stores zeros.  Kept out of kernel templates: used
// there directly, the host pass drops the templates' launch stubs.
__device__ __forceinline__ void bload16_lds(__amdgpu_buffer_rsrc_t r, void* lds, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}
// 4 bytes per lane into LDS: lane l writes lds + 4 l (lds wave-uniform); out of range: zeros.
__device__ __forceinline__ void bload4_lds(__amdgpu_buffer_rsrc_t r, void* lds, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, off, 0, 0, 0);
}
__device__ __forceinline__ u32x2 bload8(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *(const u32x4*)p; }
// Weight stream: read once, keep it out of the caches' way.
__device__ __forceinline__ u32x4 ldg16_stream(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

}  // namespace qg
