// Weight-streaming quantized GEMM for small row counts (the HBM-bound regime).
//
// "Humming: Fast, Flexible Kernels for Quantized Inference" describes a separate
// small-batch pipeline (multistage asynchronous copies + MMA) and chooses execution
// strategies by input size; the wiki article ("Device and workload selection") says
// the selector estimates where computation starts to dominate weight transfer.  At
// small M every weight byte is used by exactly one wave, so this kernel streams the
// prepared weights straight from HBM into VGPRs with 16-byte loads, issued for a whole
// wave's share of K before any arithmetic (deep memory-level parallelism), and keeps
// arithmetic per weight as low as possible:
//
//  * int4/uint4 x f16/bf16: the nibble is ORed into the mantissa of 1.0 (exact operand
//    1 + u/2^p, 7 VALU ops per 8 weights); the MFMA sums P = sum X*(1 + u/2^p) over
//    one 128-wide K chunk, a second MFMA with an all-ones operand gives the row sums R,
//    and the group scale and zero point are applied once per chunk and output:
//        y += (s * 2^p) * (P - (1 + z/2^p) * R)  ==  s * sum X*(u - z).
//  * e2m1 x 16-bit: the UE8M0 block scale is folded into the hardware e2m1 -> bf16/f16
//    conversion (exact).
//  * e4m3 x e4m3: fp8 MFMA, per-token x per-channel scale in the epilogue.
//
// Grid: x = groups of 16*NT output columns, y = row blocks of 16*MT rows (dense) or MoE
// blocks (rows gathered through sorted_ids).  A workgroup holds KW waves that split
// K among themselves; partial sums are reduced through LDS at the end, so no
// workspace, no atomics and a fixed summation order.
#pragma once

#include "qg_device.h"
#include "qg_kernels.h"

namespace qg {

template <int WP, int AF, int OF, int ST, bool ZERO, int MT, int NT, int KW, int CH, bool MOE>
__global__ __launch_bounds__(64 * KW) void stream_gemm_kernel(StreamArgs a) {
  constexpr int BM = 16 * MT;
  constexpr int BN = 16 * NT;
  constexpr bool kFp8Mfma = (WP == WP_FP8);
  constexpr int ABYTES = (AF == A_FP8) ? 1 : 2;
  // A lane supplies 32 consecutive k of each 128-wide chunk.
  constexpr int A_U4 = 32 * ABYTES / 16;   // 16-byte pieces of activations per chunk and row tile
  constexpr int B_U4 = kFp8Mfma ? 2 : 1;   // 16-byte weight units per chunk and column tile

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int g = lane >> 4;

  // ---- which rows ----------------------------------------------------------------
  int expert = 0;
  int64_t rowbase = (int64_t)blockIdx.y * BM;
  if constexpr (MOE) {
    if (rowbase >= (int64_t)(*a.num_post_pad)) return;
    expert = a.expert_ids[blockIdx.y];
  }
  // Row (activation index, output index) of this lane for each row tile.
  int64_t arow[MT];
  bool avalid[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int64_t rr = rowbase + 16 * mt + r;
    if constexpr (MOE) {
      const int f = a.sorted_ids[rr];
      avalid[mt] = f < a.sentinel;
      arow[mt] = avalid[mt] ? (f / a.topk) : 0;
    } else {
      avalid[mt] = rr < a.m;
      arow[mt] = avalid[mt] ? rr : 0;
    }
  }

  const int nb0 = blockIdx.x * NT;      // first 16-column block
  const int nchunks = a.k >> 7;
  const int per = (nchunks + KW - 1) / KW;
  const int c0 = wave * per;
  const int c1 = min(nchunks, c0 + per);
  const int myc = max(0, c1 - c0);

  const uint8_t* wbase = a.w + (int64_t)expert * a.w_expert_bytes;
  const int64_t kun = kFp8Mfma ? (a.k >> 4) : (a.k >> 5);  // units along K per 16-col block

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint8_t* xb = (const uint8_t*)a.x;
  const int64_t xrow_bytes = (int64_t)a.k * ABYTES;
  const int ngroups = a.group == 0 ? 1 : (a.k / a.group);

  // The wave's chunk range is processed in rounds of CH chunks; a round first issues
  // all its weight loads, then consumes them.
  for (int cb = 0; cb < myc; cb += CH) {
  const int cnt = min(CH, myc - cb);
  u32x4 bw[CH][NT][B_U4];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if (c < cnt) {
      const int ch = c0 + cb + c;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int u = 0; u < B_U4; ++u) {
          const int64_t ku = kFp8Mfma ? ((int64_t)ch * 8 + 2 * g + u) : ((int64_t)ch * 4 + g);
          const uint8_t* p = wbase + ((((int64_t)(nb0 + t) * kun + ku) * 16 + r) << 4);
          bw[c][t][u] = ldg16_stream(p);
        }
      }
    }
  }

#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if (c < cnt) {
      const int ch = c0 + cb + c;
      // activations for this chunk
      u32x4 av[MT][A_U4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint8_t* p = xb + arow[mt] * xrow_bytes + ((int64_t)ch * 128 + 32 * g) * ABYTES;
#pragma unroll
        for (int q = 0; q < A_U4; ++q)
          av[mt][q] = avalid[mt] ? ldg16(p + 16 * q) : u32x4{0u, 0u, 0u, 0u};
      }

      if constexpr (WP == WP_FP8) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          i32x8 A;
#pragma unroll
          for (int q = 0; q < 4; ++q) { A[q] = (int)av[mt][0][q]; A[4 + q] = (int)av[mt][1][q]; }
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            i32x8 B;
#pragma unroll
            for (int q = 0; q < 4; ++q) { B[q] = (int)bw[c][t][0][q]; B[4 + q] = (int)bw[c][t][1][q]; }
            acc[mt][t] = mfma16x16x128_fp8(A, B, acc[mt][t]);
          }
        }
      } else if constexpr (WP == WP_FP4) {
        // group 32 == one 16-byte unit: one scale per lane per chunk and column tile
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int64_t sidx = (((int64_t)expert * (a.n >> 4) + nb0 + t) * ngroups + ((int64_t)ch * 4 + g)) * 16 + r;
          const float sc = scale_to_f32<ST>(a.s, sidx);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u32x4 b = fp4_to_16<AF>(bw[c][t][0][j], sc);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              // piece j of the lane's 32 activations (16 bytes) pairs with word j of the unit
              acc[mt][t] = mfma16x16x32<AF>(av[mt][j], b, acc[mt][t]);
            }
          }
        }
      } else {
        // int4 / uint4 through the magic-number operand, promotion per chunk.
        constexpr int MAF = (AF == A_FP8) ? A_BF16 : AF;   // fp8 activations run as bf16
        constexpr bool QUAD = (WP == WP_INT4Q_MAGIC);
        f32x4 P[MT][NT];
        f32x4 R[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          R[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < NT; ++t) P[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        constexpr uint32_t ONE2 = (MAF == A_F16) ? 0x3C003C00u : 0x3F803F80u;
        const u32x4 ones = {ONE2, ONE2, ONE2, ONE2};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x4 aj[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            if constexpr (AF == A_FP8) {
              // 8 e4m3 = 2 dwords: piece j of 32 bytes -> av[mt][j>>1] dwords (j&1)*2, +1
              const uint32_t e0 = av[mt][j >> 1][(j & 1) * 2 + 0];
              const uint32_t e1 = av[mt][j >> 1][(j & 1) * 2 + 1];
              aj[mt] = e4m3x8_to_bf16_quad(e0, e1);   // QUAD-ordered bf16
            } else if constexpr (QUAD) {
              aj[mt] = a16_to_quad(av[mt][j]);
            } else {
              aj[mt] = av[mt][j];
            }
            R[mt] = mfma16x16x32<MAF>(aj[mt], ones, R[mt]);
          }
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            uint32_t wj = bw[c][t][0][j];
            if constexpr (QUAD) wj ^= 0x88888888u;     // two's complement -> q + 8
            const u32x4 b = magic4<MAF>(wj);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) P[mt][t] = mfma16x16x32<MAF>(aj[mt], b, P[mt][t]);
          }
        }
        const int grp = a.group == 0 ? 0 : (ch * 128) / a.group;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int64_t sidx = (((int64_t)expert * (a.n >> 4) + nb0 + t) * ngroups + grp) * 16 + r;
          const float sp = scale_to_f32<ST>(a.s, sidx) * MagicConst<MAF>::kInvStep;
          float zc;
          if constexpr (ZERO) {
            const uint32_t zw = a.z[((((int64_t)expert * (a.n >> 4) + nb0 + t) * ngroups + grp) << 1) + (r >> 3)];
            zc = 1.0f + (float)((zw >> ((r & 7) * 4)) & 0xF) * (1.0f / MagicConst<MAF>::kInvStep);
          } else {
            zc = 1.0f + 8.0f * (1.0f / MagicConst<MAF>::kInvStep);
          }
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[mt][t][i] = __builtin_fmaf(sp, __builtin_fmaf(-zc, R[mt][i], P[mt][t][i]), acc[mt][t][i]);
        }
      }
    }
  }

  }  // rounds

  // ---- reduce the KW partial sums through LDS and store --------------------------
  __shared__ float red[KW][BM][BN + 1];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][16 * mt + 4 * g + i][16 * t + r] = acc[mt][t][i];
  __syncthreads();

  uint16_t* yb = (uint16_t*)a.y;
  for (int idx = threadIdx.x; idx < BM * BN; idx += 64 * KW) {
    const int row = idx / BN;
    const int col = idx - row * BN;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < KW; ++w) v += red[w][row][col];
    const int64_t rr = rowbase + row;
    int64_t orow, xrow;
    bool ok;
    if constexpr (MOE) {
      const int f = a.sorted_ids[rr];
      ok = f < a.sentinel;
      orow = f;
      xrow = ok ? f / a.topk : 0;
    } else {
      ok = rr < a.m;
      orow = rr;
      xrow = rr;
    }
    if (!ok) continue;
    const int64_t n = (int64_t)nb0 * 16 + col;
    if constexpr (AF == A_FP8) v *= a.x_scale[xrow];
    if constexpr (WP == WP_FP8) v *= ((const float*)a.s)[(int64_t)expert * a.n + n];
    yb[orow * a.n + n] = f32_to_out<OF>(v);
  }
}

// ---- launch helpers (instantiated per weight path in qg_stream_*.hip) ------------
template <int WP, int AF, int OF, int ST, bool ZERO, int MT, int NT, int KW, int CH, bool MOE>
static void launch_one(const StreamArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((stream_gemm_kernel<WP, AF, OF, ST, ZERO, MT, NT, KW, CH, MOE>), grid, dim3(64 * KW), 0, st, a);
}

template <int WP, int AF, int OF, int ST, bool ZERO, int NT, int KW, int CH, bool MOE>
static bool launch_mt(const StreamArgs& a, int mt, dim3 grid, hipStream_t st) {
  switch (mt) {
    case 1: launch_one<WP, AF, OF, ST, ZERO, 1, NT, KW, CH, MOE>(a, grid, st); return true;
    case 2: launch_one<WP, AF, OF, ST, ZERO, 2, NT, KW, CH, MOE>(a, grid, st); return true;
    case 4: launch_one<WP, AF, OF, ST, ZERO, 4, NT, KW, CH, MOE>(a, grid, st); return true;
    default: return false;
  }
}

template <int WP, int AF, int OF, int ST, bool ZERO, bool MOE>
static bool launch_kw(const StreamArgs& a, const StreamTile& t, hipStream_t st) {
  dim3 grid(t.grid_x, t.grid_y);
  if (t.nt != 2 || t.ch != 8) return false;
  switch (t.kw) {
    case 2: return launch_mt<WP, AF, OF, ST, ZERO, 2, 2, 8, MOE>(a, t.mt, grid, st);
    case 4: return launch_mt<WP, AF, OF, ST, ZERO, 2, 4, 8, MOE>(a, t.mt, grid, st);
    case 8: return launch_mt<WP, AF, OF, ST, ZERO, 2, 8, 8, MOE>(a, t.mt, grid, st);
    default: return false;
  }
}

template <int WP, int AF, int OF, int ST, bool ZERO>
static bool launch_stream_variant(const StreamArgs& a, const StreamTile& t, bool moe, hipStream_t st) {
  return moe ? launch_kw<WP, AF, OF, ST, ZERO, true>(a, t, st) : launch_kw<WP, AF, OF, ST, ZERO, false>(a, t, st);
}

}  // namespace qg
