// MFMA-bound quantized GEMM for large row counts.
//
// Where computation dominates weight transfer ("Humming" wiki article, "Device and
// workload selection"), every weight is reused by many rows, so the weights are
// dequantized once per workgroup tile into the MFMA operand type and the cost of the
// conversion is spread over BM rows:
//   * int4 / uint4: nibble -> float (v_cvt_f32_ubyteN), (u - z) * s as one exact FMA
//     with z*s precomputed, rounded once to bf16/f16;
//   * e2m1: hardware e2m1 -> bf16/f16 conversion with the UE8M0 scale folded in;
//   * e4m3 x e4m3: fp8 MFMA (32x32x64) with the per-token / per-channel scales applied
//     in the epilogue.
//
// Tile: BM x 256 per workgroup.  Four waves own the column quarters [64w, 64w+64); a
// 128-row tile uses 4 waves (one per SIMD, no weight dequantized twice), a 256-row
// tile uses 8 waves (two row halves, two waves per SIMD) so that one wave's dequant
// VALU work co-executes with the other wave's MFMAs.  Activations go through
// LDS, double-buffered, one 128-byte row segment per K step with a 16-byte XOR swizzle
// by row bits 1..3 (16 consecutive rows read the same logical chunk from 16 distinct
// banks groups: conflict-free 16-byte fragment reads); weights go straight from HBM into VGPRs,
// prefetched two K steps ahead.  MFMA 32x32x16 (16-bit) or 32x32x64 (fp8), fp32
// accumulation.  MoE: rows are gathered through sorted_ids and scattered on store.
#pragma once

#include "qg_device.h"
#include "qg_kernels.h"

namespace qg {

template <int WP, int AF, int OF, int ST, bool ZERO, int BM, bool MOE, int MW>
__global__ __launch_bounds__(256 * MW) __attribute__((amdgpu_waves_per_eu(MW, MW)))
void mfma_gemm_kernel(MfmaArgs a) {
  constexpr bool F8 = (WP == WP_FP8);
  constexpr int AB = F8 ? 1 : 2;
  constexpr int BK = F8 ? 128 : 64;          // K per step; one LDS row segment = 128 bytes
  constexpr int NTHR = 256 * MW;             // MW groups of 4 waves split the rows
  constexpr int MT = BM / 32 / MW;           // 32-row MFMA tiles per wave
  constexpr int NT = 2;                      // 32-column MFMA tiles per wave
  constexpr int BN = 256;
  constexpr int ROWB = 128;
  constexpr int STAGE = BM * ROWB;
  constexpr int APT = STAGE / 16 / NTHR;     // 16-byte activation pieces per thread per step
  constexpr int BU = F8 ? 4 : 1;             // 16-byte weight units per lane per tile and step

  __shared__ __attribute__((aligned(16))) uint8_t sA[2 * STAGE];
  __shared__ int sRowTok[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);   // column quarter
  const int wm = __builtin_amdgcn_readfirstlane(tid >> 8);           // row part
  const int r = lane & 31;
  const int g = lane >> 5;

  // ---- tile coordinates ------------------------------------------------------------
  int expert = 0;
  int64_t rowbase;
  int ntile;
  if constexpr (MOE) {
    ntile = blockIdx.x;
    rowbase = (int64_t)blockIdx.y * BM;
    if (rowbase >= (int64_t)(*a.num_post_pad)) return;
    expert = a.expert_ids[blockIdx.y];
  } else {
    // The dispatcher hands workgroups to the 8 XCDs round-robin (XCD = id % 8).  When
    // the column tiles split evenly, XCD x owns a contiguous band of column tiles and
    // walks its row tiles row-major over that band, so the ~32 tiles it runs at once
    // share a few activation row blocks and weight column blocks in its own L2.
    const int mtiles = (int)((a.m + BM - 1) / BM);
    const int ntiles = (int)gridDim.x / mtiles;
    const int id = blockIdx.x;
    if ((ntiles & 7) == 0) {
      const int nper = ntiles >> 3;
      const int x = id & 7, l = id >> 3;
      ntile = x * nper + l % nper;
      rowbase = (int64_t)(l / nper) * BM;
    } else {
      ntile = id / mtiles;
      rowbase = (int64_t)(id - ntile * mtiles) * BM;
    }
  }
  for (int i = tid; i < BM; i += NTHR) {
    const int64_t rr = rowbase + i;
    int tok;
    if constexpr (MOE) {
      const int f = a.sorted_ids[rr];
      tok = f < a.sentinel ? f / a.topk : -1;
    } else {
      tok = rr < a.m ? (int)rr : -1;
    }
    sRowTok[i] = tok;
  }
  __syncthreads();

  const int nb_count = a.n >> 4;
  const int64_t col0 = (int64_t)ntile * BN + 64 * wave;     // first column of this wave
  const int nsteps = a.k / BK;
  const int64_t kun = F8 ? (a.k >> 4) : (a.k >> 5);
  const int ngroups = a.group == 0 ? 1 : a.k / a.group;
  const uint8_t* wbase = a.w + (int64_t)expert * a.w_expert_bytes;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wbase, (uint32_t)a.w_expert_bytes);
  const int64_t xrow_bytes = (int64_t)a.k * AB;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (uint32_t)(a.x_rows * xrow_bytes));

  // ---- activation staging: piece p of a step = (row p/8, physical chunk p%8) --------
  int a_off[APT];    // byte offset of the piece's source within a row-step, or -1
#pragma unroll
  for (int i = 0; i < APT; ++i) {
    const int p = tid + NTHR * i;
    const int row = p >> 3, pc = p & 7;
    const int lc = pc ^ ((row >> 1) & 7);                  // logical 16-byte chunk
    const int tok = sRowTok[row];
    a_off[i] = tok < 0 ? -1 : (int)((int64_t)tok * xrow_bytes) + 16 * lc;
  }
  auto load_a = [&](int step, u32x4* dst) {
#pragma unroll
    for (int i = 0; i < APT; ++i)
      dst[i] = bload16(xr, a_off[i] < 0 ? kOOB : a_off[i] + step * ROWB);
  };
  auto store_a = [&](int buf, const u32x4* src) {
#pragma unroll
    for (int i = 0; i < APT; ++i) *(u32x4*)(sA + buf * STAGE + (tid + NTHR * i) * 16) = src[i];
  };

  // ---- weights: per tile t, this lane's column and 16-byte units for a step ----------
  int64_t wcol[NT];
  bool wok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    wcol[t] = col0 + 32 * t + r;
    wok[t] = wcol[t] < a.n;
  }
  auto load_b = [&](int step, u32x4 (&dst)[NT][BU]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t nb = wcol[t] >> 4, c = wcol[t] & 15;
#pragma unroll
      for (int u = 0; u < BU; ++u) {
        // 4-bit: unit (step*2 + g) covers k = 64*step + 32g ..; fp8: units 8*step + 4g + u
        const int64_t ku = F8 ? ((int64_t)step * 8 + 4 * g + u) : ((int64_t)step * 2 + g);
        const bool ok = wok[t] && step < nsteps;
        dst[t][u] = bload16_stream(wr, ok ? (int)(((nb * kun + ku) * 16 + c) << 4) : kOOB);
      }
    }
  };
  // per-lane scale (and zero) for the current group of each tile
  auto load_scale = [&](int step, float (&s)[NT], float (&zs)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t nb = min((int64_t)nb_count - 1, wcol[t] >> 4), c = wcol[t] & 15;
      if constexpr (WP == WP_FP4) {
        const int64_t gi = (int64_t)step * 2 + g;           // group 32 == unit
        s[t] = scale_to_f32<ST>(a.s, (((int64_t)expert * nb_count + nb) * ngroups + gi) * 16 + c);
        zs[t] = 0.f;
      } else if constexpr (WP == WP_INT4_MAGIC) {
        const int gi = a.group == 0 ? 0 : (step * BK) / a.group;
        s[t] = scale_to_f32<ST>(a.s, (((int64_t)expert * nb_count + nb) * ngroups + gi) * 16 + c);
        float z = 8.0f;
        if constexpr (ZERO) {
          const uint32_t zw = a.z[((((int64_t)expert * nb_count + nb) * ngroups + gi) << 1) + (c >> 3)];
          z = (float)((zw >> ((c & 7) * 4)) & 0xF);
        }
        zs[t] = -z * s[t];                                  // exact: 4-bit integer x scale
      } else {
        s[t] = 1.f;
        zs[t] = 0.f;
      }
    }
  };

  using Acc = f32x16;
  Acc acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][t][i] = 0.f;

  // ---- prologue: A(0) -> LDS, A(1) in registers, B and scales of steps 0 and 1 ------
  u32x4 ast[APT];
  u32x4 b0[NT][BU], b1[NT][BU];
  float sc0[NT], zs0[NT], sc1[NT], zs1[NT];
  load_a(0, ast);
  load_b(0, b0);
  load_scale(0, sc0, zs0);
  store_a(0, ast);
  load_a(1, ast);
  load_b(1, b1);
  load_scale(1, sc1, zs1);

  // Dequantize word j of this step's weights into the 16-bit MFMA operand of each tile.
  auto dequant = [&](int j, const float* sc, const float* zs, u32x4 (&Bq)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t w = b0[t][0][j];
      if constexpr (WP == WP_FP4) {
        Bq[t] = fp4_to_16<AF>(w, sc[t]);
      } else {
        // PAIR nibble order: bytes of x0 hold elements (0,4,1,5), bytes of x1 (2,6,3,7).
        // The empty asm hides where x0/x1 come from so that each byte converts with a
        // single v_cvt_f32_ubyteN instead of a bit-field extract plus a conversion.
        uint32_t x0 = w & 0x0F0F0F0Fu, x1 = (w >> 4) & 0x0F0F0F0Fu;
        asm volatile("" : "+v"(x0), "+v"(x1));
        const float e0 = __builtin_fmaf((float)(x0 & 0xFF), sc[t], zs[t]);
        const float e4 = __builtin_fmaf((float)((x0 >> 8) & 0xFF), sc[t], zs[t]);
        const float e1 = __builtin_fmaf((float)((x0 >> 16) & 0xFF), sc[t], zs[t]);
        const float e5 = __builtin_fmaf((float)(x0 >> 24), sc[t], zs[t]);
        const float e2 = __builtin_fmaf((float)(x1 & 0xFF), sc[t], zs[t]);
        const float e6 = __builtin_fmaf((float)((x1 >> 8) & 0xFF), sc[t], zs[t]);
        const float e3 = __builtin_fmaf((float)((x1 >> 16) & 0xFF), sc[t], zs[t]);
        const float e7 = __builtin_fmaf((float)(x1 >> 24), sc[t], zs[t]);
        Bq[t] = u32x4{pack2<AF>(e0, e1), pack2<AF>(e2, e3), pack2<AF>(e4, e5), pack2<AF>(e6, e7)};
      }
    }
  };
  // A fragments of 16-bit sub-step j (k = 32g + 8j of the step) for every row tile.
  auto read_a16 = [&](const uint8_t* sAb, int j, u32x4 (&Af)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = 32 * (MT * wm + mt) + r;
      Af[mt] = *(const u32x4*)(sAb + row * ROWB + 16 * ((4 * g + j) ^ ((row >> 1) & 7)));
    }
  };

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    __syncthreads();                                         // A(step) visible; other buffer free
    store_a(buf ^ 1, ast);                                   // A(step+1) (zeros past the end)
    load_a(step + 2, ast);                                   // out-of-range steps read nothing
    const uint8_t* sAb = sA + buf * STAGE;

    if constexpr (F8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        i32x8 B[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) { B[t][i] = (int)b0[t][2 * j][i]; B[t][4 + i] = (int)b0[t][2 * j + 1][i]; }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int row = 32 * (MT * wm + mt) + r;
          const int lc0 = 4 * g + 2 * j;
          const u32x4 a0 = *(const u32x4*)(sAb + row * ROWB + 16 * (lc0 ^ ((row >> 1) & 7)));
          const u32x4 a1 = *(const u32x4*)(sAb + row * ROWB + 16 * ((lc0 + 1) ^ ((row >> 1) & 7)));
          i32x8 A;
#pragma unroll
          for (int i = 0; i < 4; ++i) { A[i] = (int)a0[i]; A[4 + i] = (int)a1[i]; }
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[mt][t] = mfma32x32x64_fp8(A, B[t], acc[mt][t]);
        }
      }
    } else {
      // Software pipeline over the 4 sub-steps: fragments and dequantized weights of
      // sub-step j+1 are produced while the MFMAs of sub-step j run.
      u32x4 Af[2][MT], Bq[2][NT];
      read_a16(sAb, 0, Af[0]);
      dequant(0, sc0, zs0, Bq[0]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j + 1 < 4) {
          read_a16(sAb, j + 1, Af[(j + 1) & 1]);
          dequant(j + 1, sc0, zs0, Bq[(j + 1) & 1]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[mt][t] = mfma32x32x16<AF>(Af[j & 1][mt], Bq[j & 1][t], acc[mt][t]);
      }
    }
    // rotate the weight and scale prefetch
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int u = 0; u < BU; ++u) b0[t][u] = b1[t][u];
      sc0[t] = sc1[t];
      zs0[t] = zs1[t];
    }
    load_b(step + 2, b1);
    load_scale(min(step + 2, nsteps - 1), sc1, zs1);
  }

  // ---- epilogue: lane (r, g) of a 32x32 tile holds column r, rows 8*(i/4) + 4*g + i%4 ----
  uint16_t* yb = (uint16_t*)a.y;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t n = wcol[t];
    if (!wok[t]) continue;
    float sw = 1.f;
    if constexpr (F8) sw = ((const float*)a.s)[(int64_t)expert * a.n + n];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 32 * (MT * wm + mt) + 8 * (i >> 2) + 4 * g + (i & 3);
        const int tok = sRowTok[row];
        if (tok < 0) continue;
        float v = acc[mt][t][i] * sw;
        if constexpr (AF == A_FP8) v *= a.x_scale[tok];
        int64_t orow;
        if constexpr (MOE) orow = a.sorted_ids[rowbase + row];
        else orow = rowbase + row;
        yb[orow * a.n + n] = f32_to_out<OF>(v);
      }
  }
}

template <int WP, int AF, int OF, int ST, bool ZERO, int BM, bool MOE>
static void launch_mfma_one(const MfmaArgs& a, dim3 grid, hipStream_t st) {
  // 256-row tiles run as 8 waves (2 row halves x 4 column quarters, 2 waves per SIMD)
  constexpr int MW = BM == 256 ? 2 : 1;
  hipLaunchKernelGGL((mfma_gemm_kernel<WP, AF, OF, ST, ZERO, BM, MOE, MW>), grid, dim3(256 * MW), 0, st, a);
}

template <int WP, int AF, int OF, int ST, bool ZERO>
static bool launch_mfma_variant(const MfmaArgs& a, const MfmaTile& t, bool moe, hipStream_t st) {
  const dim3 grid(t.grid_x, t.grid_y);
  if (moe) {
    if (t.bm == 128) { launch_mfma_one<WP, AF, OF, ST, ZERO, 128, true>(a, grid, st); return true; }
    if (t.bm == 256) { launch_mfma_one<WP, AF, OF, ST, ZERO, 256, true>(a, grid, st); return true; }
  } else {
    if (t.bm == 128) { launch_mfma_one<WP, AF, OF, ST, ZERO, 128, false>(a, grid, st); return true; }
    if (t.bm == 256) { launch_mfma_one<WP, AF, OF, ST, ZERO, 256, false>(a, grid, st); return true; }
  }
  return false;
}

}  // namespace qg
