// MFMA-bound quantized GEMM for large row counts.
//
// Where computation dominates weight transfer ("Humming" wiki article, "Device and
// workload selection"), every weight is reused by many rows, so the weights are
// dequantized once per workgroup tile into the MFMA operand type and the cost of the
// conversion is spread over BM rows:
//   * int4 / uint4: nibble -> float (v_cvt_f32_ubyteN), (u - z) * s as one exact FMA
//     with z*s precomputed, rounded once to bf16/f16;
//   * int4 x e4m3 (W4A8): int4 -> e4m3 by a byte table (exact), fp8 MFMA (32x32x64) per
//     128-wide step = one scale group, each step's product promoted by its group scale,
//     per-token scale in the epilogue;
//   * e2m1: hardware e2m1 -> bf16/f16 conversion with the UE8M0 scale folded in;
//   * e4m3 x e4m3: fp8 MFMA (32x32x64) with the per-token / per-channel scales applied
//     in the epilogue;
//   * e4m3 x e4m3 with 128 x 128 weight-block and per-(row, 128-K) activation scales: each
//     128-wide step's product from zero, promoted by (row scale x block scale); the weights
//     are the MFMAs' first operand, so a lane's products share one activation row and one
//     row scale;
//   * e4m3 x e2m1 (W4A8 MXFP4): no dequantization at all, the e2m1 codes and their UE8M0
//     block scales are operands of the scaled fp8/fp4 MFMA; per-token scale in the epilogue;
//   * e2m1 x e2m1 (W4A4 MXFP4): both operands and both UE8M0 exponents go to the scaled
//     fp4 x fp4 MFMA; a 128-byte row segment holds 256 K, and each step's activation
//     exponents travel into LDS with the step's activations.
//
// Tile: BM x 256 per workgroup, CW waves, wave w owning all BM rows of the columns
// [w 256/CW, (w+1) 256/CW), so that every weight is dequantized exactly once per tile.
// Tiles use 8 waves of 32 columns (two waves per SIMD: one wave's dequant VALU work
// co-executes with the other's MFMAs); only MoE blocks of 128 rows with 16-bit
// activations or with e2m1 weights under e4m3 activations keep 4 waves of 64.  Activations go HBM -> LDS directly through a ring of four
// stages (16-bit) or three (byte operands), one 128-byte row segment per K step with a 16-byte XOR swizzle by row bits
// 1..3 (conflict-free 16-byte fragment reads); weights go straight from HBM into VGPRs,
// prefetched two or three K steps ahead; the scale and zero records of a step travel
// with the activations into LDS (two loads per workgroup and step, not one per lane).
// MFMA 32x32x16 (16-bit) or 32x32x64 (fp8), fp32 accumulation.  MoE: rows are gathered
// through sorted_ids and scattered on store.
#pragma once

#include "qg_device.h"
#include "qg_kernels.h"

namespace qg {

template <int WP, int AF, int OF, int ST, bool ZERO, int BM, bool MOE, bool SPLIT, int CW>
__global__ __launch_bounds__(64 * CW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_gemm_kernel(MfmaArgs a) {
  constexpr bool F4A = (AF == A_FP4);                // e2m1 activations: fp4 x fp4 MFMAs
  constexpr bool F8 = (AF == A_FP8) || F4A;          // byte operands to scaled / fp8 MFMAs as stored
  constexpr bool FP4B = (AF == A_FP8) && WP == WP_FP4;   // e4m3 activations with e2m1 weights
  constexpr bool I4F8 = (AF == A_FP8) && WP == WP_INT4Q_FP8;   // int4 weights converted to e4m3 here
  constexpr bool BLK = (AF == A_FP8) && WP == WP_FP8_BLOCK;     // e4m3 x e4m3 with 128 x 128 block scales
  constexpr int AB = F8 ? 1 : 2;
  constexpr int BK = F4A ? 256 : F8 ? 128 : 64;   // K per step; one LDS row segment = 128 bytes
  constexpr int NTHR = 64 * CW;              // CW waves, each owning BN / CW columns and all BM rows
  constexpr int MT = BM / 32;                // 32-row MFMA tiles per wave
  constexpr int WCOL = 256 / CW;             // columns per wave: 64 (4 waves) or 32 (8 waves)
  constexpr int NT = WCOL / 32;              // 32-column MFMA tiles per wave
  constexpr int BN = 256;
  constexpr int ROWB = 128;
  constexpr int STAGE = BM * ROWB;
  // activation stages in LDS (ring): 16-bit paths 4 (the stage three steps ahead is loaded
  // after the mid-step hand-over, so its loads get two steps to land), byte paths 3
  constexpr int NS = F8 ? 3 : 4;
  constexpr int AHEAD = NS - 1;              // steps between a stage's loads and its use
  constexpr int APT = STAGE / 16 / NTHR;     // 16-byte activation pieces per thread per step
  constexpr int BU = F8 ? ((FP4B || I4F8) ? 2 : 4) : 1;   // 16-byte weight units per lane per tile and step (F4A: 4)
  // elements held by the bytes of the low / high nibble words of a 4-bit code word (PAIR order)
  constexpr int M0[4] = {0, 4, 1, 5};
  constexpr int M1[4] = {2, 6, 3, 7};

  // one array per stage: the compiler then sees which stage an LDS read and an
  // HBM->LDS load touch, and waits only where they really overlap
  __shared__ __attribute__((aligned(16))) uint8_t sA0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sA1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sA2[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sA3[NS == 4 ? STAGE : 16];
  // 16-bit paths: the next step's scale (and zero) records of the tile's 256 columns,
  // one region per activation stage, loaded HBM -> LDS with that stage's activations
  // (scales in the first KiB, zero words in the second)
  constexpr bool SDMA = !F8;
  constexpr int SREG = SDMA ? 2048 : 16;
  __shared__ __attribute__((aligned(16))) uint8_t sS0[SREG];
  __shared__ __attribute__((aligned(16))) uint8_t sS1[SREG];
  __shared__ __attribute__((aligned(16))) uint8_t sS2[SREG];
  __shared__ __attribute__((aligned(16))) uint8_t sS3[NS == 4 ? SREG : 16];
  // e2m1 activations: the step's UE8M0 exponents of each tile row (8 bytes: K groups
  // 8 step .. 8 step + 7), one region per activation stage, loaded with that stage
  // block scales: the step's float scale of each tile row
  constexpr int XSB = F4A ? BM * 8 : BLK ? BM * 4 : 16;
  __shared__ __attribute__((aligned(16))) uint8_t sX0[XSB];
  __shared__ __attribute__((aligned(16))) uint8_t sX1[XSB];
  __shared__ __attribute__((aligned(16))) uint8_t sX2[XSB];
  __shared__ int sRowTok[BM];
  __shared__ int sRowOut[BM];    // output row of each tile row (-1: none)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);         // column slice of the tile
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
    // The dispatcher hands workgroups to the 8 XCDs round-robin (XCD = id % 8), each XCD
    // with its own L2.  The tile grid is cut into XR x (8 / XR) blocks, one per XCD, with
    // XR chosen so that an XCD's share of activation rows plus weight columns is
    // smallest (each XCD then fetches only its own rows and columns); inside its block
    // an XCD walks row tiles fastest, so the ~32 tiles it runs at once form a compact
    // rectangle sharing activation and weight slices in L2.
    const int mtiles = (int)((a.m + BM - 1) / BM);
    const int ntiles = (int)gridDim.x / mtiles;
    const int id = blockIdx.x;
    const int64_t rowb = F4A ? a.k / 2 : (int64_t)a.k * AB, colb = (WP == WP_FP8 || BLK) ? a.k : a.k / 2;   // bytes per row / column
    int xr = 0;
    int64_t best = 0;
    for (int cand = 1; cand <= 8; cand <<= 1) {
      if (mtiles % cand != 0 || ntiles % (8 / cand) != 0) continue;
      const int64_t cost = (int64_t)mtiles * BM * rowb / cand + (int64_t)ntiles * BN * colb / (8 / cand);
      if (xr == 0 || cost < best) { xr = cand; best = cost; }
    }
    if (xr != 0) {
      const int xc = 8 / xr;
      const int mt_x = mtiles / xr, nt_x = ntiles / xc;   // tiles per XCD block
      const int x = id & 7, l = id >> 3;                   // XCD and its local tile index
      const int lm = l % mt_x, ln = l / mt_x;
      rowbase = (int64_t)((x / xc) * mt_x + lm) * BM;
      ntile = (x % xc) * nt_x + ln;
    } else {
      ntile = id / mtiles;
      rowbase = (int64_t)(id - ntile * mtiles) * BM;
    }
  }
  for (int i = tid; i < BM; i += NTHR) {
    const int64_t rr = rowbase + i;
    int tok;
    int orow;
    if constexpr (MOE) {
      const int f = a.sorted_ids[rr];
      tok = f < a.sentinel ? f / a.topk : -1;
      orow = f;
    } else {
      tok = rr < a.m ? (int)rr : -1;
      orow = (int)rr;
    }
    sRowTok[i] = tok;
    sRowOut[i] = tok < 0 ? -1 : orow;
  }
  __syncthreads();

  const int nb_count = a.n >> 4;
  const int64_t col0 = (int64_t)ntile * BN + WCOL * wave;   // first column of this wave
  // Split K: workgroup z owns steps [kstep0, kstep0 + nsteps) and writes fp32 partial
  // sums (the host makes the slices whole scale groups); otherwise all of K.
  const int nsteps = SPLIT ? a.k / BK / a.ksplit : a.k / BK;
  const int kstep0 = SPLIT ? (int)blockIdx.z * nsteps : 0;
  const int64_t kun = (WP == WP_FP8 || BLK) ? (a.k >> 4) : (a.k >> 5);   // 16-byte units along K per column
  const int ngroups = a.group == 0 ? 1 : a.k / a.group;
  const uint8_t* wbase = a.w + (int64_t)expert * a.w_expert_bytes;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wbase, (uint32_t)a.w_expert_bytes);
  const int64_t xrow_bytes = F4A ? a.k / 2 : (int64_t)a.k * AB;
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
  // Activations go HBM -> LDS directly (buffer_load ... lds): lane l of a wave writes the
  // 16 bytes at the wave's LDS base + 16 l, so piece p = tid + NTHR*i lands in slot p of the
  // stage.  Rows without a token and steps past the end read out of range, which stores
  // zeros.  Exactly APT loads per thread per step, no branches (the wait counts rely on it).
  const int wave_slot = (tid & ~63) * 16;
  auto issue_a_piece = [&](int step, uint8_t* stage, int i) {
    bload16_lds(xr, stage + NTHR * 16 * i + wave_slot,
                a_off[i] < 0 || step >= nsteps ? kOOB : a_off[i] + (kstep0 + step) * ROWB);
  };
  auto issue_a = [&](int step, uint8_t* stage) {
#pragma unroll
    for (int i = 0; i < APT; ++i) issue_a_piece(step, stage, i);
  };
  // e2m1 activations: dword h of tile row r's step exponents comes from thread 2r + h (a
  // wave-uniform subset of the threads), into region + 4 tid; issued just before the same
  // step's activations, so the wait for those covers it too.
  // Block scales: the float scale of tile row r for the step comes from thread r the same way.
  int xs_off = -1;
  if constexpr (F4A) {
    if (tid < 2 * BM) {
      const int tok = sRowTok[tid >> 1];
      xs_off = tok < 0 ? -1 : tok * (a.k >> 5) + 4 * (tid & 1);
    }
  } else if constexpr (BLK) {
    if (tid < BM) {
      const int tok = sRowTok[tid];
      xs_off = tok < 0 ? -1 : tok * (a.k >> 7) * 4;
    }
  }
  const __amdgpu_buffer_rsrc_t xsr =
      make_rsrc(a.x_scale, F4A ? (uint32_t)(a.x_rows * (a.k >> 5)) : BLK ? (uint32_t)(a.x_rows * (a.k >> 7) * 4) : 0u);
  auto issue_xs = [&](int step, uint8_t* reg) {
    if constexpr (F4A) {
      if (tid < 2 * BM)
        bload4_lds(xsr, reg + (tid & ~63) * 4, xs_off < 0 || step >= nsteps ? kOOB : xs_off + 8 * (kstep0 + step));
    } else if constexpr (BLK) {
      if (tid < BM)
        bload4_lds(xsr, reg + (tid & ~63) * 4, xs_off < 0 || step >= nsteps ? kOOB : xs_off + 4 * (kstep0 + step));
    }
  };

  // ---- scale and zero records: 16 bytes per lane, one load on wave 0 (scales) and one
  // on wave 1 (zeros) per step instead of one per lane and tile.  Group of K half h of
  // step t (k = 64t + 32h ..): e2m1 blocks of 32, two per step; int4 groups are a
  // multiple of 128 (or the whole K), so both halves share one (a wave-uniform division).
  constexpr int ES = ST == S_UE8M0 ? 1 : 2;               // bytes per stored scale
  // int4 scale group of step t = (kstep0 + t) / gsteps, steps per group gsteps (the whole K,
  // group 0, is one group), as a multiply-high by grec = ceil(2^32 / gsteps): exact for
  // step indices and divisors below 2^16 (the error term x (grec gsteps - 2^32) / 2^32 stays
  // below 1 / gsteps), and for any power-of-two divisor (no error term); no division in the loop
  // (gsteps 1: grec 0 and gone 1, the quotient is x itself)
  const uint32_t gsteps = a.group == 0 ? (1u << 30) : (uint32_t)max(1, a.group / BK);
  const uint32_t grec = gsteps == 1 ? 0u : (uint32_t)((((uint64_t)1 << 32) + gsteps - 1) / gsteps);
  const uint32_t gone = gsteps == 1 ? 1u : 0u;
  auto group_of = [&](int t, int h) -> int {
    if constexpr (WP == WP_FP4) return (kstep0 + t) * 2 + h;
    else {
      const uint32_t x = (uint32_t)(kstep0 + t);
      return (int)(__umulhi(x, grec) + x * gone);
    }
  };
  // scale lane -> K half, 16-column block of the tile, 16-byte part of the block's 16 scales
  const int s_h = lane / (16 * ES), s_nb = (lane % (16 * ES)) / ES, s_part = lane % ES;
  const bool s_ok = lane < 32 * ES && ntile * 16 + s_nb < nb_count;
  const bool z_ok = lane < 16 && ntile * 16 + lane < nb_count;   // zero lane -> column block
  const int64_t sc_expert = (int64_t)expert * nb_count * ngroups;  // records before this expert
  const __amdgpu_buffer_rsrc_t sr =
      make_rsrc((const uint8_t*)a.s + sc_expert * 16 * ES, (uint32_t)(nb_count * ngroups * 16 * ES));
  const __amdgpu_buffer_rsrc_t zr =
      make_rsrc(ZERO ? (const void*)(a.z + sc_expert * 2) : a.s, ZERO ? (uint32_t)(nb_count * ngroups * 8) : 0u);
  // Step t's records into region reg: scales of half h at reg + 256 ES h + 16 ES nb + ES c;
  // the two zero words of the step's group (and the next group's) at reg + 1024 + 16 nb.
  // Wave 0 loads the scales, wave 1 the zero words: the wave's source, destination, lane
  // offset and bytes per group are chosen once here, so each step costs one wave-uniform
  // branch and one load.
  const bool sz_wave = SDMA && (wave == 0 || (ZERO && wave == 1));
  const bool sz_zero = ZERO && wave == 1;
  const __amdgpu_buffer_rsrc_t szr = sz_zero ? zr : sr;
  const int sz_dst = sz_zero ? 1024 : 0;
  const bool sz_ok = sz_zero ? z_ok : s_ok;
  const int sz_h = sz_zero ? 0 : s_h;
  const int sz_base = sz_zero ? (ntile * 16 + lane) * ngroups * 8 : (ntile * 16 + s_nb) * ngroups * 16 * ES + 16 * s_part;
  const int sz_gb = sz_zero ? 8 : 16 * ES;                          // bytes per group
  auto issue_sz = [&](int t, uint8_t* reg) {
    if constexpr (SDMA) {
      if (sz_wave) {
        const int off = sz_base + group_of(t, sz_h) * sz_gb;
        bload16_lds(szr, reg + sz_dst, ((t < nsteps) && sz_ok) ? off : kOOB);
      }
    }
  };
  // the 32-bit words holding this lane's stored scale and zero for tile column 32 tt + r,
  // from region reg (whole words: nothing to extend until the values are used)
  auto read_sz = [&](const uint8_t* reg, uint32_t (&sb)[NT], uint32_t (&zw)[NT]) {
    if constexpr (SDMA) {
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const int cl = WCOL * wave + 32 * tt + r, nbl = cl >> 4, c = cl & 15;
        sb[tt] = *(const uint32_t*)(reg + 256 * ES * g + 16 * ES * nbl + ((ES * c) & ~3));
        zw[tt] = ZERO ? *(const uint32_t*)(reg + 1024 + 16 * nbl + 4 * (c >> 3)) : 0u;
      }
    }
  };
  // ... and the scale and z * scale they give
  auto scale_of = [&](const uint32_t (&sb)[NT], const uint32_t (&zw)[NT], float (&s)[NT], float (&zs)[NT]) {
    if constexpr (SDMA) {
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const int c = (WCOL * wave + 32 * tt + r) & 15;
        s[tt] = scale_bits_to_f32<ST>((sb[tt] >> (8 * ((ES * c) & 3))) & (ES == 1 ? 0xFFu : 0xFFFFu));
        if constexpr (WP == WP_FP4) {
          zs[tt] = 0.f;
        } else {
          const float z = ZERO ? (float)((zw[tt] >> ((c & 7) * 4)) & 0xF) : 8.0f;
          zs[tt] = -z * s[tt];
        }
      }
    }
  };

  // ---- weights: per tile t, this lane's column and 16-byte units for a step ----------
  int64_t wcol[NT];
  bool wok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    wcol[t] = col0 + 32 * t + r;
    wok[t] = wcol[t] < a.n;
  }
  auto load_b_unit = [&](int step, u32x4 (&dst)[NT][BU], int t, int u) {
      const int64_t nb = wcol[t] >> 4, c = wcol[t] & 15;
      {
        // 4-bit: unit (step*2 + g) covers k = 64*step + 32g ..; fp8: units 8*step + 4g + u;
        // e2m1 under e4m3 activations: unit 4*step + 2u + g covers k = 128*step + 64u + 32g ..,
        // the e2m1 operand of MFMA u on this lane (int4 converted to e4m3: the same units, each
        // becoming the 32-byte operand of MFMA u); under e2m1 activations unit 8*step + 2u + g
        // (k = 256*step + 64u + 32g ..), the operand of MFMA u
        const int64_t gs = (int64_t)(kstep0 + step);
        const int64_t ku = F4A ? gs * 8 + 2 * u + g
                         : F8 ? ((FP4B || I4F8) ? gs * 4 + 2 * u + g : gs * 8 + 4 * g + u) : (gs * 2 + g);
        const bool ok = wok[t] && step < nsteps;
        // cached: every weight tile is read again by the other row tiles of the XCD
        dst[t][u] = bload16(wr, ok ? (int)(((nb * kun + ku) * 16 + c) << 4) : kOOB);
      }
  };
  auto load_b = [&](int step, u32x4 (&dst)[NT][BU]) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < BU; ++u) load_b_unit(step, dst, t, u);
  };
  // per-lane scale (and zero) for the current group of each tile
  auto load_scale = [&](int step, float (&s)[NT], float (&zs)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t nb = min((int64_t)nb_count - 1, wcol[t] >> 4), c = wcol[t] & 15;
      if constexpr (F4A) {
        // the UE8M0 exponents of the lane's four units (groups 8*step + 2u + g), bytes 0..3
        // of one word kept in the float slot as raw bits; the MFMAs apply them
        const uint8_t* sp = (const uint8_t*)a.s + (((int64_t)expert * nb_count + nb) * ngroups +
                                                   (int64_t)(kstep0 + step) * 8 + g) * 16 + c;
        s[t] = __uint_as_float((uint32_t)sp[0] | ((uint32_t)sp[32] << 8) | ((uint32_t)sp[64] << 16) |
                               ((uint32_t)sp[96] << 24));
        zs[t] = 0.f;
      } else if constexpr (FP4B) {
        // the UE8M0 exponents of the lane's two units (groups 4*step + 2u + g), bytes 0 and 1
        // of one word kept in the float slot as raw bits; the MFMA applies them
        const uint8_t* sp = (const uint8_t*)a.s + (((int64_t)expert * nb_count + nb) * ngroups +
                                                   (int64_t)(kstep0 + step) * 4 + g) * 16 + c;
        s[t] = __uint_as_float((uint32_t)sp[0] | ((uint32_t)sp[32] << 8));
        zs[t] = 0.f;
      } else if constexpr (WP == WP_FP4) {
        const int64_t gi = (int64_t)(kstep0 + step) * 2 + g;   // group 32 == unit
        s[t] = scale_to_f32<ST>(a.s, (((int64_t)expert * nb_count + nb) * ngroups + gi) * 16 + c);
        zs[t] = 0.f;
      } else if constexpr (BLK) {
        // the weight block's scale: the wave's columns lie inside one 128-column block, so
        // the value is uniform over the wave
        const int64_t nblk = a.n >> 7;
        const int64_t blk = min(nblk - 1, (col0 + 32 * t) >> 7);
        s[t] = ((const float*)a.s)[((int64_t)expert * nblk + blk) * (a.k >> 7) + kstep0 + step];
        zs[t] = 0.f;
      } else if constexpr (I4F8) {
        // one step (128 K) lies inside one scale group: the step's products are promoted by it
        const int gi = group_of(step, 0);
        s[t] = scale_to_f32<ST>(a.s, (((int64_t)expert * nb_count + nb) * ngroups + gi) * 16 + c);
        zs[t] = 0.f;
      } else if constexpr (WP == WP_INT4_MAGIC) {
        const int gi = group_of(step, 0);
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

  // ---- prologue: A(0), A(1) -> LDS stages 0, 1; weights and scales -------------------
  // Weights and scales live in a ring of NS register sets, slot = step % NS (a
  // compile-time index in the unrolled loop), loaded DIST steps ahead.  16-bit
  // activations: DIST = 3, since the last sub-step of step s already dequantizes step
  // s+1.  e4m3 weights go to the MFMA as they are: DIST = 2, so that one slot is always
  // idle and its registers free for other values.  Vector-memory issue order, kept by
  // sched_barrier: [B(0)] R(1) A(0) B(DIST-2) R(2) A(1) B(DIST-1), then per step s R(s+3)
  // and A(s+AHEAD) (16-bit: in sub-steps 2 and 3, after the mid-step barrier; byte operands:
  // spread over the step's MFMAs, or at the top) and B(s+DIST) spread after them (int4 ->
  // e4m3: before them), or right after them at the top.
  // R(t) are the scale / zero records of step t (16-bit paths; one load on waves 0 and 1
  // only), issued with A(t-1) into that stage's region, so they land when A(t-1) does and
  // are read at the top of step t-1.  Where a stage is published (the top of its step for
  // byte operands, before the loop for the first 16-bit stage), the loads issued after A(s)
  // include at least B(s+DIST-2) (unless issued before A(s)), A(s+1) and B(s+DIST-1), so
  // vmcnt <= VM_A means A(s) has landed; the record and scale loads only make that count
  // larger.
  constexpr int DIST = F8 ? 2 : 3;
  // Byte-operand paths spread a step's loads over its MFMAs (one every NQ / NL MFMAs)
  // instead of issuing them all after the barrier, where every wave of the workgroup would
  // queue its loads at once in front of its first MFMA (measured 4-10% faster).  Int4 ->
  // e4m3 issues the weights first, since they are converted during the step before their
  // MFMAs, and keeps the loads at the top for 128-row blocks, whose steps are too short to
  // leave the activations their lead (measured 4% slower spread).
  constexpr bool SPREAD = F8 && (!I4F8 || BM == 256);
  constexpr bool BFIRST = I4F8;
  constexpr int NL = APT + NT * BU;            // loads per thread and step
  // Where a slot takes two loads (more loads than MFMAs: e4m3-weight 64-row tiles, 5 loads
  // over 4), a scheduling barrier keeps them in this order: the wait counts (VM_A below)
  // count the loads issued after a stage's last activation piece, and the scheduler may
  // otherwise move that piece behind a weight load of the same slot (seen after an
  // unrelated change: the stage was then read before it had landed).  Slots of one load are
  // ordered by the barrier after each MFMA.
  auto spread_loads = [&](int step, int q, int nq, uint8_t* sAn, u32x4 (&bdst)[NT][BU]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      if (k * nq / NL != q) continue;
      const int kb = BFIRST ? k : k - APT;     // weight unit, if this load is one
      if (kb >= 0 && kb < NT * BU) load_b_unit(step + DIST, bdst, kb / BU, kb % BU);
      else issue_a_piece(step + AHEAD, sAn, BFIRST ? k - NT * BU : k);
      if (NL > nq) __builtin_amdgcn_sched_barrier(0);
    }
  };
  u32x4 bw[NS][NT][BU];
  float scl[NS][NT], zsl[NS][NT];
  if constexpr (DIST == 3) {
    load_b(0, bw[0]);
    load_scale(0, scl[0], zsl[0]);           // later steps' scales come through LDS
    __builtin_amdgcn_sched_barrier(0);
  }
  issue_sz(1, sS0);
  issue_xs(0, sX0);
  issue_a(0, sA0);
  __builtin_amdgcn_sched_barrier(0);
  load_b(DIST - 2, bw[DIST - 2]);
  if constexpr (F8) load_scale(min(DIST - 2, nsteps - 1), scl[DIST - 2], zsl[DIST - 2]);
  __builtin_amdgcn_sched_barrier(0);
  issue_sz(2, sS1);
  issue_xs(1, sX1);
  issue_a(1, sA1);
  __builtin_amdgcn_sched_barrier(0);
  load_b(DIST - 1, bw[DIST - 1]);
  if constexpr (NS == 4) {
    __builtin_amdgcn_sched_barrier(0);
    issue_sz(3, sS2);
    issue_a(2, sA2);
  }
  if constexpr (F8) load_scale(min(DIST - 1, nsteps - 1), scl[DIST - 1], zsl[DIST - 1]);
  __builtin_amdgcn_sched_barrier(0);
  constexpr int NB = NT * BU;                // weight loads per thread per step
  // loads issued after a stage's last activation piece, at least: the weights of that
  // step (unless they go first) and the whole next step
  constexpr int VM_A = (SPREAD && BFIRST) ? APT + NB : APT + 2 * NB;
  static_assert(VM_A < 64, "vmcnt field is 6 bits");

  // Dequantize word j of this step's weights into the 16-bit MFMA operand of each tile.
  auto dequant = [&](const u32x4 (&bsrc)[NT][BU], int j, const float* sc, const float* zs, u32x4 (&Bq)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t w = bsrc[t][0][j];
      if constexpr (WP == WP_FP4) {
        Bq[t] = fp4_to_16<AF>(w, sc[t]);
      } else {
        // PAIR nibble order (biased u = q + 8 or uint4): bytes of x0 hold elements
        // (0,4,1,5), bytes of x1 (2,6,3,7).  The empty asm hides where x0/x1 come from so
        // that each byte converts with a single v_cvt_f32_ubyteN instead of a bit-field
        // extract plus a conversion.
        const uint32_t wb = w;
        uint32_t x0 = wb & 0x0F0F0F0Fu, x1 = (wb >> 4) & 0x0F0F0F0Fu;
        asm volatile("" : "+v"(x0), "+v"(x1));
        float e[8];
        e[M0[0]] = __builtin_fmaf((float)(x0 & 0xFF), sc[t], zs[t]);
        e[M0[1]] = __builtin_fmaf((float)((x0 >> 8) & 0xFF), sc[t], zs[t]);
        e[M0[2]] = __builtin_fmaf((float)((x0 >> 16) & 0xFF), sc[t], zs[t]);
        e[M0[3]] = __builtin_fmaf((float)(x0 >> 24), sc[t], zs[t]);
        e[M1[0]] = __builtin_fmaf((float)(x1 & 0xFF), sc[t], zs[t]);
        e[M1[1]] = __builtin_fmaf((float)((x1 >> 8) & 0xFF), sc[t], zs[t]);
        e[M1[2]] = __builtin_fmaf((float)((x1 >> 16) & 0xFF), sc[t], zs[t]);
        e[M1[3]] = __builtin_fmaf((float)(x1 >> 24), sc[t], zs[t]);
        Bq[t] = u32x4{pack2<AF>(e[0], e[1]), pack2<AF>(e[2], e[3]), pack2<AF>(e[4], e[5]), pack2<AF>(e[6], e[7])};
      }
    }
  };
  // The same dequantization split into 4 stages per tile, so that it can be spread
  // between MFMAs: stage 0 splits the nibbles, 1 and 2 convert and scale four elements
  // each, 3 packs (e2m1: one hardware conversion per stage).
  struct DQ {
    uint32_t x0, x1;
    float e[8];
  };
  auto dq_stage = [&](const u32x4 (&bsrc)[NT][BU], int j, int t, int stg, const float* sc, const float* zs,
                      DQ& d, u32x4& out) {
    const uint32_t w = bsrc[t][0][j];
    if constexpr (WP == WP_FP4) {
      out[stg] = (AF == A_F16) ? fp4_to_16<A_F16>(w, sc[t])[stg] : fp4_to_16<A_BF16>(w, sc[t])[stg];
    } else {
      if (stg == 0) {
        d.x0 = w & 0x0F0F0F0Fu;
        d.x1 = (w >> 4) & 0x0F0F0F0Fu;
        asm volatile("" : "+v"(d.x0), "+v"(d.x1));   // keep v_cvt_f32_ubyteN (see dequant)
      } else if (stg == 1) {
        d.e[M0[0]] = __builtin_fmaf((float)(d.x0 & 0xFF), sc[t], zs[t]);
        d.e[M0[1]] = __builtin_fmaf((float)((d.x0 >> 8) & 0xFF), sc[t], zs[t]);
        d.e[M0[2]] = __builtin_fmaf((float)((d.x0 >> 16) & 0xFF), sc[t], zs[t]);
        d.e[M0[3]] = __builtin_fmaf((float)(d.x0 >> 24), sc[t], zs[t]);
      } else if (stg == 2) {
        d.e[M1[0]] = __builtin_fmaf((float)(d.x1 & 0xFF), sc[t], zs[t]);
        d.e[M1[1]] = __builtin_fmaf((float)((d.x1 >> 8) & 0xFF), sc[t], zs[t]);
        d.e[M1[2]] = __builtin_fmaf((float)((d.x1 >> 16) & 0xFF), sc[t], zs[t]);
        d.e[M1[3]] = __builtin_fmaf((float)(d.x1 >> 24), sc[t], zs[t]);
      } else {
        out = u32x4{pack2<AF>(d.e[0], d.e[1]), pack2<AF>(d.e[2], d.e[3]), pack2<AF>(d.e[4], d.e[5]),
                    pack2<AF>(d.e[6], d.e[7])};
      }
    }
  };
  // A fragments of 16-bit sub-step j (k = 32g + 8j of the step) for every row tile.
  auto read_a16 = [&](const uint8_t* sAb, int j, u32x4 (&Af)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = 32 * mt + r;
      Af[mt] = *(const u32x4*)(sAb + row * ROWB + 16 * ((4 * g + j) ^ ((row >> 1) & 7)));
    }
  };

  u32x4 Bq[2][NT];
  if constexpr (!F8) dequant(bw[0], 0, scl[0], zsl[0], Bq[0]);
  // 16-bit paths publish a stage in the middle of the step before it (below), so the
  // first step's stage is published here and its first fragments read before the loop
  u32x4 Af[MT];   // one fragment register set per row tile (16-bit path)
  if constexpr (!F8) {
    __builtin_amdgcn_s_waitcnt(0x0F70 | (VM_A & 15) | ((VM_A >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read_a16(sA0, 0, Af);
  }
  // int4 -> e4m3: unit u of the lane (32 K, QUAD order) -> the 32 e4m3 bytes of MFMA u's B
  // operand, in k order.  Step 0's units are converted here; each later step's during the
  // step before it, one word per row tile between the MFMAs.
  i32x8 Bc[NT][2];
  auto cvt_word = [&](const u32x4 (&src)[NT][BU], int t, int u, int j, i32x8 (&dst)[NT][2]) {
    const u32x2 e = int4q_to_e4m3(src[t][u][j]);
    dst[t][u][2 * j] = (int)e[0];
    dst[t][u][2 * j + 1] = (int)e[1];
  };
  if constexpr (I4F8) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) cvt_word(bw[0], t, u, j, Bc);
  }

  // One K step; S = step % NS is a compile-time stage index (the loop below is unrolled
  // by NS), so every LDS address names its stage array.
  auto stA = [&](int i) -> uint8_t* { return i == 0 ? sA0 : i == 1 ? sA1 : i == 2 ? sA2 : sA3; };
  auto stS = [&](int i) -> uint8_t* { return i == 0 ? sS0 : i == 1 ? sS1 : i == 2 ? sS2 : sS3; };
  auto step_body = [&](const int step, auto S_) __attribute__((always_inline)) {
    constexpr int S = decltype(S_)::value;
    constexpr int SN = (S + AHEAD) % NS;                      // stage of step + AHEAD
    uint8_t* const sAb = stA(S);
    uint8_t* const sAn = stA(SN);
    const uint8_t* const sSb = stS(S);
    const uint8_t* const sXb = S == 0 ? sX0 : S == 1 ? sX1 : sX2;
    uint8_t* const sXn = S == 0 ? sX2 : S == 1 ? sX0 : sX1;   // exponents of step + 2 (3 stages)
    constexpr int S1 = (S + 1) % NS;                          // slot of step + 1
    uint8_t* const sSn = stS(SN);
    const uint8_t* const sA1b = stA(S1);                      // stage of step + 1
    if constexpr (F8) {
      // this wave's A(step) loads have landed; the barrier makes every wave's visible and
      // frees the stage read during step-1 for A(step+2).  No fence: nothing else is shared.
      __builtin_amdgcn_s_waitcnt(0x0F70 | (VM_A & 15) | ((VM_A >> 4) << 14));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    // 16-bit: the next step's scale and zero words (published with this step's stage)
    uint32_t sbits[NT], zbits[NT];
    if constexpr (!F8) read_sz(sSb, sbits, zbits);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (F8) issue_sz(step + AHEAD + 1, sSn);   // 16-bit: after the mid-step barrier, below
    issue_xs(step + 2, sXn);
    if constexpr (F8 && !SPREAD) issue_a(step + AHEAD, sAn);   // 16-bit: in sub-steps 2 and 3, below
    __builtin_amdgcn_sched_barrier(0);
    constexpr int SL = (S + DIST) % NS;                       // slot of step + DIST
    if constexpr (SPREAD) {
      load_scale(min(step + DIST, nsteps - 1), scl[SL], zsl[SL]);
      __builtin_amdgcn_sched_barrier(0);
    } else if constexpr (DIST == 2) {
      // e4m3 weights: the slot of step + 2 (last read in step - 1) is free already, so
      // its loads go out here, two full steps ahead of use, right after A(step + 2)
      load_b(step + DIST, bw[SL]);
      load_scale(min(step + DIST, nsteps - 1), scl[SL], zsl[SL]);
      __builtin_amdgcn_sched_barrier(0);
    }
    auto& b0 = bw[S];
    auto& b1 = bw[S1];
    // The next step's scales are pinned as plain register values (left as "-8 * s" the
    // symmetric form sends the register allocator into heavy spilling): here for e4m3
    // (constants), after the first sub-step's MFMAs for the 16-bit paths (their LDS
    // reads have landed by then).
    auto pin_scales = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < NT; ++t) asm volatile("" : "+v"(scl[S1][t]), "+v"(zsl[S1][t]));
    };
    if constexpr (F8) pin_scales();

    // Byte-operand paths issue all of a step's loads above, so a padded step (past the end of
    // K) can skip its MFMAs, which would only add zeros; the 16-bit path interleaves its
    // activation loads with the MFMAs and runs padded steps in full.
    if (F8 && !SPREAD && step >= nsteps) {
    } else if constexpr (F4A) {
      // 4 x MT MFMAs per step (K quarters j, row tiles mt), 32x32x64 with both operands e2m1:
      // lane (r, g) gives row r's K 64j + 32g .. + 31 (16 bytes, chunk 2j + g of the row
      // segment) and its exponent; fragments are read two MFMAs ahead as in the e4m3 loop
      auto read_a4 = [&](int q) -> i32x8 {
        const int j = q / MT, mt = q % MT;
        const int row = 32 * mt + r;
        const u32x4 a0 = *(const u32x4*)(sAb + row * ROWB + 16 * ((2 * j + g) ^ ((row >> 1) & 7)));
        i32x8 A;
#pragma unroll
        for (int i = 0; i < 4; ++i) { A[i] = (int)a0[i]; A[4 + i] = 0; }
        return A;
      };
      // The lane's four exponents of row 32 mt + r (groups 2j + g of the step, j = 0..3) as
      // bytes 0..3 of one word: one 8-byte read per row tile and a byte permute; each MFMA
      // picks its byte (and the weight word's byte j) with the instruction's byte select.
      uint32_t ea[MT];
      const uint32_t esel = g ? 0x07050301u : 0x06040200u;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x2 e = *(const u32x2*)(sXb + (32 * mt + r) * 8);
        ea[mt] = __builtin_amdgcn_perm(e[1], e[0], esel);
      }
      // (256-row tiles read one MFMA ahead: their accumulators leave no room for a third set)
      constexpr int NQ = 4 * MT;
      constexpr int AH = BM == 256 ? 1 : 2;      // fragments read ahead
      i32x8 Af4[AH + 1];
#pragma unroll
      for (int q = 0; q < AH; ++q) Af4[q] = read_a4(q);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int j = q / MT, mt = q % MT;
        if (q + AH < NQ) Af4[(q + AH) % (AH + 1)] = read_a4(q + AH);
        if constexpr (SPREAD) spread_loads(step, q, NQ, sAn, bw[SL]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          i32x8 B;
#pragma unroll
          for (int i = 0; i < 4; ++i) { B[i] = (int)b0[t][j][i]; B[4 + i] = 0; }
          acc[mt][t] = mfma32x32x64_fp4_fp4_byte(j, Af4[q % (AH + 1)], B, (int)ea[mt], (int)__float_as_uint(scl[S][t]),
                                                 acc[mt][t]);
          keep_in_vgprs(acc[mt][t]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (BLK) {
      // Block scales: the step is one 128-wide block of K.  The weights are the MFMAs' first
      // operand, so lane (r, g) of a product holds one activation row (32 mt + r) and 16 of the
      // tile's columns (8(i/4) + 4g + i%4), and the promotion acc += (sa[row] * sw) * P needs
      // one row scale per lane and row tile (sw is uniform over the wave: its 32 columns lie
      // inside one 128-column block).  Both operands give the lane the same 32 K (chunks
      // 4g + 2j and 4g + 2j + 1 of the row segment for MFMA j).  Per row tile two MFMAs from
      // zero give P, promoted LAG row tiles later; fragments are read one MFMA ahead.
      auto read_a8b = [&](int mt, int j) -> i32x8 {
        const int row = 32 * mt + r;
        const int lc0 = 4 * g + 2 * j;
        const u32x4 a0 = *(const u32x4*)(sAb + row * ROWB + 16 * (lc0 ^ ((row >> 1) & 7)));
        const u32x4 a1 = *(const u32x4*)(sAb + row * ROWB + 16 * ((lc0 + 1) ^ ((row >> 1) & 7)));
        i32x8 A;
#pragma unroll
        for (int i = 0; i < 4; ++i) { A[i] = (int)a0[i]; A[4 + i] = (int)a1[i]; }
        return A;
      };
      const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      // (256-row tiles have no registers for a second product buffer: 64 bytes per lane spill)
      constexpr int LAG = BM == 256 ? 0 : 1;
      i32x8 Bw[NT][2];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) { Bw[t][j][i] = (int)b0[t][2 * j][i]; Bw[t][j][4 + i] = (int)b0[t][2 * j + 1][i]; }
      i32x8 Ai[2];
      f32x16 P[LAG + 1][NT];
      Ai[0] = read_a8b(0, 0);
#pragma unroll
      for (int mt = 0; mt < MT + LAG; ++mt) {
        if (mt < MT) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int q = 2 * mt + j;
            if (q + 1 < 2 * MT) Ai[(q + 1) & 1] = read_a8b((q + 1) >> 1, (q + 1) & 1);
            if constexpr (SPREAD) spread_loads(step, q, 2 * MT, sAn, bw[SL]);
#pragma unroll
            for (int t = 0; t < NT; ++t)
              P[mt % (LAG + 1)][t] = mfma32x32x64_fp8(Bw[t][j], Ai[q & 1], j == 0 ? zero16 : P[mt % (LAG + 1)][t]);
          }
        }
        const int pm = mt - LAG;                       // row tile promoted now
        if (pm >= 0) {
          const float sa = *(const float*)(sXb + 4 * (32 * pm + r));
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const float c = sa * scl[S][t];
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[pm][t][i] = __builtin_fmaf(c, P[pm % (LAG + 1)][t][i], acc[pm][t][i]);
            keep_in_vgprs(acc[pm][t]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (I4F8) {
      // The lane's two units of this step were converted during the previous step (Bc): each
      // is the 32-byte e4m3 B operand of one 32x32x64 MFMA (k = 64u + 32g .. of the step, in k
      // order); the activation operand is the same 32 K of the row (chunks 4u + 2g and
      // 4u + 2g + 1 of the row segment), so both sides share one k order.
      auto read_a8i = [&](int mt, int j) -> i32x8 {
        const int row = 32 * mt + r;
        const int lc0 = 4 * j + 2 * g;
        const u32x4 a0 = *(const u32x4*)(sAb + row * ROWB + 16 * (lc0 ^ ((row >> 1) & 7)));
        const u32x4 a1 = *(const u32x4*)(sAb + row * ROWB + 16 * ((lc0 + 1) ^ ((row >> 1) & 7)));
        i32x8 A;
#pragma unroll
        for (int i = 0; i < 4; ++i) { A[i] = (int)a0[i]; A[4 + i] = (int)a1[i]; }
        return A;
      };
      // The step is one scale group: each row tile's product P over the step's 128 K starts
      // from zero (two MFMAs) and is promoted, acc += s * P, one row tile behind, so that the
      // promotion of tile mt - 1 runs while the MFMAs of tile mt do; activation fragments
      // (q = 2 mt + j) are read one MFMA ahead.  Between them the next step's weights are
      // converted, NT * 8 / MT words per row tile (the step's VALU work spread over its MFMAs
      // instead of a burst after the barrier, when both waves of a SIMD would convert at once).
      const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      constexpr int NWD = NT * 8;                      // words to convert per step
      constexpr int WPM = (NWD + MT - 1) / MT;         // words per row tile
      // 128-row tiles promote one row tile behind (two product buffers); 256-row tiles have no
      // registers for a second buffer and promote each tile right after its MFMAs, the
      // conversion words in between covering part of the MFMA latency
      constexpr int LAG = BM == 256 ? 0 : 1;
      i32x8 Bn[NT][2];
      i32x8 Ai[2];
      f32x16 P[LAG + 1][NT];
      Ai[0] = read_a8i(0, 0);
#pragma unroll
      for (int mt = 0; mt < MT + LAG; ++mt) {
        if (mt < MT) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int q = 2 * mt + j;
            if (q + 1 < 2 * MT) Ai[(q + 1) & 1] = read_a8i((q + 1) >> 1, (q + 1) & 1);
            if constexpr (SPREAD) spread_loads(step, q, 2 * MT, sAn, bw[SL]);
#pragma unroll
            for (int t = 0; t < NT; ++t)
              P[mt % (LAG + 1)][t] = mfma32x32x64_fp8(Ai[q & 1], Bc[t][j], j == 0 ? zero16 : P[mt % (LAG + 1)][t]);
          }
#pragma unroll
          for (int w = 0; w < WPM; ++w) {
            const int wd = mt * WPM + w;
            if (wd < NWD) cvt_word(b1, wd / 8, (wd / 4) & 1, wd & 3, Bn);
          }
        }
        const int pm = mt - LAG;                       // row tile promoted now
        if (pm >= 0) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
              acc[pm][t][i] = __builtin_fmaf(scl[S][t], P[pm % (LAG + 1)][t][i], acc[pm][t][i]);
            keep_in_vgprs(acc[pm][t]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        Bc[t][0] = Bn[t][0];
        Bc[t][1] = Bn[t][1];
      }
    } else if constexpr (F8) {
      // 2 x MT MFMA pairs per step (k halves j, row tiles mt); each pair's activation
      // fragment is read two pairs ahead, and sched_barrier keeps the compiler from
      // hoisting every read (that would need 16 more fragments live).
      auto read_a8 = [&](int q) -> i32x8 {
        const int j = q / MT, mt = q % MT;
        const int row = 32 * mt + r;
        // The fp8 operand of lane g holds k = 16g .. 16g+15 of the MFMA's 64 in its first 16
        // bytes and k = 32 + 16g .. in the other 16.  With e4m3 weights both operands take
        // any common order (here 32 contiguous bytes per lane); the e2m1 operand's order is
        // fixed (k = 32g + i), so then the activations follow it: MFMA j covers k = 64j ..
        const int lc0 = FP4B ? 4 * j + g : 4 * g + 2 * j;
        const int lc1 = FP4B ? lc0 + 2 : lc0 + 1;
        const u32x4 a0 = *(const u32x4*)(sAb + row * ROWB + 16 * (lc0 ^ ((row >> 1) & 7)));
        const u32x4 a1 = *(const u32x4*)(sAb + row * ROWB + 16 * (lc1 ^ ((row >> 1) & 7)));
        i32x8 A;
#pragma unroll
        for (int i = 0; i < 4; ++i) { A[i] = (int)a0[i]; A[4 + i] = (int)a1[i]; }
        return A;
      };
      constexpr int NQ = 2 * MT;
      i32x8 Af8[3];
      Af8[0] = read_a8(0);
      Af8[1] = read_a8(1);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int j = q / MT, mt = q % MT;
        if (q + 2 < NQ) Af8[(q + 2) % 3] = read_a8(q + 2);
        if constexpr (SPREAD) spread_loads(step, q, NQ, sAn, bw[SL]);
        i32x8 B[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (FP4B) { B[t][i] = (int)b0[t][j][i]; B[t][4 + i] = 0; }
            else { B[t][i] = (int)b0[t][2 * j][i]; B[t][4 + i] = (int)b0[t][2 * j + 1][i]; }
          }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if constexpr (FP4B)
            acc[mt][t] = mfma32x32x64_fp8_fp4_byte(j, Af8[q % 3], B[t], (int)__float_as_uint(scl[S][t]), acc[mt][t]);
          else
            acc[mt][t] = mfma32x32x64_fp8(Af8[q % 3], B[t], acc[mt][t]);
          // Nothing else depends on an MFMA result, and the code generator otherwise sinks
          // whole steps of MFMAs below later barriers (no overlap, every fragment live at
          // once).  The empty asm takes the result here; with the accumulators in VGPRs
          // (two waves per SIMD) it costs nothing.
          keep_in_vgprs(acc[mt][t]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // Software pipeline over the 4 sub-steps, ordered by hand: after the two MFMAs of
      // each row tile come one stage of the next sub-step's dequantization and that tile's
      // next activation fragment read; sched_barrier keeps the order.  Sub-step 3
      // dequantizes sub-step 0 of the next step (its weights and scales are in registers)
      // and reads its fragments from the next stage.  A row tile's next fragment is read
      // into its register set right after its MFMAs, one sub-step (MT * NT MFMAs) ahead.
      //
      // Stage hand-over in the middle of the step, so that no MFMA waits for an LDS read
      // issued after a barrier: after sub-step 1 every wave waits for its own A(step + 1)
      // loads and passes the barrier.  Past it, A(step + 1) is visible to every wave
      // (sub-step 3 reads it), and every wave has finished step - 1, the last reader of the
      // stage and record region that A(step + AHEAD) and R(step + AHEAD + 1) then
      // overwrite (sub-steps 2 and 3, records first, so that they land no later than the
      // stage they ride with).  With four stages a stage's loads have two steps to land.
      constexpr int PH = NT * 4;                 // dequant stages per sub-step
      constexpr int PPM = (PH + MT - 1) / MT;    // stages after each row tile
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool last = (j == 3);
        DQ dq[NT];
        if (j == 2) {
          // loads this wave issued after its share of the next stage, at least: 3 stages
          // B(step + 2) (NB); 4 stages the stage after it and one step of weights (APT + NB:
          // B(2) and A(2) of the prologue for step 0, A(3) and B(3) for step 1, more later)
          constexpr int VM_MID = NS == 4 ? APT + NB : NB;
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_waitcnt(0x0F70 | (VM_MID & 15) | ((VM_MID >> 4) << 14));
          asm volatile("" ::: "memory");
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[mt][t] = mfma32x32x16<AF>(Af[mt], Bq[j & 1][t], acc[mt][t]);
          // R(step + AHEAD + 1), A(step + AHEAD) and B(step + 3) go out in sub-steps 2 and 3,
          // records first, then one piece or weight unit every 2 MT / (APT + NB) row tiles
          // (all weights after every piece, as the waits assume)
          if (j >= 2) {
            if (j == 2 && mt == 0) issue_sz(step + AHEAD + 1, sSn);
            const int slot = (j - 2) * MT + mt;
            constexpr int NL16 = APT + NB;
#pragma unroll
            for (int k = 0; k < NL16; ++k) {
              if (k * 2 * MT / NL16 != slot) continue;
              if (k < APT) issue_a_piece(step + AHEAD, sAn, k);
              else load_b_unit(step + DIST, bw[SL], (k - APT) / BU, (k - APT) % BU);
            }
          }
#pragma unroll
          for (int q = 0; q < PPM; ++q) {
            const int ph = mt * PPM + q;
            if (ph < PH) {
              const int t = ph / 4, stg = ph % 4;
              if (last) dq_stage(b1, 0, t, stg, scl[S1], zsl[S1], dq[t], Bq[(j + 1) & 1][t]);
              else dq_stage(b0, j + 1, t, stg, scl[S], zsl[S], dq[t], Bq[(j + 1) & 1][t]);
            }
          }
          {
            const int row = 32 * mt + r;
            const uint8_t* const src = last ? sA1b : sAb;
            Af[mt] = *(const u32x4*)(src + row * ROWB + 16 * ((4 * g + ((j + 1) & 3)) ^ ((row >> 1) & 7)));
          }
          if (j == 0 && mt == MT - 1) {
            // the raw words are taken as they are here, so no conversion moves up to
            // the loads and waits for them there
#pragma unroll
            for (int t = 0; t < NT; ++t) asm volatile("" : "+v"(sbits[t]), "+v"(zbits[t]));
            scale_of(sbits, zbits, scl[S1], zsl[S1]);
            pin_scales();
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  // The step count is padded to a multiple of NS rather than leaving the unrolled
  // loop early (early exits make the accumulators spill).  A padded step reads its
  // activations out of range, i.e. zeros, so its MFMAs add exact zeros whatever the
  // (finite) weights of that step dequantize to.
  const int nstepsR = (nsteps + NS - 1) / NS * NS;
  for (int step = 0; step < nstepsR; step += NS) {
    step_body(step, std::integral_constant<int, 0>{});
    step_body(step + 1, std::integral_constant<int, 1>{});
    step_body(step + 2, std::integral_constant<int, 2>{});
    if constexpr (NS == 4) step_body(step + 3, std::integral_constant<int, 3>{});
  }
  // the two out-of-range A loads of the last steps are still writing (zeros) into LDS:
  // let them land before the workgroup can finish and its LDS be handed to another
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // ---- epilogue ----------------------------------------------------------------------
  // Lane (r, g) of a 32x32 tile holds column r, rows 8*(i/4) + 4*g + i%4.  Each wave
  // stages CR rows x its 64 columns in LDS (the activation stages are free now), then
  // writes whole row segments with 16-byte stores: 128 bytes per output row (16-bit)
  // or 256 bytes (fp32 split-K partials, unscaled: the reduction applies the scales).
  __syncthreads();                                   // every wave is done with the stages
  if (!wok[0]) return;                               // n % 64 == 0: all or none of a wave's columns
  constexpr int OB = SPLIT ? 4 : 2;                  // output bytes per element
  constexpr int CR = SPLIT ? 16 : 32;                // rows per staged chunk
  constexpr int PITCH = WCOL * OB + 16;              // padded LDS row
  constexpr int PER = STAGE / (CR * PITCH);          // waves' chunks per stage array
  static_assert(3 * PER >= CW, "every wave's chunk fits in the stage arrays");
  uint8_t* const ep = (wave < PER ? sA0 : wave < 2 * PER ? sA1 : sA2) + (wave % PER) * CR * PITCH;
  const int64_t col0w = col0;                        // first column of this wave
  float sw[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) sw[t] = WP == WP_FP8 && !SPLIT ? ((const float*)a.s)[(int64_t)expert * a.n + wcol[t]] : 1.f;
  constexpr int HALVES = 32 / CR;                    // chunks per 32-row tile
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int h = 0; h < HALVES; ++h) {
      const int rbase = 32 * mt + CR * h;          // first tile row of the chunk
      // stage: element (row, col) of the chunk at ep + row * PITCH + col * OB
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if constexpr (BLK) {
            // transposed products (scales applied): lane (r, g) holds tile row r, columns
            // 8(i/4) + 4g + i%4 of tile t
            if (r / CR != h) continue;
            const int rl = r - CR * h, cl = 32 * t + 8 * (i >> 2) + 4 * g + (i & 3);
            if constexpr (SPLIT) *(float*)(ep + rl * PITCH + cl * 4) = acc[mt][t][i];
            else *(uint16_t*)(ep + rl * PITCH + cl * 2) = f32_to_out<OF>(acc[mt][t][i]);
            continue;
          }
          if ((8 * (i >> 2)) / CR != h) continue;              // rows of element i: 8(i/4) + 0..7
          const int rl = 8 * (i >> 2) + 4 * g + (i & 3) - CR * h;
          float v = acc[mt][t][i];
          if constexpr (SPLIT) {
            *(float*)(ep + rl * PITCH + (32 * t + r) * 4) = v;
          } else {
            v *= sw[t];
            if constexpr (AF == A_FP8) {   // per-token scale (e4m3 activations)
              const int tok = sRowTok[rbase + rl];
              v *= tok < 0 ? 0.f : a.x_scale[tok];
            }
            *(uint16_t*)(ep + rl * PITCH + (32 * t + r) * 2) = f32_to_out<OF>(v);
          }
        }
      // write: CR rows x WCOL * OB bytes in pieces of 16 bytes, 64 per lane pass
      constexpr int PPR = WCOL * OB / 16;                      // pieces per row
#pragma unroll
      for (int q = 0; q < CR * PPR / 64; ++q) {
        const int pc = lane + 64 * q;
        const int rl = pc / PPR, c16 = pc - rl * PPR;
        const int orow = sRowOut[rbase + rl];
        if (orow < 0) continue;
        const u32x4 val = *(const u32x4*)(ep + rl * PITCH + 16 * c16);
        if constexpr (SPLIT) {
          float* dst = a.part + ((int64_t)blockIdx.z * a.m + orow) * a.n + col0w + 4 * c16;
          *(u32x4*)dst = val;
        } else {
          uint16_t* dst = (uint16_t*)a.y + (int64_t)orow * a.n + col0w + 8 * c16;
          *(u32x4*)dst = val;
        }
      }
    }
  }
}

template <int WP, int AF, int OF, int ST, bool ZERO, int BM, bool MOE, bool SPLIT = false>
static void launch_mfma_one(const MfmaArgs& a, dim3 grid, hipStream_t st) {
  // Two waves per SIMD throughout.  8 waves of BM x 32 for dense tiles, 256-row MoE blocks
  // and every e4m3-weight tile; 128-row MoE blocks of the other weights (16-bit activations,
  // and e2m1 under e4m3 activations) keep 4 waves of 128 x 64 with two workgroups per CU
  // (their blocks are many and short, and independent workgroups hide each other's barriers
  // better: measured 15% faster for 16-bit, 13-21% for e2m1 x e4m3, while dense 128-row
  // tiles gain ~10% from 8 waves and 4-wave e4m3-weight tiles spill).
  constexpr int CW = (BM == 256 || !MOE || WP == WP_FP8 || WP == WP_FP8_BLOCK || WP == WP_INT4Q_FP8 || AF == A_FP4) ? 8 : 4;
  hipLaunchKernelGGL((mfma_gemm_kernel<WP, AF, OF, ST, ZERO, BM, MOE, SPLIT, CW>), grid, dim3(64 * CW), 0, st, a);
}

template <int WP, int AF, int OF, int ST, bool ZERO>
static bool launch_mfma_variant(const MfmaArgs& a, const MfmaTile& t, bool moe, hipStream_t st) {
  const dim3 grid(t.grid_x, t.grid_y);
  if constexpr (AF == A_FP4) {
    // e2m1 activations: 128-row tiles (dense and MoE) and 256-row dense tiles, one K slice
    if (t.ksplit > 1) return false;
    if (t.bm == 128) {
      if (moe) launch_mfma_one<WP, AF, OF, ST, ZERO, 128, true>(a, grid, st);
      else launch_mfma_one<WP, AF, OF, ST, ZERO, 128, false>(a, grid, st);
      return true;
    }
    if (t.bm == 256 && !moe) { launch_mfma_one<WP, AF, OF, ST, ZERO, 256, false>(a, grid, st); return true; }
    return false;
  } else {
    if (moe) {
      if (t.bm == 128) { launch_mfma_one<WP, AF, OF, ST, ZERO, 128, true>(a, grid, st); return true; }
      if (t.bm == 256) { launch_mfma_one<WP, AF, OF, ST, ZERO, 256, true>(a, grid, st); return true; }
    } else {
      if (t.ksplit > 1) {
        if (t.bm == 64) {   // few rows: 64-row tiles, K split
          launch_mfma_one<WP, AF, OF, ST, ZERO, 64, false, true>(a, dim3(t.grid_x, t.grid_y, t.ksplit), st);
          return true;
        }
        if (t.bm != 128) return false;
        launch_mfma_one<WP, AF, OF, ST, ZERO, 128, false, true>(a, dim3(t.grid_x, t.grid_y, t.ksplit), st);
        return true;
      }
      if (t.bm == 128) { launch_mfma_one<WP, AF, OF, ST, ZERO, 128, false>(a, grid, st); return true; }
      if (t.bm == 256) { launch_mfma_one<WP, AF, OF, ST, ZERO, 256, false>(a, grid, st); return true; }
    }
    return false;
  }
}

}  // namespace qg
