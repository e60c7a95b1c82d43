// Weight-streaming quantized GEMM for small row counts (the HBM-bound regime).
//
// "Humming: Fast, Flexible Kernels for Quantized Inference" describes a separate
// small-batch pipeline (multistage asynchronous copies + MMA) and chooses execution
// strategies by input size; the wiki article ("Device and workload selection") says
// the selector estimates where computation starts to dominate weight transfer.  At
// small M every weight byte is used by exactly one wave, so this kernel streams the
// prepared weights straight from HBM into VGPRs with 16-byte buffer loads, issued for
// a wave's whole share (up to 16 KB) before any arithmetic, and keeps arithmetic per
// weight low:
//
//  * int4/uint4 x f16/bf16: the nibble is ORed into the mantissa of 1.0 (exact operand
//    1 + u/2^p, 7 VALU ops per 8 weights); the MFMA sums P = sum X*(1 + u/2^p) over
//    one 128-wide K chunk, a second MFMA with an all-ones operand gives the row sums R,
//    and the group scale and zero point are applied once per chunk and output:
//        y += (s * 2^p) * (P - (1 + z/2^p) * R)  ==  s * sum X*(u - z).
//  * e2m1 x 16-bit: the UE8M0 block scale is folded into the hardware e2m1 -> bf16/f16
//    conversion (exact).
//  * e4m3 x e4m3: fp8 MFMA, per-token x per-channel scale in the epilogue.
//  * e4m3 x e2m1 (W4A8 MXFP4): the e2m1 codes and their UE8M0 block scales go to the
//    scaled fp8/fp4 MFMA as they are; per-token scale in the epilogue.
//  * block-scaled e4m3: one fp8 MFMA per chunk (= one 128-wide scale group) from zero,
//    promoted by the row's activation scale times the weight block's scale.
//
// Work split inside a workgroup of NCB x KQ waves: wave (cb, q) owns 16-column block cb
// and the q-th contiguous part of K.  Activations, scales and zero points for all parts
// are staged in LDS in rounds (the next round's staging loads are in flight while the
// current round computes); the KQ partial sums of a column block are added through LDS
// in a fixed order at the end.  No workspace, no atomics, deterministic.
// Grid: x = groups of NCB column blocks, y = row blocks of 16*MT (MT = 0: 4) rows (dense) or MoE
// blocks (rows gathered through sorted_ids).
#pragma once

#include "qg_device.h"
#include "qg_kernels.h"

namespace qg {

template <int WP, int AF>
struct StreamTraits {
  static constexpr bool kFp8Mfma = (WP == WP_FP8 || WP == WP_FP8_BLOCK);
  static constexpr int ABYTES = (AF == A_FP8) ? 1 : 2;
  static constexpr int B_U4 = kFp8Mfma ? 2 : 1;       // 16-byte weight units per lane per chunk
  // staged scale bytes per (column block, chunk): int4 paths 16 scales, fp4 4 groups x 16 bytes
  static constexpr int SBYTES = kFp8Mfma ? 0 : (WP == WP_FP4 ? 64 : 32);
};

// Chunks per wave whose weights are in flight at once (<= 16 KB per wave).
template <int WP>
constexpr int stream_max_chunks() { return (WP == WP_FP8 || WP == WP_FP8_BLOCK) ? 8 : 16; }

// Chunks per K part staged per round: <= 64 KB of activations in LDS.
template <int WP, int AF, int MT, int KQ>
constexpr int stream_round_chunks() {
  constexpr int per_chunk = (MT == 0 ? 4 : 16 * MT) * KQ * 128 * StreamTraits<WP, AF>::ABYTES;
  constexpr int rc = (64 * 1024) / per_chunk;
  constexpr int cap = stream_max_chunks<WP>();       // a round never spans two weight batches
  return rc < 1 ? 1 : (rc > cap ? cap : rc);
}

template <int WP, int AF, int OF, int ST, bool ZERO, int MT, int NCB, int KQ, bool MOE>
__global__ __launch_bounds__(64 * NCB * KQ) void stream_gemm_kernel(StreamArgs a) {
  using T = StreamTraits<WP, AF>;
  constexpr int NW = NCB * KQ;
  constexpr int NTHR = 64 * NW;
  // MT 16-row MFMA tiles; MT == 0 is a 4-row tile (one MFMA tile whose rows 4..15 are
  // zero operands, never staged): for 1..4 rows, the whole K of every part fits one round.
  constexpr int BM = MT == 0 ? 4 : 16 * MT;
  constexpr int NMT = MT == 0 ? 1 : MT;
  constexpr int RCR = stream_round_chunks<WP, AF, MT, KQ>();   // chunks per part per round
  constexpr int CHMAX = stream_max_chunks<WP>();
  static_assert(CHMAX % RCR == 0, "whole rounds per weight batch");
  constexpr int PART = RCR * 128 * T::ABYTES;                   // bytes of one part's round in an LDS row
  constexpr int AROW = KQ * PART + 16;                          // padded LDS row (bytes)
  constexpr int SB = T::SBYTES > 0 ? T::SBYTES : 16;

  __shared__ __attribute__((aligned(16))) uint8_t sA[BM * AROW];
  __shared__ __attribute__((aligned(16))) uint8_t sS[NCB * KQ * RCR * SB];
  __shared__ __attribute__((aligned(8))) uint32_t sZ[NCB * KQ * RCR * 2];
  __shared__ int sRowTok[BM];     // activation row of each tile row (-1: none)
  // int4 / uint4 with 16-bit activations: the magic-number operand needs each 128-wide chunk's
  // activation row sums; they are the same for every column block, so for tiles of 16 rows and
  // more the workgroup adds them once per round in LDS (slot = part * RCR + chunk, then row)
  // instead of an all-ones MFMA per chunk in every wave (measured: 16 rows -6%, 64 rows -2%;
  // 4-row tiles, one round of a few chunks, are faster with the MFMA)
  constexpr bool RSUM = (WP == WP_INT4_MAGIC || WP == WP_INT4Q_MAGIC) && AF != A_FP8 && MT != 0;
  constexpr int NRS = RSUM ? KQ * RCR * BM : 4;
  static_assert(!RSUM || 2 * NRS <= NTHR, "two threads per row sum");
  __shared__ __attribute__((aligned(16))) float sR[NRS];
  // block-scaled e4m3: each 128-wide chunk is one scale group; its product is promoted by the
  // row's activation scale (staged per round, slot = part * RCR + chunk, then row) times the
  // 128-column weight block's scale (loaded with the chunk's weights)
  constexpr bool BLOCK = (WP == WP_FP8_BLOCK);
  constexpr int NSA = BLOCK ? KQ * RCR * BM : 4;
  static_assert(!BLOCK || NSA <= NTHR, "one thread per staged row scale");
  __shared__ __attribute__((aligned(16))) float sSA[NSA];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cb = wave % NCB;            // column block of this wave within the workgroup
  const int q = wave / NCB;             // K part of this wave
  const int r = lane & 15;
  const int g = lane >> 4;

  // ---- rows of this block -----------------------------------------------------------
  int expert = 0;
  const int64_t rowbase = (int64_t)blockIdx.y * BM;
  if constexpr (MOE) {
    if (rowbase >= (int64_t)(*a.num_post_pad)) return;
    expert = a.expert_ids[blockIdx.y];
  }
  if (tid < BM) {
    const int64_t rr = rowbase + tid;
    int tok;
    if constexpr (MOE) {
      const int f = a.sorted_ids[rr];
      tok = f < a.sentinel ? f / a.topk : -1;
    } else {
      tok = rr < a.m ? (int)rr : -1;
    }
    sRowTok[tid] = tok;
  }

  const int nb_count = a.n >> 4;
  const int nbw = blockIdx.x * NCB + cb;                 // this wave's 16-column block
  const bool wact = nbw < nb_count;                      // waves past N only help with staging
  // Dense split K (a.ksplit > 1): workgroup z owns chunks [cbase, cbase + nchunks) of K
  // (whole scale groups, chosen by the host) and writes fp32 partial sums.
  const int ksl = (!MOE && a.ksplit > 1) ? a.ksplit : 1;
  const int nchunks = (a.k >> 7) / ksl;
  const int cbase = ksl > 1 ? (int)blockIdx.z * nchunks : 0;
  const int per = (nchunks + KQ - 1) / KQ;               // chunks per K part
  const int my0 = q * per;
  const int myn = max(0, min(nchunks, my0 + per) - my0);

  const uint8_t* wbase = a.w + (int64_t)expert * a.w_expert_bytes;
  const int64_t kun = T::kFp8Mfma ? (a.k >> 4) : (a.k >> 5);   // 16-byte units along K per column block
  const int ngroups = a.group == 0 ? 1 : (a.k / a.group);
  const int64_t xrow_bytes = (int64_t)a.k * T::ABYTES;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (uint32_t)(a.x_rows * xrow_bytes));
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wbase, (uint32_t)a.w_expert_bytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.s, a.s_bytes);
  const __amdgpu_buffer_rsrc_t zr = make_rsrc(a.z, a.z_bytes);

  __syncthreads();   // sRowTok

  // ---- staging of one round: activations, scales, zeros (registers first) --------------
  constexpr int APR = KQ * PART / 16;                    // 16-byte pieces per activation row
  constexpr int APIECES = BM * APR;
  constexpr int AP_PER_T = (APIECES + NTHR - 1) / NTHR;
  constexpr int SPPC = T::SBYTES / 16;                   // scale pieces per (block, part, chunk)
  constexpr int SPIECES = NCB * KQ * RCR * SPPC;
  constexpr int ZSLOTS = ZERO ? NCB * KQ * RCR : 0;
  static_assert(SPIECES <= NTHR && ZSLOTS <= NTHR, "staging layout");

  struct Stage {
    u32x4 a[AP_PER_T];
    u32x4 s;
    u32x2 z;
    float sa;
  };
  auto load_stage = [&](int rnd, Stage& st) {
#pragma unroll
    for (int i = 0; i < AP_PER_T; ++i) {
      const int p = tid + i * NTHR;
      const int row = min(p / APR, BM - 1);
      const int cp = p - (p / APR) * APR;                // piece within the row
      const int pq = cp / (PART / 16);                   // K part of this piece
      const int pc = cp - pq * (PART / 16);              // piece within that part's round
      const int chunk_in_part = rnd * RCR + pc / (128 * T::ABYTES / 16);
      const int tok = sRowTok[row];
      const int pn = max(0, min(nchunks, pq * per + per) - pq * per);
      const bool ok = p < APIECES && tok >= 0 && chunk_in_part < pn;
      const int64_t off = (int64_t)tok * xrow_bytes + (int64_t)(cbase + pq * per + rnd * RCR) * 128 * T::ABYTES + 16 * pc;
      st.a[i] = bload16(xr, ok ? (int)off : kOOB);
    }
    if constexpr (BLOCK) {
      const int slot = tid / BM, row = tid - slot * BM;             // slot = part * RCR + chunk
      const int spq = slot / RCR, sc = slot - spq * RCR;
      const int chunk_in_part = rnd * RCR + sc;
      const int pn = max(0, min(nchunks, spq * per + per) - spq * per);
      const int tok = sRowTok[min(row, BM - 1)];
      const bool ok = tid < NSA && tok >= 0 && chunk_in_part < pn;
      st.sa = ok ? a.x_scale[(int64_t)tok * (a.k >> 7) + cbase + spq * per + chunk_in_part] : 0.f;
    }
    if constexpr (T::SBYTES > 0) {
      const int slot = tid / SPPC, sq = tid - slot * SPPC;          // slot = (cb, part, chunk)
      const int scb = slot / (KQ * RCR);
      const int srem = slot - scb * KQ * RCR;
      const int spq = srem / RCR, sc = srem - spq * RCR;
      const int64_t nb = (int64_t)blockIdx.x * NCB + scb;
      const int chunk_in_part = rnd * RCR + sc;
      const int pn = max(0, min(nchunks, spq * per + per) - spq * per);
      const int ch = cbase + spq * per + chunk_in_part;
      const bool ok = tid < SPIECES && nb < nb_count && chunk_in_part < pn;
      int64_t elem;
      if constexpr (WP == WP_FP4) elem = (((int64_t)expert * nb_count + nb) * ngroups + (int64_t)ch * 4) * 16;
      else elem = (((int64_t)expert * nb_count + nb) * ngroups + (a.group == 0 ? 0 : (ch * 128) / a.group)) * 16;
      constexpr int EB = (ST == S_UE8M0) ? 1 : 2;
      st.s = bload16(sr, ok ? (int)(elem * EB + 16 * sq) : kOOB);
      if constexpr (ZERO) {
        const int zcb = tid / (KQ * RCR);
        const int zrem = tid - zcb * KQ * RCR;
        const int zpq = zrem / RCR, zc = zrem - zpq * RCR;
        const int64_t znb = (int64_t)blockIdx.x * NCB + zcb;
        const int zcp = rnd * RCR + zc;
        const int zpn = max(0, min(nchunks, zpq * per + per) - zpq * per);
        const int zch = cbase + zpq * per + zcp;
        const bool zok = tid < ZSLOTS && znb < nb_count && zcp < zpn;
        const int grp = a.group == 0 ? 0 : (zch * 128) / a.group;
        st.z = bload8(zr, zok ? (int)(((((int64_t)expert * nb_count + znb) * ngroups + grp) << 1) * 4) : kOOB);
      }
    }
  };
  auto store_stage = [&](const Stage& st) {
#pragma unroll
    for (int i = 0; i < AP_PER_T; ++i) {
      const int p = tid + i * NTHR;
      if (p < APIECES) {
        const int row = p / APR, cp = p - row * APR;
        *(u32x4*)(sA + row * AROW + 16 * cp) = st.a[i];
      }
    }
    if constexpr (BLOCK) {
      if (tid < NSA) sSA[tid] = st.sa;
    }
    if constexpr (T::SBYTES > 0) {
      if (tid < SPIECES) *(u32x4*)(sS + 16 * tid) = st.s;
      if constexpr (ZERO) {
        if (tid < ZSLOTS) *(u32x2*)(sZ + 2 * tid) = st.z;
      }
    }
  };

  f32x4 acc[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the lane's activation row within a 16-row tile: staged rows only.  4-row tiles: rows
  // 4..15 of the MFMA operand read row r & 3 again; the products of those rows are finite
  // copies that land in accumulator rows 4..15, which nothing stores, so they need no zeroing
  const int ar = MT == 0 ? (r & 3) : r;

  const int nrounds = (per + RCR - 1) / RCR;

  // Weights: batches of CHMAX chunks of this wave's part, all loads of a batch in flight.
  // The batch's first staging round is issued before its weights: load counters
  // complete in order, so the first round can start as soon as its own data is in.
  for (int b0 = 0; b0 < per; b0 += CHMAX) {
    const int r0 = b0 / RCR, r1 = min(nrounds, (b0 + CHMAX) / RCR);
    Stage st;
    load_stage(r0, st);
    u32x4 bw[CHMAX][T::B_U4];
    float swb[BLOCK ? CHMAX : 1];          // block-scaled: the weight block's scale per chunk
#pragma unroll
    for (int c = 0; c < CHMAX; ++c) {
      const int ch = cbase + my0 + b0 + c;
#pragma unroll
      for (int u = 0; u < T::B_U4; ++u) {
        const int64_t ku = T::kFp8Mfma ? ((int64_t)ch * 8 + 2 * g + u) : ((int64_t)ch * 4 + g);
        const bool ok = (b0 + c) < myn && wact;
        bw[c][u] = bload16_stream(wr, ok ? (int)((((int64_t)nbw * kun + ku) * 16 + r) << 4) : kOOB);
      }
      if constexpr (BLOCK) {
        const bool ok = (b0 + c) < myn && wact;
        swb[c] = ok ? ((const float*)a.s)[((int64_t)expert * (a.n >> 7) + (nbw >> 3)) * (a.k >> 7) + ch] : 0.f;
      }
    }

    // Rounds of this batch, unrolled so that every chunk's registers appear once.
#pragma unroll
    for (int rr = 0; rr < CHMAX / RCR; ++rr) {
      const int rnd = r0 + rr;
      if (rnd < r1) {                                   // uniform over the workgroup
        store_stage(st);
        __syncthreads();
        if (rnd + 1 < r1) load_stage(rnd + 1, st);     // next round in flight during this one
        if constexpr (RSUM) {
          // thread pair (2s, 2s+1) adds the two halves of row sum s (64 values each); rows
          // without a token and chunks past the end were staged as zeros
          if (tid < 2 * NRS) {
            const int sidx = tid >> 1, h = tid & 1;
            const int row = sidx % BM, slot = sidx / BM;
            const int pq = slot / RCR, pc = slot - pq * RCR;
            const uint8_t* src = sA + row * AROW + pq * PART + pc * 256 + h * 128;
            float sum = 0.f;
#pragma unroll
            for (int v = 0; v < 8; ++v) {
              const u32x4 w = *(const u32x4*)(src + 16 * v);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if constexpr (AF == A_F16) sum += f16_bits_to_f32(w[e] & 0xFFFFu) + f16_bits_to_f32(w[e] >> 16);
                else sum += bf16_bits_to_f32(w[e] & 0xFFFFu) + bf16_bits_to_f32(w[e] >> 16);
              }
            }
            sum += __shfl_xor(sum, 1, 64);
            if (h == 0) sR[slot * BM + row] = sum;
          }
          __syncthreads();
        }
#pragma unroll
        for (int lc = 0; lc < RCR; ++lc) {
          const int c = rr * RCR + lc;                  // chunk of the batch (compile-time)
          // int4 / uint4 in 4-row tiles: a chunk past this wave's part of K, or columns past N,
          // computes with the zeros its out-of-range loads returned (weights, activations,
          // scales), so it adds exactly zero and needs no branch; without one the 16 chunks of a
          // batch form one block the scheduler can overlap (one chunk's decode with the previous
          // chunk's MFMAs): M = 1 12.0 -> 11.3 us; 16-row tiles were not faster without it
          constexpr bool NOBR = (WP == WP_INT4_MAGIC || WP == WP_INT4Q_MAGIC) && MT == 0;
          if (!NOBR && ((b0 + c) >= myn || !wact)) continue;
            const uint8_t* arow0 = sA + q * PART + lc * 128 * T::ABYTES;
            const int slot = (cb * KQ + q) * RCR + lc;
            if constexpr (WP == WP_FP8 || WP == WP_FP8_BLOCK) {
    #pragma unroll
              for (int mt = 0; mt < NMT; ++mt) {
                const uint8_t* ap = arow0 + (16 * mt + ar) * AROW + 32 * g;
                const u32x4 a0 = *(const u32x4*)ap, a1 = *(const u32x4*)(ap + 16);
                i32x8 A, B;
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                  A[i] = (int)a0[i]; A[4 + i] = (int)a1[i];
                  B[i] = (int)bw[c][0][i]; B[4 + i] = (int)bw[c][1][i];
                }
                if constexpr (BLOCK) {
                  // rows 16mt + 4g .. + 3 of the lane's accumulator (4-row tiles: lanes g > 0
                  // hold the copied rows 4..15, scaled by 0 here and never stored)
                  const f32x4 P = mfma16x16x128_fp8(A, B, f32x4{0.f, 0.f, 0.f, 0.f});
                  const int rs = (q * RCR + lc) * BM + 16 * mt + 4 * g;
                  const f32x4 sa4 = (16 * mt + 4 * g + 3 < BM) ? *(const f32x4*)&sSA[rs] : f32x4{0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                  for (int i = 0; i < 4; ++i) acc[mt][i] = __builtin_fmaf(sa4[i] * swb[c], P[i], acc[mt][i]);
                } else {
                  acc[mt] = mfma16x16x128_fp8(A, B, acc[mt]);
                }
              }
            } else if constexpr (WP == WP_FP4 && AF == A_FP8) {
              // e4m3 activations x e2m1 weights, natively: the lane's 16-byte unit is the
              // e2m1 operand of one 16x16x128 scaled MFMA (k = 32g + i at nibble i, low nibble
              // first), and the UE8M0 exponent of those 32 K (group 4*chunk + g) is its block
              // scale.  The e4m3 operand of lane g holds k = 16g .. 16g+15 in its first 16
              // bytes and k = 64 + 16g .. in the other 16 (the fp8 operand's K order).
              const int e8 = sS[slot * 64 + g * 16 + r];
              i32x8 B;
    #pragma unroll
              for (int i = 0; i < 4; ++i) { B[i] = (int)bw[c][0][i]; B[4 + i] = 0; }
    #pragma unroll
              for (int mt = 0; mt < NMT; ++mt) {
                const uint8_t* ap = arow0 + (16 * mt + ar) * AROW + 16 * g;
                const u32x4 a0 = *(const u32x4*)ap, a1 = *(const u32x4*)(ap + 64);
                i32x8 A;
    #pragma unroll
                for (int i = 0; i < 4; ++i) { A[i] = (int)a0[i]; A[4 + i] = (int)a1[i]; }
                acc[mt] = mfma16x16x128_fp8_fp4(A, B, e8, acc[mt]);
              }
            } else if constexpr (WP == WP_FP4) {
              // group 32 == one 16-byte unit: the lane's scale is group 4*chunk + g
              const uint32_t e8 = sS[slot * 64 + g * 16 + r];
              const float sc = e8 == 0 ? __uint_as_float(0x00400000u)
                                       : (e8 == 255 ? __uint_as_float(0x7fc00000u) : __uint_as_float(e8 << 23));
    #pragma unroll
              for (int j = 0; j < 4; ++j) {
                const u32x4 b = fp4_to_16<AF>(bw[c][0][j], sc);
    #pragma unroll
                for (int mt = 0; mt < NMT; ++mt) {
                  u32x4 av = *(const u32x4*)(arow0 + (16 * mt + ar) * AROW + (32 * g + 8 * j) * 2);
                  acc[mt] = mfma16x16x32<AF>(av, b, acc[mt]);
                }
              }
            } else {
              // int4 / uint4 through the magic-number operand, promotion per chunk.
              constexpr int MAF = (AF == A_FP8) ? A_BF16 : AF;   // e4m3 activations run as bf16
              constexpr bool QUAD = (WP == WP_INT4Q_MAGIC);
              constexpr uint32_t ONE2 = (MAF == A_F16) ? 0x3C003C00u : 0x3F803F80u;
              const u32x4 ones = {ONE2, ONE2, ONE2, ONE2};
              f32x4 P[NMT], R[NMT];
    #pragma unroll
              for (int mt = 0; mt < NMT; ++mt) {
                P[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
                R[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
              }
    #pragma unroll
              for (int j = 0; j < 4; ++j) {
                uint32_t wj = bw[c][0][j];
                if constexpr (QUAD) wj ^= 0x88888888u;      // two's complement -> q + 8
                const u32x4 b = magic4<MAF>(wj);
    #pragma unroll
                for (int mt = 0; mt < NMT; ++mt) {
                  u32x4 av;
                  if constexpr (AF == A_FP8) {
                    const u32x2 e = *(const u32x2*)(arow0 + (16 * mt + ar) * AROW + 32 * g + 8 * j);
                    av = e4m3x8_to_bf16_quad(e[0], e[1]);
                  } else {
                    av = *(const u32x4*)(arow0 + (16 * mt + ar) * AROW + (32 * g + 8 * j) * 2);
                    if constexpr (QUAD) av = a16_to_quad(av);
                  }
                  if constexpr (!RSUM) R[mt] = mfma16x16x32<MAF>(av, ones, R[mt]);
                  P[mt] = mfma16x16x32<MAF>(av, b, P[mt]);
                }
              }
              if constexpr (RSUM) {
                // rows 16mt + 4g .. + 3 of the lane's accumulator
                const int rslot = q * RCR + lc;
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt)
                  R[mt] = (16 * mt + 4 * g + 3 < BM) ? *(const f32x4*)&sR[rslot * BM + 16 * mt + 4 * g]
                                                     : f32x4{0.f, 0.f, 0.f, 0.f};
              }
              const uint32_t sbits = ((const uint16_t*)sS)[slot * 16 + r];
              const float sp = (ST == S_F16 ? f16_bits_to_f32(sbits) : bf16_bits_to_f32(sbits)) *
                               MagicConst<MAF>::kInvStep;
              float zc;
              if constexpr (ZERO) {
                const uint32_t zw = sZ[slot * 2 + (r >> 3)];
                zc = 1.0f + (float)((zw >> ((r & 7) * 4)) & 0xF) * (1.0f / MagicConst<MAF>::kInvStep);
              } else {
                zc = 1.0f + 8.0f * (1.0f / MagicConst<MAF>::kInvStep);
              }
    #pragma unroll
              for (int mt = 0; mt < NMT; ++mt)
    #pragma unroll
                for (int i = 0; i < 4; ++i) acc[mt][i] = __builtin_fmaf(sp, __builtin_fmaf(-zc, R[mt][i], P[mt][i]), acc[mt][i]);
            }
        }
        __syncthreads();   // LDS is rewritten by the next round
      }
    }
  }

  // ---- add the K parts through LDS (fixed order) and store ------------------------------
  // (the activation buffer is free after the last round's barrier)
  typedef float RedRow[NCB * 16 + 1];
  static_assert(sizeof(float) * KQ * BM * (NCB * 16 + 1) <= sizeof(sA), "reduction buffer");
  RedRow* sRed0 = reinterpret_cast<RedRow*>(sA);
  auto sRed = [&](int p, int row) -> float* { return sRed0[p * BM + row]; };
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (16 * mt + 4 * g + i < BM) sRed(q, 16 * mt + 4 * g + i)[16 * cb + r] = acc[mt][i];
  __syncthreads();
  uint16_t* yb = (uint16_t*)a.y;
  constexpr int BN = NCB * 16;
  for (int idx = tid; idx < BM * BN; idx += NTHR) {
    const int row = idx / BN, col = idx - row * BN;
    const int tok = sRowTok[row];
    const int64_t n = (int64_t)blockIdx.x * BN + col;
    if (tok < 0 || n >= a.n) continue;
    float v = 0.f;
#pragma unroll
    for (int p = 0; p < KQ; ++p) v += sRed(p, row)[col];
    if (ksl > 1) {                                    // partial sum of this K slice, unscaled
      a.part[((int64_t)blockIdx.z * a.m + rowbase + row) * a.n + n] = v;
      continue;
    }
    if constexpr (WP == WP_FP8) v *= ((const float*)a.s)[(int64_t)expert * a.n + n];
    if constexpr (AF == A_FP8 && !BLOCK) v *= a.x_scale[tok];
    int64_t orow;
    if constexpr (MOE) orow = a.sorted_ids[rowbase + row];
    else orow = rowbase + row;
    yb[orow * a.n + n] = f32_to_out<OF>(v);
  }
}

// ---- launch helpers (instantiated per weight path in qg_stream_*.hip) --------------
template <int WP, int AF, int OF, int ST, bool ZERO, int MT, int NCB, int KQ, bool MOE>
static void launch_one(const StreamArgs& a, const StreamTile& t, hipStream_t st) {
  hipLaunchKernelGGL((stream_gemm_kernel<WP, AF, OF, ST, ZERO, MT, NCB, KQ, MOE>),
                     dim3(t.grid_x, t.grid_y, a.ksplit > 1 ? a.ksplit : 1),
                     dim3(64 * NCB * KQ), 0, st, a);
}

// Shapes: (NCB, KQ) = (2, 4) for 4-bit weights, (1, 8) for e4m3 weights; MoE blocks with
// 4-bit weights (8, 1): 128 columns per workgroup, so a block's activation rows are staged
// by 4x fewer workgroups and no K parts need adding (the grid has blocks to spare; a dense
// layer needs the K parts to fill the GPU).
template <int WP, int AF, int OF, int ST, bool ZERO, bool MOE, int NCB, int KQ>
static bool launch_shape(const StreamArgs& a, const StreamTile& t, hipStream_t st) {
  switch (t.mt) {
    case 0: launch_one<WP, AF, OF, ST, ZERO, 0, NCB, KQ, MOE>(a, t, st); return true;
    case 1: launch_one<WP, AF, OF, ST, ZERO, 1, NCB, KQ, MOE>(a, t, st); return true;
    case 2: launch_one<WP, AF, OF, ST, ZERO, 2, NCB, KQ, MOE>(a, t, st); return true;
    case 4: launch_one<WP, AF, OF, ST, ZERO, 4, NCB, KQ, MOE>(a, t, st); return true;
    default: return false;
  }
}

template <int WP, int AF, int OF, int ST, bool ZERO, bool MOE>
static bool launch_mt(const StreamArgs& a, const StreamTile& t, hipStream_t st) {
  if constexpr (WP == WP_FP8 || WP == WP_FP8_BLOCK) {
    if (t.ncb == 1 && t.kq == 8) return launch_shape<WP, AF, OF, ST, ZERO, MOE, 1, 8>(a, t, st);
    if constexpr (!MOE)
      if (t.ncb == 8 && t.kq == 1) return launch_shape<WP, AF, OF, ST, ZERO, MOE, 8, 1>(a, t, st);
  } else {
    if (t.ncb == 2 && t.kq == 4) return launch_shape<WP, AF, OF, ST, ZERO, MOE, 2, 4>(a, t, st);
    if (t.ncb == 8 && t.kq == 1) return launch_shape<WP, AF, OF, ST, ZERO, MOE, 8, 1>(a, t, st);
  }
  return false;
}

template <int WP, int AF, int OF, int ST, bool ZERO>
static bool launch_stream_variant(const StreamArgs& a, const StreamTile& t, bool moe, hipStream_t st) {
  return moe ? launch_mt<WP, AF, OF, ST, ZERO, true>(a, t, st) : launch_mt<WP, AF, OF, ST, ZERO, false>(a, t, st);
}

}  // namespace qg
