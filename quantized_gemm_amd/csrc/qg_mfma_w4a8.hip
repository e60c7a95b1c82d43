// MFMA-bound W4A8 GEMM: int4 weights converted to e4m3 in-kernel, e4m3 activations,
// bf16/f16 scales per group of a multiple of 128 along K, or per output channel.
//
// "Humming: Fast, Flexible Kernels for Quantized Inference" (device paragraphs) and "Ant
// Group's Humming ..." (*Coverage reaches beyond standard PTX types*): weights are stored
// 4-bit and converted inside the kernel into a format the matrix cores multiply natively;
// at larger M the conversion and the scaling are what limits such kernels.  Here:
//   * int4 -> e4m3 is exact (every value in [-8, 7] is an e4m3 value) and costs a byte
//     table lookup (v_perm_b32) per 4 weights, once per workgroup tile;
//   * one 16x16x128 fp8 MFMA covers 128 K, which lies inside one scale group, so its fp32
//     result is promoted into the accumulator with one FMA per output: acc += s[n, g] * P;
//   * the per-token activation scale is applied in the epilogue.
// Tile: 128 rows x 256 columns, 4 waves owning 64 columns each; activations staged in
// LDS (double-buffered, 128-byte row segment per 128-k step, XOR swizzle by row bits
// 1..3), weights and scales HBM -> VGPR two steps ahead.
#include "qg_device.h"
#include "qg_kernels.h"

namespace qg {

template <int OF, int ST, bool MOE>
__global__ __launch_bounds__(256) void mfma_w4a8_kernel(MfmaArgs a) {
  constexpr int BM = 128, BN = 256;
  constexpr int ROWB = 128;                 // one 128-k step of e4m3 activations
  constexpr int STAGE = BM * ROWB;
  constexpr int APT = STAGE / 16 / 256;
  constexpr int MT = BM / 16;               // 16-row MFMA tiles
  constexpr int NT = 4;                     // 16-column MFMA tiles per wave

  __shared__ __attribute__((aligned(16))) uint8_t sA[2 * STAGE];
  __shared__ int sRowTok[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15;
  const int g = lane >> 4;

  int expert = 0;
  int64_t rowbase;
  int ntile;
  if constexpr (MOE) {
    ntile = blockIdx.x;
    rowbase = (int64_t)blockIdx.y * BM;
    if (rowbase >= (int64_t)(*a.num_post_pad)) return;
    expert = a.expert_ids[blockIdx.y];
  } else {
    const int mtiles = (int)((a.m + BM - 1) / BM);
    const int ntiles = (int)gridDim.x / mtiles;
    const int id = blockIdx.x;
    if ((ntiles & 7) == 0) {   // XCD x owns a band of column tiles (see the MFMA kernel)
      const int nper = ntiles >> 3;
      const int x = id & 7, l = id >> 3;
      ntile = x * nper + l % nper;
      rowbase = (int64_t)(l / nper) * BM;
    } else {
      ntile = id / mtiles;
      rowbase = (int64_t)(id - ntile * mtiles) * BM;
    }
  }
  for (int i = tid; i < BM; i += 256) {
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
  const int64_t col0 = (int64_t)ntile * BN + 64 * wave;
  const int nsteps = a.k >> 7;
  const int64_t kun = a.k >> 5;
  const int ngroups = a.group == 0 ? 1 : a.k / a.group;   // group 0: one scale per output channel
  const uint8_t* wbase = a.w + (int64_t)expert * a.w_expert_bytes;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wbase, (uint32_t)a.w_expert_bytes);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (uint32_t)(a.x_rows * a.k));
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.s, a.s_bytes);

  // activation staging (same swizzle as the 16-bit MFMA kernel)
  int a_off[APT];
#pragma unroll
  for (int i = 0; i < APT; ++i) {
    const int p = tid + 256 * i;
    const int row = p >> 3, pc = p & 7;
    const int lc = pc ^ ((row >> 1) & 7);
    const int tok = sRowTok[row];
    a_off[i] = tok < 0 ? -1 : (int)((int64_t)tok * a.k) + 16 * lc;
  }
  auto load_a = [&](int step, u32x4* dst) {
#pragma unroll
    for (int i = 0; i < APT; ++i) dst[i] = bload16(xr, a_off[i] < 0 || step >= nsteps ? kOOB : a_off[i] + step * ROWB);
  };
  auto store_a = [&](int buf, const u32x4* src) {
#pragma unroll
    for (int i = 0; i < APT; ++i) *(u32x4*)(sA + buf * STAGE + (tid + 256 * i) * 16) = src[i];
  };

  int64_t wcol[NT];
  bool wok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    wcol[t] = col0 + 16 * t + r;
    wok[t] = wcol[t] < a.n;
  }
  // weights of a step: one 16-byte unit (32 k of one column) per lane and tile
  auto load_b = [&](int step, u32x4 (&dst)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t nb = wcol[t] >> 4;
      const bool ok = wok[t] && step < nsteps;
      dst[t] = bload16_stream(wr, ok ? (int)(((nb * kun + (int64_t)step * 4 + g) * 16 + r) << 4) : kOOB);
    }
  };
  // scale of group `step` for each tile's column (bf16/f16 bits)
  auto load_s = [&](int step, uint32_t (&dst)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t nb = wcol[t] >> 4;
      const bool ok = wok[t] && step < nsteps;
      const int gi = a.group == 0 ? 0 : (step << 7) / a.group;   // 128-wide step -> scale group
      const int64_t e = (((int64_t)expert * nb_count + nb) * ngroups + gi) * 16 + r;
      dst[t] = __builtin_amdgcn_raw_buffer_load_b16(sr, ok ? (int)(e * 2) : kOOB, 0, 0);
    }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ast[APT];
  u32x4 b0[NT], b1[NT];
  uint32_t s0[NT], s1[NT];
  load_a(0, ast);
  load_b(0, b0);
  load_s(0, s0);
  store_a(0, ast);
  load_a(1, ast);
  load_b(1, b1);
  load_s(1, s1);

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    __syncthreads();
    store_a(buf ^ 1, ast);
    load_a(step + 2, ast);
    const uint8_t* sAb = sA + buf * STAGE;

    // int4 (QUAD order) -> 32 e4m3 bytes per lane and tile, once per step
    i32x8 B[NT];
    float sc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2 e = int4q_to_e4m3(b0[t][j]);
        B[t][2 * j] = (int)e[0];
        B[t][2 * j + 1] = (int)e[1];
      }
      sc[t] = ST == S_F16 ? f16_bits_to_f32(s0[t]) : bf16_bits_to_f32(s0[t]);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = 16 * mt + r;
      const int sw = (row >> 1) & 7;
      const u32x4 a0 = *(const u32x4*)(sAb + row * ROWB + 16 * ((2 * g) ^ sw));
      const u32x4 a1 = *(const u32x4*)(sAb + row * ROWB + 16 * ((2 * g + 1) ^ sw));
      i32x8 A;
#pragma unroll
      for (int i = 0; i < 4; ++i) { A[i] = (int)a0[i]; A[4 + i] = (int)a1[i]; }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const f32x4 P = mfma16x16x128_fp8(A, B[t], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][t][i] = __builtin_fmaf(sc[t], P[i], acc[mt][t][i]);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      b0[t] = b1[t];
      s0[t] = s1[t];
    }
    load_b(step + 2, b1);
    load_s(step + 2, s1);
  }

  // epilogue: lane (r, g) of a 16x16 tile holds column r, rows 4g + i
  uint16_t* yb = (uint16_t*)a.y;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (!wok[t]) continue;
    const int64_t n = wcol[t];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mt + 4 * g + i;
        const int tok = sRowTok[row];
        if (tok < 0) continue;
        int64_t orow;
        if constexpr (MOE) orow = a.sorted_ids[rowbase + row];
        else orow = rowbase + row;
        yb[orow * a.n + n] = f32_to_out<OF>(acc[mt][t][i] * a.x_scale[tok]);
      }
  }
}

bool mfma_w4a8(const MfmaArgs& a, const MfmaTile& t, int wp, int af, int of, int stype, bool zero, bool moe,
               hipStream_t st) {
  if (wp != WP_INT4Q_FP8 || af != A_FP8 || zero || t.bm != 128) return false;
  const dim3 grid(t.grid_x, t.grid_y);
#define QG_W4A8(OF_, ST_)                                                                                  \
  if (of == OF_ && stype == ST_) {                                                                         \
    if (moe) hipLaunchKernelGGL((mfma_w4a8_kernel<OF_, ST_, true>), grid, dim3(256), 0, st, a);            \
    else hipLaunchKernelGGL((mfma_w4a8_kernel<OF_, ST_, false>), grid, dim3(256), 0, st, a);               \
    return true;                                                                                           \
  }
  QG_W4A8(O_BF16, S_BF16)
  QG_W4A8(O_F16, S_F16)
#undef QG_W4A8
  return false;
}

}  // namespace qg
