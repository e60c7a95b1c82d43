// Block-scaled W8A8: e4m3 weights with one float32 scale per 128 x 128 block of (output
// channel, K) and e4m3 activations with one float32 scale per (row, 128-wide K group)
// ("Humming" wiki article, "Quantization representation": block scales share one scale
// across both matrix dimensions).  Neither scale is a power of two, so the matrix cores'
// block exponents cannot carry them: each 128-wide K step is one 16x16x128 fp8 MFMA per
// tile, computed from zero and promoted into the float32 accumulator,
//     acc += (sa[row, step] * sw[n / 128, step]) * P.
// Tile: 128 rows x 256 columns, 8 waves owning 32 columns each (inside one 128-column scale
// block, so sw is one value per wave and step; two waves per SIMD, so one wave's promotion
// arithmetic overlaps the other's matrix products); activations staged through LDS
// (double-buffered, 128-byte row segment per step, XOR swizzle by row bits 1..3), the
// step's 128 row scales staged beside them; weights HBM -> VGPR two steps ahead.  Dense
// shapes with few tiles split K over workgroups (grid z) into fp32 partials that are
// already scaled; the split-K reduction only adds them.
#include "qg_device.h"
#include "qg_kernels.h"

namespace qg {

template <int OF, bool MOE, bool SPLIT, int NW>
__global__ __launch_bounds__(64 * NW) void mfma_fp8_block_kernel(MfmaArgs a) {
  constexpr int BM = 128, BN = 256;
  constexpr int NTHR = 64 * NW;             // NW waves, each owning BN / NW columns
  constexpr int ROWB = 128;                 // one 128-k step of e4m3 activations
  constexpr int STAGE = BM * ROWB;
  constexpr int APT = STAGE / 16 / NTHR;
  constexpr int MT = BM / 16;               // 16-row MFMA tiles
  constexpr int WCOL = BN / NW;
  constexpr int NT = WCOL / 16;             // 16-column MFMA tiles per wave

  __shared__ __attribute__((aligned(16))) uint8_t sA[2 * STAGE];
  __shared__ __attribute__((aligned(16))) float sSA[2][BM];
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
    if ((ntiles & 7) == 0) {   // XCD x (workgroup id mod 8) owns a band of column tiles
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

  const int64_t col0 = (int64_t)ntile * BN + WCOL * wave;   // this wave's first column
  const int ngroups = a.k >> 7;                              // 128-wide K groups = steps
  const int nsteps = SPLIT ? ngroups / a.ksplit : ngroups;
  const int kstep0 = SPLIT ? (int)blockIdx.z * nsteps : 0;
  const int64_t kun = a.k >> 4;                              // 16-byte units along K per column
  const int nblk = a.n >> 7;                                 // 128-column scale blocks
  const uint8_t* wbase = a.w + (int64_t)expert * a.w_expert_bytes;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wbase, (uint32_t)a.w_expert_bytes);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (uint32_t)(a.x_rows * a.k));
  const float* swp = (const float*)a.s + ((int64_t)expert * nblk + min((int64_t)nblk - 1, col0 >> 7)) * ngroups;
  const bool wave_ok = col0 < a.n;

  // activation staging (chunk lc of row `row` at physical chunk lc ^ ((row >> 1) & 7))
  int a_off[APT];
#pragma unroll
  for (int i = 0; i < APT; ++i) {
    const int p = tid + NTHR * i;
    const int row = p >> 3, pc = p & 7;
    const int lc = pc ^ ((row >> 1) & 7);
    const int tok = sRowTok[row];
    a_off[i] = tok < 0 ? -1 : (int)((int64_t)tok * a.k) + 16 * lc;
  }
  const int my_tok = tid < BM ? sRowTok[tid] : -1;
  auto load_a = [&](int step, u32x4* dst, float& sa) {
#pragma unroll
    for (int i = 0; i < APT; ++i)
      dst[i] = bload16(xr, a_off[i] < 0 || step >= nsteps ? kOOB : a_off[i] + (kstep0 + step) * ROWB);
    sa = (my_tok >= 0 && step < nsteps) ? a.x_scale[(int64_t)my_tok * ngroups + kstep0 + step] : 0.f;
  };
  auto store_a = [&](int buf, const u32x4* src, float sa) {
#pragma unroll
    for (int i = 0; i < APT; ++i) *(u32x4*)(sA + buf * STAGE + (tid + NTHR * i) * 16) = src[i];
    if (tid < BM) sSA[buf][tid] = sa;
  };

  int64_t wcol[NT];
  bool wok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    wcol[t] = col0 + 16 * t + r;
    wok[t] = wcol[t] < a.n;
  }
  // weights of a step: units 8*step + 2g, 2g + 1 (k = 128*step + 32g .. + 31) per lane and tile
  auto load_b = [&](int step, u32x4 (&dst)[NT][2], float& sw) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t nb = wcol[t] >> 4;
      const bool ok = wok[t] && step < nsteps;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t ku = (int64_t)(kstep0 + step) * 8 + 2 * g + u;
        dst[t][u] = bload16_stream(wr, ok ? (int)(((nb * kun + ku) * 16 + r) << 4) : kOOB);
      }
    }
    sw = (wave_ok && step < nsteps) ? swp[kstep0 + step] : 0.f;
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ast[APT];
  float sa_st = 0.f;
  u32x4 b0[NT][2], b1[NT][2];
  float sw0 = 0.f, sw1 = 0.f;
  load_a(0, ast, sa_st);
  load_b(0, b0, sw0);
  store_a(0, ast, sa_st);
  load_a(1, ast, sa_st);
  load_b(1, b1, sw1);

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    __syncthreads();
    store_a(buf ^ 1, ast, sa_st);
    load_a(step + 2, ast, sa_st);
    const uint8_t* sAb = sA + buf * STAGE;

    i32x8 B[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) { B[t][i] = (int)b0[t][0][i]; B[t][4 + i] = (int)b0[t][1][i]; }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = 16 * mt + r;
      const int sw = (row >> 1) & 7;
      const u32x4 a0 = *(const u32x4*)(sAb + row * ROWB + 16 * ((2 * g) ^ sw));
      const u32x4 a1 = *(const u32x4*)(sAb + row * ROWB + 16 * ((2 * g + 1) ^ sw));
      i32x8 A;
#pragma unroll
      for (int i = 0; i < 4; ++i) { A[i] = (int)a0[i]; A[4 + i] = (int)a1[i]; }
      // the lane's accumulator rows 16mt + 4g + i: their activation scales times the block's
      const f32x4 sa4 = *(const f32x4*)&sSA[buf][16 * mt + 4 * g];
      float c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = sa4[i] * sw0;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const f32x4 P = mfma16x16x128_fp8(A, B[t], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][t][i] = __builtin_fmaf(c[i], P[i], acc[mt][t][i]);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      b0[t][0] = b1[t][0];
      b0[t][1] = b1[t][1];
    }
    sw0 = sw1;
    load_b(step + 2, b1, sw1);
  }

  // epilogue: lane (r, g) of a 16x16 tile holds column r, rows 4g + i (scales applied)
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (!wok[t]) continue;
    const int64_t n = wcol[t];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mt + 4 * g + i;
        if (sRowTok[row] < 0) continue;
        if constexpr (SPLIT) {
          a.part[((int64_t)blockIdx.z * a.m + rowbase + row) * a.n + n] = acc[mt][t][i];
        } else {
          int64_t orow;
          if constexpr (MOE) orow = a.sorted_ids[rowbase + row];
          else orow = rowbase + row;
          ((uint16_t*)a.y)[orow * a.n + n] = f32_to_out<OF>(acc[mt][t][i]);
        }
      }
  }
}

bool mfma_fp8_block(const MfmaArgs& a, const MfmaTile& t, int wp, int af, int of, int stype, bool zero, bool moe,
                    hipStream_t st) {
  if (wp != WP_FP8_BLOCK || af != A_FP8 || stype != S_F32 || zero || t.bm != 128) return false;
  const dim3 grid(t.grid_x, t.grid_y, t.ksplit > 1 ? t.ksplit : 1);
  constexpr int NW = 8;
#define QG_FP8B(OF_)                                                                                        \
  if (of == OF_) {                                                                                          \
    if (moe) hipLaunchKernelGGL((mfma_fp8_block_kernel<OF_, true, false, NW>), grid, dim3(64 * NW), 0, st, a); \
    else if (t.ksplit > 1)                                                                                  \
      hipLaunchKernelGGL((mfma_fp8_block_kernel<OF_, false, true, NW>), grid, dim3(64 * NW), 0, st, a);    \
    else hipLaunchKernelGGL((mfma_fp8_block_kernel<OF_, false, false, NW>), grid, dim3(64 * NW), 0, st, a); \
    return true;                                                                                            \
  }
  QG_FP8B(O_BF16)
  QG_FP8B(O_F16)
#undef QG_FP8B
  return false;
}

}  // namespace qg
