// W4A4 MXFP4: e2m1 activations with one UE8M0 exponent per 32 K of a row times e2m1
// weights with one UE8M0 exponent per 32 K of an output channel ("Humming" README, "Key
// Features": FP4 activations and UE8M0 scales; wiki article, "Quantization
// representation": per-group scales).  On gfx950 the scaled 16x16x128 MFMA takes both
// operands as e2m1 codes and both exponents as E8M0 lane operands, so nothing is
// dequantized: operands go HBM -> VGPR as stored.
//
// Operand order of the fp4 x fp4 MFMA: lane (i, g), i = lane % 16, g = lane / 16, holds row
// (A) or column (B) i, K 32g .. 32g + 31 of the 128-wide chunk as 16 bytes with the even K in
// the low nibble, and supplies the exponent of that 32-wide block.  That is 16 contiguous
// bytes of a packed activation row, and one 16-byte unit of the prepared weights.
//
// Used for up to 64 rows, mid M and MoE blocks up to 64, and for batch invariance; larger
// products run on the MFMA kernel (activations staged through LDS).
// Workgroup: KW x WC x WR waves.  Wave (wr, wc, kw) owns rows [16 MT wr, +16 MT) and columns
// [16 NT wc, +16 NT) of the workgroup tile and the K chunks kw, kw + KW, ...; with KW > 1
// the waves' partial sums are added in LDS in wave order (a fixed order), then written by
// the kw = 0 waves.  Each wave keeps three chunks of operands in flight.  Accumulator lane
// (i, g) of a 16x16 tile holds column i, rows 4g .. 4g + 3.
#include "qg_device.h"
#include "qg_kernels.h"

namespace qg {

template <int OF, bool MOE, int MT, int NT, int WR, int WC, int KW>
__global__ __launch_bounds__(64 * WR * WC * KW) void w4a4_kernel(StreamArgs a) {
  constexpr int BMW = WR * 16 * MT;   // rows per workgroup
  constexpr int BNW = WC * 16 * NT;   // columns per workgroup
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave % KW, wc = (wave / KW) % WC, wr = wave / (KW * WC);
  const int li = lane & 15, g = lane >> 4;

  int expert = 0;
  int64_t rowbase;
  int ntile;
  if constexpr (MOE) {
    ntile = blockIdx.x;
    rowbase = (int64_t)blockIdx.y * BMW;
    if (rowbase >= (int64_t)(*a.num_post_pad)) return;
    expert = a.expert_ids[blockIdx.y];
  } else {
    const int mtiles = (int)((a.m + BMW - 1) / BMW);
    const int ntiles = (int)gridDim.x / mtiles;
    const int id = blockIdx.x;
    if ((ntiles & 7) == 0) {   // XCD x (workgroup id mod 8) owns a band of column tiles
      const int nper = ntiles >> 3;
      const int x = id & 7, l = id >> 3;
      ntile = x * nper + l % nper;
      rowbase = (int64_t)(l / nper) * BMW;
    } else {
      ntile = id / mtiles;
      rowbase = (int64_t)(id - ntile * mtiles) * BMW;
    }
  }
  const int row0 = wr * 16 * MT;                           // first workgroup row of this wave
  const int kb = a.k >> 1;                                 // bytes per activation row
  const int kg = a.k >> 5;                                 // 32-wide groups per row
  const int nchunks = a.k >> 7;
  const int nb_count = a.n >> 4;

  // A operand rows of this lane (row li of each 16-row tile): source offsets, -1 if none
  int a_off[MT], s_off[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int64_t rr = rowbase + row0 + 16 * mt + li;
    int tok;
    if constexpr (MOE) {
      const int f = a.sorted_ids[rr];
      tok = f < a.sentinel ? f / a.topk : -1;
    } else {
      tok = rr < a.m ? (int)rr : -1;
    }
    a_off[mt] = tok < 0 ? -1 : tok * kb + 16 * g;
    s_off[mt] = tok < 0 ? -1 : tok * kg;
  }
  // B operand columns: unit 4c + g of column n at ((n/16 * K/32 + 4c + g) * 16 + n%16) * 16
  const int64_t col0 = (int64_t)ntile * BNW + wc * 16 * NT;
  int b_off[NT], sb_off[NT];
  bool wok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t n = col0 + 16 * t + li;
    wok[t] = n < a.n;
    const int64_t nb = min((int64_t)nb_count - 1, n >> 4);
    b_off[t] = (int)(((nb * kg + g) * 16 + li) * 16);
    sb_off[t] = (int)((((int64_t)expert * nb_count + nb) * kg + g) * 16 + li);
  }
  const uint8_t* wbase = a.w + (int64_t)expert * a.w_expert_bytes;
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(wbase, (uint32_t)a.w_expert_bytes);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.s, a.s_bytes);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x, (uint32_t)(a.x_rows * kb));
  const __amdgpu_buffer_rsrc_t xsrs = make_rsrc(a.x_scale, (uint32_t)(a.x_rows * kg));

  struct Frag {
    u32x4 a[MT];
    uint32_t sa[MT];   // the row's 4 exponents of the chunk (one byte per 32-wide group)
    u32x4 b[NT];
    uint32_t sb[NT];
  };
  // chunk it of this wave (c = kw + KW it); past the end every load reads zeros
  auto load = [&](int it, Frag& f) {
    const int c = kw + KW * it;
    const bool ok = c < nchunks;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f.a[mt] = bload16(xrs, ok && a_off[mt] >= 0 ? a_off[mt] + 64 * c : kOOB);
      f.sa[mt] = __builtin_amdgcn_raw_buffer_load_b32(xsrs, ok && s_off[mt] >= 0 ? s_off[mt] + 4 * c : kOOB, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f.b[t] = bload16_stream(wrs, ok && wok[t] ? b_off[t] + 1024 * c : kOOB);
      f.sb[t] = __builtin_amdgcn_raw_buffer_load_b8(srs, ok && wok[t] ? sb_off[t] + 64 * c : kOOB, 0, 0);
    }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      i32x8 A;
#pragma unroll
      for (int i = 0; i < 4; ++i) { A[i] = (int)f.a[mt][i]; A[4 + i] = 0; }
      const int sa = (int)((f.sa[mt] >> (8 * g)) & 0xFFu);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        i32x8 B;
#pragma unroll
        for (int i = 0; i < 4; ++i) { B[i] = (int)f.b[t][i]; B[4 + i] = 0; }
        acc[mt][t] = mfma16x16x128_fp4_fp4(A, B, sa, (int)(f.sb[t] & 0xFFu), acc[mt][t]);
      }
    }
  };

  // three chunks in flight: the loop is unrolled by three so that every slot is a fixed set
  // of registers, and padded to a multiple of three (padded chunks read zeros and add 0)
  const int niter = nchunks > kw ? (nchunks - kw + KW - 1) / KW : 0;
  const int niter3 = (niter + 2) / 3 * 3;
  Frag f0, f1, f2;
  load(0, f0);
  load(1, f1);
  for (int it = 0; it < niter3; it += 3) {
    load(it + 2, f2);
    mma(f0);
    load(it + 3, f0);
    mma(f1);
    load(it + 4, f1);
    mma(f2);
  }

  if constexpr (KW > 1) {
    // partial sums of the kw > 0 waves, [slot][element][lane], added by the kw = 0 wave
    constexpr int EL = MT * NT * 4;
    __shared__ float red[(KW - 1) * WR * WC][EL][64];
    const int rc = wr * WC + wc;
    if (kw > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[(kw - 1) * WR * WC + rc][(mt * NT + t) * 4 + i][lane] = acc[mt][t][i];
    }
    __syncthreads();
    if (kw > 0) return;
#pragma unroll
    for (int q = 1; q < KW; ++q)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][t][i] += red[(q - 1) * WR * WC + rc][(mt * NT + t) * 4 + i][lane];
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t rr = rowbase + row0 + 16 * mt + 4 * g + i;
      int64_t orow;
      if constexpr (MOE) {
        const int f = a.sorted_ids[rr];
        if (f >= a.sentinel) continue;
        orow = f;
      } else {
        if (rr >= a.m) continue;
        orow = rr;
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (wok[t]) ((uint16_t*)a.y)[orow * a.n + col0 + 16 * t + li] = f32_to_out<OF>(acc[mt][t][i]);
    }
}

template <int OF, bool MOE>
static bool launch_w4a4_of(const StreamArgs& a, int bm, unsigned grid_x, unsigned grid_y, hipStream_t st) {
  const dim3 grid(grid_x, grid_y);
  switch (bm) {
    case 16: hipLaunchKernelGGL((w4a4_kernel<OF, MOE, 1, 2, 1, 1, 8>), grid, dim3(512), 0, st, a); return true;
    case 32: hipLaunchKernelGGL((w4a4_kernel<OF, MOE, 2, 4, 1, 1, 8>), grid, dim3(512), 0, st, a); return true;
    case 64: hipLaunchKernelGGL((w4a4_kernel<OF, MOE, 4, 4, 1, 1, 4>), grid, dim3(256), 0, st, a); return true;
    case 128: hipLaunchKernelGGL((w4a4_kernel<OF, MOE, 4, 4, 2, 2, 1>), grid, dim3(256), 0, st, a); return true;
    default: return false;
  }
}

// columns per workgroup: 32- and 64-row workgroups take 64 columns (each row block's
// activations are then re-read by half as many column tiles: 5% faster for MoE blocks of 32,
// 31% for dense M = 128), 16-row workgroups 32 (more workgroups in flight: faster at M <= 16)
int w4a4_cols(int bm) { return bm == 128 ? 128 : bm == 16 ? 32 : 64; }

bool launch_w4a4(const StreamArgs& a, int bm, bool moe, int of, unsigned grid_y, hipStream_t st) {
  const unsigned ntiles = (unsigned)((a.n + w4a4_cols(bm) - 1) / w4a4_cols(bm));
  if (moe) {
    return of == O_BF16 ? launch_w4a4_of<O_BF16, true>(a, bm, ntiles, grid_y, st)
                        : launch_w4a4_of<O_F16, true>(a, bm, ntiles, grid_y, st);
  }
  const unsigned grid_x = ntiles * (unsigned)((a.m + bm - 1) / bm);
  return of == O_BF16 ? launch_w4a4_of<O_BF16, false>(a, bm, grid_x, 1, st)
                      : launch_w4a4_of<O_F16, false>(a, bm, grid_x, 1, st);
}

// ---- MXFP4 activation quantization -----------------------------------------------------
// One thread per 32-element block of a row (mxfp4_encode32: the OCP Microscaling conversion).
template <int IN>
__global__ __launch_bounds__(256) void quant_e2m1_rows_kernel(const uint16_t* x, int64_t blocks, int kg,
                                                               uint8_t* codes, uint8_t* scales) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= blocks) return;
  const int64_t row = b / kg, blk = b - row * kg;
  const u32x4* src = (const u32x4*)(x + row * (int64_t)kg * 32 + blk * 32);
  float v[32];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const u32x4 w = src[p];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = w[j] & 0xFFFFu, hi = w[j] >> 16;
      v[8 * p + 2 * j] = IN == A_BF16 ? bf16_bits_to_f32(lo) : f16_bits_to_f32(lo);
      v[8 * p + 2 * j + 1] = IN == A_BF16 ? bf16_bits_to_f32(hi) : f16_bits_to_f32(hi);
    }
  }
  u32x4 out;
  const uint32_t e8 = mxfp4_encode32(v, out);
  *(u32x4*)(codes + row * (int64_t)kg * 16 + blk * 16) = out;
  scales[b] = (uint8_t)e8;
}

bool launch_quant_rows_e2m1(const void* x, int64_t rows, int64_t k, int in_t, uint8_t* codes, uint8_t* scales,
                            hipStream_t st) {
  const int64_t blocks = rows * (k / 32);
  const unsigned grid = (unsigned)((blocks + 255) / 256);
  if (in_t == A_BF16)
    hipLaunchKernelGGL((quant_e2m1_rows_kernel<A_BF16>), dim3(grid), dim3(256), 0, st, (const uint16_t*)x, blocks,
                       (int)(k / 32), codes, scales);
  else if (in_t == A_F16)
    hipLaunchKernelGGL((quant_e2m1_rows_kernel<A_F16>), dim3(grid), dim3(256), 0, st, (const uint16_t*)x, blocks,
                       (int)(k / 32), codes, scales);
  else
    return false;
  return true;
}

}  // namespace qg
