// Host-visible launch interfaces of the device kernels (internal to libqg.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

// Arguments of the weight-streaming GEMM (dense and MoE).
struct StreamArgs {
  const uint8_t* w;          // prepared W region
  const void* s;             // prepared S region
  const uint32_t* z;         // prepared Z region or null
  const void* x;             // activations [rows][k]
  const float* x_scale;      // per-row scales for e4m3 activations
  void* y;                   // output [rows][n]
  int64_t m;                 // dense rows
  int64_t x_rows;            // rows of x (dense: m, MoE: tokens)
  uint32_t s_bytes, z_bytes; // sizes of the S / Z regions (all experts)
  int n, k, group;
  int64_t w_expert_bytes;
  const int32_t* sorted_ids; // MoE only
  const int32_t* expert_ids;
  const int32_t* num_post_pad;
  int topk, sentinel;
  float* part;               // split K: fp32 partial sums [ksplit][m][n] (workspace)
  int ksplit;                // K slices (1: none)
};

struct StreamTile {
  int mt;                    // row tiles of 16 rows per workgroup
  int ncb, kq;               // 16-column blocks x K parts = waves per workgroup
  unsigned grid_x, grid_y;
};

// The MFMA-bound kernel takes the same arguments.
typedef StreamArgs MfmaArgs;
struct MfmaTile {
  int bm;                    // rows per workgroup tile (128 or 256); 256 columns per tile
  unsigned grid_x, grid_y;   // dense: grid_x = all tiles; MoE: grid_x = column tiles, grid_y = blocks
  int ksplit;                // dense, 128-row tiles: K slices (grid z), 1 = none
};
bool launch_mfma_gemm(const MfmaArgs& a, const MfmaTile& t, int wp, int af, int of, int stype, bool zero, bool moe,
                      hipStream_t st);

// Sum of the split-K partials a.part[ksplit][m][n] into a.y, with the e4m3 per-channel
// (w_scale, fp8 weights) and per-token (a.x_scale, e4m3 activations) scales.
bool launch_split_reduce(const MfmaArgs& a, bool w_scale, bool x_scale, int of, hipStream_t st);

bool launch_stream_gemm(const StreamArgs& a, const StreamTile& t, int wp, int af, int of, int stype, bool zero,
                        bool moe, hipStream_t st);

// Weight transform kernels.
struct RepackArgs {
  const void* w; const void* s; const uint8_t* z;
  uint8_t* out_w; uint8_t* out_s; uint32_t* out_z;
  int experts, n, k, groups;
  int w4;                    // 1: 4-bit codes, 0: e4m3 bytes
  int order;                 // 0 natural, 1 pair, 2 quad
  int bias8;                 // xor every nibble with 8
  int s_bytes;               // bytes per scale element
  int64_t s_plain;           // > 0: block scales, this many 4-byte elements copied as they are
};
void launch_repack(const RepackArgs& a, hipStream_t st);

struct DequantArgs {
  const uint8_t* w; const void* s; const uint32_t* z; float* out;
  int n, k, groups, group, wp, af, stype, zero;
};
void launch_dequant(const DequantArgs& a, hipStream_t st);

// MoE layer steps around the grouped products (qg_moe_layer.hip).  in_t / dtype: O_F16 or
// O_BF16; out_t: A_F16, A_BF16, A_FP8 (out_scale: float32, one scale per row) or A_FP4
// (out: packed e2m1 codes, out_scale: uint8 UE8M0 exponent per 32 outputs).
bool launch_swiglu(const void* gu, int64_t rows, int64_t inter, int in_t, int out_t, void* out, void* out_scale,
                   hipStream_t st);
// Per-row absmax e4m3 quantization of 16-bit rows (in_t O_F16 / O_BF16), k <= 8192, k % 8 == 0.
bool launch_quant_rows_e4m3(const void* x, int64_t rows, int64_t k, int in_t, void* codes, float* scale,
                            hipStream_t st);
// W4A4 MXFP4 (qg_w4a4.hip): e2m1 x e2m1 with UE8M0 exponents on both sides.  bm = rows per
// workgroup (16, 32, 64 or 128; MoE: the align block); dense: grid over a.m, MoE: grid_y blocks.
int w4a4_cols(int bm);
bool launch_w4a4(const StreamArgs& a, int bm, bool moe, int of, unsigned grid_y, hipStream_t st);
// MXFP4 quantization of 16-bit rows (in_t A_F16 / A_BF16), k % 32 == 0.
bool launch_quant_rows_e2m1(const void* x, int64_t rows, int64_t k, int in_t, uint8_t* codes, uint8_t* scales,
                            hipStream_t st);
bool launch_combine(const void* y, const float* w, const int32_t* ids, int64_t tokens, int topk, int experts, int64_t n,
                    int dtype, void* out, hipStream_t st);

// Block map of the grouped-contiguous (offsets [E+1]) or grouped-masked (counts [E], cap rows
// per expert) MoE input organizations; false if the expert count is beyond the kernel's limit.
bool launch_grouped_map(const int32_t* arr, bool masked, int experts, int64_t rows_total, int cap, int block_m,
                        int32_t* sorted_ids, int64_t cap_sorted, int32_t* expert_ids, int64_t cap_blocks,
                        int32_t* num_post_pad, hipStream_t st);

void launch_moe_align(const int32_t* ids, int tk, int experts, int block_m, int32_t* sorted_ids, int64_t cap_sorted,
                      int32_t* expert_ids, int64_t cap_blocks, int32_t* num_post_pad, hipStream_t st);

}  // namespace qg
