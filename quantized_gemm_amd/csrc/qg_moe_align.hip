// Token-to-expert sort and padding for the indexed MoE path ("Humming" wiki article,
// "Device and workload selection": an indexed path gathers input rows through routing
// indices).  Counting sort in one workgroup, deterministic and stable:
//   1. per-wave histograms of expert ids over contiguous ranges of the flat index;
//   2. padded counts, exclusive scan over experts, per-wave bases, block->expert map;
//   3. each wave walks its range in order and places every flat index at
//      base[wave][e] + its rank among equal ids within the 64-lane chunk (ranks from
//      bitwise match masks built with ballots), so within an expert the order is
//      ascending flat index;
//   4. sentinel padding and tails.
#include "qg_device.h"
#include "qg_kernels.h"

namespace qg {

constexpr int kAlignWaves = 16;
constexpr int kAlignMaxExperts = 512;

__global__ __launch_bounds__(64 * kAlignWaves) void moe_align_kernel(const int32_t* __restrict__ ids, int tk,
                                                                      int experts, int block_m,
                                                                      int32_t* __restrict__ sorted_ids,
                                                                      int64_t cap_sorted,
                                                                      int32_t* __restrict__ expert_ids,
                                                                      int64_t cap_blocks, int32_t* num_post_pad) {
  __shared__ int hist[kAlignWaves][kAlignMaxExperts];
  __shared__ int offs[kAlignMaxExperts + 1];
  __shared__ int cnts[kAlignMaxExperts];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int i = tid; i < kAlignWaves * kAlignMaxExperts; i += blockDim.x) (&hist[0][0])[i] = 0;
  __syncthreads();

  const int per = (tk + kAlignWaves - 1) / kAlignWaves;
  const int f0 = wave * per;
  const int f1 = min(tk, f0 + per);

  // 1. histograms
  for (int f = f0 + lane; f < f1; f += 64) {
    const int e = ids[f];
    if (e >= 0 && e < experts) atomicAdd(&hist[wave][e], 1);
  }
  __syncthreads();

  // 2. counts, padding, scan (wave 0, 64 experts per step), bases
  if (wave == 0) {
    int carry = 0;
    for (int e0 = 0; e0 < experts; e0 += 64) {
      const int e = e0 + lane;
      int c = 0;
      if (e < experts) {
        for (int w = 0; w < kAlignWaves; ++w) c += hist[w][e];
        cnts[e] = c;
      }
      const int p = (c + block_m - 1) / block_m * block_m;
      int incl = p;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
      }
      if (e < experts) offs[e] = carry + incl - p;
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) offs[experts] = carry;
  }
  __syncthreads();
  const int total = offs[experts];
  for (int e = tid; e < experts; e += blockDim.x) {
    int b = offs[e];
    for (int w = 0; w < kAlignWaves; ++w) {
      const int h = hist[w][e];
      hist[w][e] = b;   // becomes the base of wave w for expert e
      b += h;
    }
    const int blk0 = offs[e] / block_m, blk1 = offs[e + 1] / block_m;
    for (int blk = blk0; blk < blk1; ++blk) expert_ids[blk] = e;
    for (int s = offs[e] + cnts[e]; s < offs[e + 1]; ++s) sorted_ids[s] = tk;
  }
  if (tid == 0) *num_post_pad = total;
  for (int64_t s = total + tid; s < cap_sorted; s += blockDim.x) sorted_ids[s] = tk;
  for (int64_t b = total / block_m + tid; b < cap_blocks; b += blockDim.x) expert_ids[b] = -1;
  __syncthreads();

  // 3. stable scatter
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int fb = f0; fb < f1; fb += 64) {
    const int f = fb + lane;
    const bool in = f < f1;
    const int e = in ? ids[f] : -1;
    const bool valid = in && e >= 0 && e < experts;
    // lanes holding the same expert id: AND of per-bit ballots
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
      const uint64_t b = __ballot(valid && ((e >> bit) & 1));
      same &= ((e >> bit) & 1) ? b : ~b;
    }
    int base = 0;
    if (valid) {
      base = hist[wave][e];
      sorted_ids[base + __popcll(same & lt)] = f;
    }
    // the lowest lane of each id class advances that class's base
    if (valid && (same & lt) == 0) hist[wave][e] = base + __popcll(same);
  }
}

void launch_moe_align(const int32_t* ids, int tk, int experts, int block_m, int32_t* sorted_ids, int64_t cap_sorted,
                      int32_t* expert_ids, int64_t cap_blocks, int32_t* num_post_pad, hipStream_t st) {
  hipLaunchKernelGGL(moe_align_kernel, dim3(1), dim3(64 * kAlignWaves), 0, st, ids, tk, experts, block_m, sorted_ids,
                     cap_sorted, expert_ids, cap_blocks, num_post_pad);
}

}  // namespace qg
