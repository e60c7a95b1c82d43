// Token-to-expert sort and padding for the indexed MoE path ("Humming" wiki article,
// "Device and workload selection": the indexed organization reads each expert's input
// rows through the routing indices).  Counting sort, deterministic and stable, in one launch of G workgroups with
// no scratch memory: workgroup g owns the contiguous flat-index range [r0, r1).
//   1. every workgroup counts the expert ids of the whole list (a few hundred KB at most,
//      read from L2): ids before its range, after it, and inside it per wave (each of its
//      waves owns a contiguous part of the range);
//   2. padded counts and their exclusive scan over experts (the same in every
//      workgroup); the base of wave w for expert e is the expert's offset plus the ids of
//      e before the range plus those of the earlier waves;
//   3. each wave walks its part in order and places every flat index at its base plus
//      its rank among equal ids within the 64-lane chunk (ranks from bitwise match masks
//      built with ballots), so within an expert the order is ascending flat index;
//   4. workgroup 0 writes the block -> expert map, the sentinel padding, the tails and
//      the padded total.
// Reads go in batches of kAlignBatch 64-id chunks per wave with all loads of a batch in
// flight (one load latency per batch, not per chunk).
#include "qg_device.h"
#include "qg_kernels.h"

namespace qg {

constexpr int kAlignWaves = 16;
constexpr int kAlignMaxExperts = 512;
constexpr int kAlignBatch = 8;
constexpr int kAlignPerGroup = 2048;    // flat indices per workgroup (before the cap below)
constexpr int kAlignMaxGroups = 64;

__global__ __launch_bounds__(64 * kAlignWaves) void moe_align_kernel(const int32_t* __restrict__ ids, int tk,
                                                                      int experts, int block_m,
                                                                      int32_t* __restrict__ sorted_ids,
                                                                      int64_t cap_sorted,
                                                                      int32_t* __restrict__ expert_ids,
                                                                      int64_t cap_blocks, int32_t* num_post_pad) {
  __shared__ int hist[kAlignWaves][kAlignMaxExperts];   // per-wave counts, then per-wave bases
  __shared__ int before[kAlignMaxExperts];
  __shared__ int after[kAlignMaxExperts];
  __shared__ int offs[kAlignMaxExperts + 1];
  __shared__ int cnts[kAlignMaxExperts];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int i = tid; i < kAlignWaves * kAlignMaxExperts; i += blockDim.x) (&hist[0][0])[i] = 0;
  for (int i = tid; i < kAlignMaxExperts; i += blockDim.x) { before[i] = 0; after[i] = 0; }
  __syncthreads();

  // this workgroup's range and its waves' parts
  const int chunk = (tk + (int)gridDim.x - 1) / (int)gridDim.x;
  const int r0 = min(tk, (int)blockIdx.x * chunk), r1 = min(tk, r0 + chunk);
  const int per = (chunk + kAlignWaves - 1) / kAlignWaves;
  const int f0 = min(r1, r0 + wave * per);
  const int f1 = min(r1, f0 + per);

  // 1. counts over the whole list
  for (int fb = 64 * kAlignBatch * wave; fb < tk; fb += 64 * kAlignBatch * kAlignWaves) {
    int eb[kAlignBatch];
#pragma unroll
    for (int u = 0; u < kAlignBatch; ++u) {
      const int f = fb + 64 * u + lane;
      eb[u] = f < tk ? ids[f] : -1;
    }
#pragma unroll
    for (int u = 0; u < kAlignBatch; ++u) {
      const int f = fb + 64 * u + lane;
      const int e = eb[u];
      if (e < 0 || e >= experts) continue;
      if (f < r0) atomicAdd(&before[e], 1);
      else if (f >= r1) atomicAdd(&after[e], 1);
      else atomicAdd(&hist[(f - r0) / per][e], 1);
    }
  }
  __syncthreads();

  // 2. counts, padding, scan (wave 0, 64 experts per step), bases
  if (wave == 0) {
    int carry = 0;
    for (int e0 = 0; e0 < experts; e0 += 64) {
      const int e = e0 + lane;
      int c = 0;
      if (e < experts) {
        c = before[e] + after[e];
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
    int b = offs[e] + before[e];
    for (int w = 0; w < kAlignWaves; ++w) {
      const int h = hist[w][e];
      hist[w][e] = b;   // becomes the base of wave w for expert e
      b += h;
    }
    if (blockIdx.x == 0) {
      const int blk0 = offs[e] / block_m, blk1 = offs[e + 1] / block_m;
      for (int blk = blk0; blk < blk1; ++blk) expert_ids[blk] = e;
      for (int s = offs[e] + cnts[e]; s < offs[e + 1]; ++s) sorted_ids[s] = tk;
    }
  }
  if (blockIdx.x == 0) {
    if (tid == 0) *num_post_pad = total;
    for (int64_t s = total + tid; s < cap_sorted; s += blockDim.x) sorted_ids[s] = tk;
    for (int64_t b = total / block_m + tid; b < cap_blocks; b += blockDim.x) expert_ids[b] = -1;
  }
  __syncthreads();

  // 3. stable scatter of this wave's part
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int fbb = f0; fbb < f1; fbb += 64 * kAlignBatch) {
    int eb[kAlignBatch];
#pragma unroll
    for (int u = 0; u < kAlignBatch; ++u) {
      const int f = fbb + 64 * u + lane;
      eb[u] = f < f1 ? ids[f] : -1;
    }
#pragma unroll
    for (int u = 0; u < kAlignBatch; ++u) {
      const int f = fbb + 64 * u + lane;
      const bool in = f < f1;
      const int e = eb[u];
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
}

void launch_moe_align(const int32_t* ids, int tk, int experts, int block_m, int32_t* sorted_ids, int64_t cap_sorted,
                      int32_t* expert_ids, int64_t cap_blocks, int32_t* num_post_pad, hipStream_t st) {
  const int groups = std::max(1, std::min(kAlignMaxGroups, (tk + kAlignPerGroup - 1) / kAlignPerGroup));
  hipLaunchKernelGGL(moe_align_kernel, dim3(groups), dim3(64 * kAlignWaves), 0, st, ids, tk, experts, block_m,
                     sorted_ids, cap_sorted, expert_ids, cap_blocks, num_post_pad);
}

}  // namespace qg
