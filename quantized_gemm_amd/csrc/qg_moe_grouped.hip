// Block map of the grouped MoE input organizations ("Humming" wiki article, "Device and
// workload selection": grouped-contiguous execution keeps each expert's rows together,
// grouped-masked execution gives each expert its own storage with a count of valid rows).
// Both name input rows directly, so the map is the indexed path's contract with one expert
// per row: for each expert in ascending order its rows in ascending order, padded with the
// sentinel rows_total to a multiple of block_m; the expert of every block; the padded total.
//   contiguous: expert e owns rows [offsets[e], offsets[e+1]);
//   masked:     expert e owns rows e*cap .. e*cap + counts[e] - 1 (counts clamped to [0, cap]).
// One launch of G workgroups and no scratch memory: every workgroup recomputes the padded
// counts and their scan over experts in LDS (at most kGmapMaxExperts), then writes its own
// range of positions and blocks, finding each one's expert by binary search over the starts.
// Offsets are clamped to [0, rows_total] and made non-decreasing, so malformed input gives a
// wrong map but never a write outside the caller's buffers.
#include "qg_device.h"
#include "qg_kernels.h"

namespace qg {

constexpr int kGmapThreads = 256;
constexpr int kGmapMaxExperts = 1024;
constexpr int kGmapPerGroup = 8192;   // positions per workgroup (before the cap below)
constexpr int kGmapMaxGroups = 256;
constexpr int kGmapPerThread = kGmapMaxExperts / kGmapThreads;

__global__ __launch_bounds__(kGmapThreads) void grouped_map_kernel(const int32_t* __restrict__ arr, int masked,
                                                                   int experts, int64_t rows_total, int cap,
                                                                   int block_m, int32_t* __restrict__ sorted_ids,
                                                                   int64_t cap_sorted, int32_t* __restrict__ expert_ids,
                                                                   int64_t cap_blocks, int32_t* num_post_pad) {
  __shared__ int64_t s_base[kGmapMaxExperts];
  __shared__ int s_cnt[kGmapMaxExperts];
  __shared__ int64_t s_start[kGmapMaxExperts + 1];
  __shared__ int64_t s_part[kGmapThreads];
  const int tid = threadIdx.x;

  // 1. rows of each expert
  if (masked) {
    for (int e = tid; e < experts; e += kGmapThreads) {
      s_base[e] = (int64_t)e * cap;
      s_cnt[e] = min(max(arr[e], 0), cap);
    }
  } else {
    // offsets clamped to [0, rows_total], then made non-decreasing by a prefix maximum
    // (Hillis-Steele in LDS): expert e owns [c[e], c[e+1])
    constexpr int U = (kGmapMaxExperts + kGmapThreads) / kGmapThreads;   // entries 0..E per thread
    for (int i = tid; i <= experts; i += kGmapThreads) s_start[i] = min(max((int64_t)arr[i], (int64_t)0), rows_total);
    __syncthreads();
    for (int off = 1; off <= experts; off <<= 1) {
      int64_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = tid + kGmapThreads * u;
        v[u] = i <= experts ? (i >= off ? max(s_start[i], s_start[i - off]) : s_start[i]) : 0;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = tid + kGmapThreads * u;
        if (i <= experts) s_start[i] = v[u];
      }
      __syncthreads();
    }
    for (int e = tid; e < experts; e += kGmapThreads) {
      s_base[e] = s_start[e];
      s_cnt[e] = (int)(s_start[e + 1] - s_start[e]);
    }
  }
  __syncthreads();

  // 2. exclusive scan of the padded counts: kGmapPerThread experts per thread, then a
  // Hillis-Steele scan of the per-thread sums
  int64_t local[kGmapPerThread];
  int64_t sum = 0;
#pragma unroll
  for (int i = 0; i < kGmapPerThread; ++i) {
    const int e = tid * kGmapPerThread + i;
    const int64_t c = e < experts ? s_cnt[e] : 0;
    local[i] = (c + block_m - 1) / block_m * block_m;
    sum += local[i];
  }
  s_part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kGmapThreads; off <<= 1) {
    const int64_t v = tid >= off ? s_part[tid - off] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  int64_t run = s_part[tid] - sum;   // exclusive prefix of this thread's experts
#pragma unroll
  for (int i = 0; i < kGmapPerThread; ++i) {
    const int e = tid * kGmapPerThread + i;
    if (e < experts) s_start[e] = run;
    run += local[i];
  }
  const int64_t total = min(s_part[kGmapThreads - 1], cap_sorted);
  if (tid == 0) s_start[experts] = s_part[kGmapThreads - 1];
  __syncthreads();

  // the expert whose padded segment holds position p < total: the last e with start <= p
  // (empty experts have start == the next start and are skipped by taking the last)
  auto expert_of = [&](int64_t p) -> int {
    int lo = 0, hi = experts - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_start[mid] <= p) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };

  // 3. this workgroup's positions
  const int64_t chunk = (cap_sorted + gridDim.x - 1) / gridDim.x;
  const int64_t p0 = min(cap_sorted, (int64_t)blockIdx.x * chunk), p1 = min(cap_sorted, p0 + chunk);
  const int sentinel = (int)rows_total;
  for (int64_t p = p0 + tid; p < p1; p += kGmapThreads) {
    int v = sentinel;
    if (p < total) {
      const int e = expert_of(p);
      const int64_t i = p - s_start[e];
      if (i < s_cnt[e]) v = (int)(s_base[e] + i);
    }
    sorted_ids[p] = v;
  }
  // 4. this workgroup's blocks
  const int64_t chunkb = (cap_blocks + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = min(cap_blocks, (int64_t)blockIdx.x * chunkb), b1 = min(cap_blocks, b0 + chunkb);
  for (int64_t b = b0 + tid; b < b1; b += kGmapThreads)
    expert_ids[b] = b * block_m < total ? expert_of(b * block_m) : -1;
  if (blockIdx.x == 0 && tid == 0) *num_post_pad = (int32_t)total;
}

bool launch_grouped_map(const int32_t* arr, bool masked, int experts, int64_t rows_total, int cap, int block_m,
                        int32_t* sorted_ids, int64_t cap_sorted, int32_t* expert_ids, int64_t cap_blocks,
                        int32_t* num_post_pad, hipStream_t st) {
  if (experts <= 0 || experts > kGmapMaxExperts) return false;
  const int64_t g = min((int64_t)kGmapMaxGroups, max((int64_t)1, (cap_sorted + kGmapPerGroup - 1) / kGmapPerGroup));
  hipLaunchKernelGGL(grouped_map_kernel, dim3((unsigned)g), dim3(kGmapThreads), 0, st, arr, masked ? 1 : 0, experts,
                     rows_total, cap, block_m, sorted_ids, cap_sorted, expert_ids, cap_blocks, num_post_pad);
  return true;
}

}  // namespace qg
