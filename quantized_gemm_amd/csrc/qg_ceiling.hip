// Measured ceilings of this GPU, the yardsticks next to the published peaks:
//
//  * streaming read: the rate at which a plain kernel reads a buffer once from HBM with
//    16-byte loads, every lane's loads issued before any is used (the access pattern of
//    the weight stream), reduced to one word per wave so the loads cannot be dropped;
//  * MFMA loop: the rate of back-to-back independent MFMAs of one type with operands in
//    registers, two waves per SIMD, nothing else in the loop;
//  * LDS reads: the rate at which 8 waves of a workgroup read their CU's LDS with
//    conflict-free 16-byte reads.
//
// Neither computes anything of the GEMM; both exist so that a kernel's time can be read
// against what the memory system and the matrix cores deliver on the same box.
#include "qg.h"
#include "qg_device.h"
#include "qg_kernels.h"

namespace qg {

template <int U>
__global__ __launch_bounds__(256) void ceiling_read_kernel(const uint8_t* __restrict__ p, uint32_t bytes,
                                                           uint32_t* __restrict__ sink) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(p, bytes);
  const int64_t stride = (int64_t)gridDim.x * 256 * 16;
  const int64_t base = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 16;
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t off = base + u * stride;
    v[u] = bload16_stream(r, off < (int64_t)bytes ? (int)off : kOOB);
  }
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = x;
}

// DT: 0 = bf16 32x32x16, 1 = e4m3 32x32x64, 2 = e2m1 32x32x64 (scaled MFMA, neutral scales).
template <int DT>
__global__ __launch_bounds__(256) void ceiling_mfma_kernel(int64_t iters, float* __restrict__ sink) {
  const uint32_t seed = threadIdx.x * 0x9E3779B9u + blockIdx.x;
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
  if constexpr (DT == 0) {
    u32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = (seed >> i) & 0x3F803F80u;
      b[i] = (seed << i) & 0x3F803F80u;
    }
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = mfma32x32x16<A_BF16>(a, b, acc[i]);
    }
  } else {
    i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (int)((seed >> i) & 0x38383838u);
      b[i] = (int)((seed << i) & 0x38383838u);
    }
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (DT == 1) acc[i] = mfma32x32x64_fp8(a, b, acc[i]);
        else acc[i] = mfma32x32x64_fp4_fp4(a, b, 127, 127, acc[i]);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[i][j];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// LDS reads: 8 waves per workgroup, each lane reading 16 bytes per instruction at
// consecutive addresses (conflict-free), eight instructions in flight per lane.
__global__ __launch_bounds__(512) void ceiling_lds_kernel(int64_t iters, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[65536];
  for (int i = threadIdx.x; i < 65536 / 16; i += 512) *(u32x4*)(buf + 16 * i) = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  const int lane_off = (threadIdx.x & 63) * 16 + (threadIdx.x >> 6) * 8192;
  u32x4 x = {0u, 0u, 0u, 0u};
  for (int64_t it = 0; it < iters; ++it) {
    const int base = (int)((it * 1024) & 8191);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const u32x4 v = *(const u32x4*)(buf + ((lane_off + base + u * 1024 * 8) & 65535));
      x ^= v;
    }
  }
  sink[blockIdx.x * 512 + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

}  // namespace qg

using namespace qg;

extern "C" {

qg_status qg_ceiling_read(const void* buf, uint64_t bytes, int32_t loads_per_lane, uint32_t* sink, uint64_t sink_words,
                          void* stream) {
  if (!buf || !sink || bytes == 0 || bytes >= ((uint64_t)1 << 31) || (bytes & 15u) != 0 || ((uintptr_t)buf & 15u))
    return QG_ERR_INVALID_ARG;
  const int u = loads_per_lane;
  if (u != 1 && u != 2 && u != 4 && u != 8 && u != 16) return QG_ERR_INVALID_ARG;
  const uint64_t per_wg = 256ull * 16ull * (uint64_t)u;
  const uint64_t grid = (bytes + per_wg - 1) / per_wg;
  if (sink_words < grid * 4) return QG_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const uint8_t* p = (const uint8_t*)buf;
  switch (u) {
    case 1: hipLaunchKernelGGL(ceiling_read_kernel<1>, dim3((unsigned)grid), dim3(256), 0, st, p, (uint32_t)bytes, sink); break;
    case 2: hipLaunchKernelGGL(ceiling_read_kernel<2>, dim3((unsigned)grid), dim3(256), 0, st, p, (uint32_t)bytes, sink); break;
    case 4: hipLaunchKernelGGL(ceiling_read_kernel<4>, dim3((unsigned)grid), dim3(256), 0, st, p, (uint32_t)bytes, sink); break;
    case 8: hipLaunchKernelGGL(ceiling_read_kernel<8>, dim3((unsigned)grid), dim3(256), 0, st, p, (uint32_t)bytes, sink); break;
    default: hipLaunchKernelGGL(ceiling_read_kernel<16>, dim3((unsigned)grid), dim3(256), 0, st, p, (uint32_t)bytes, sink); break;
  }
  return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_HIP;
}

qg_status qg_ceiling_mfma(int32_t dtype, int64_t iters, int32_t workgroups, float* sink, uint64_t sink_floats,
                          void* stream) {
  if (dtype < 0 || dtype > 2 || iters <= 0 || workgroups <= 0 || !sink) return QG_ERR_INVALID_ARG;
  if (sink_floats < (uint64_t)workgroups * 256) return QG_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == 0) hipLaunchKernelGGL(ceiling_mfma_kernel<0>, dim3(workgroups), dim3(256), 0, st, iters, sink);
  else if (dtype == 1) hipLaunchKernelGGL(ceiling_mfma_kernel<1>, dim3(workgroups), dim3(256), 0, st, iters, sink);
  else hipLaunchKernelGGL(ceiling_mfma_kernel<2>, dim3(workgroups), dim3(256), 0, st, iters, sink);
  return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_HIP;
}

qg_status qg_ceiling_lds(int64_t iters, int32_t workgroups, uint32_t* sink, uint64_t sink_words, void* stream) {
  if (iters <= 0 || workgroups <= 0 || !sink) return QG_ERR_INVALID_ARG;
  if (sink_words < (uint64_t)workgroups * 512) return QG_ERR_WORKSPACE;
  hipLaunchKernelGGL(ceiling_lds_kernel, dim3(workgroups), dim3(512), 0, (hipStream_t)stream, iters, sink);
  return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_HIP;
}

}  // extern "C"
