// combine.hip -- Combine stage: gate-weighted un-permute and sum.
//
// y[t] = sum_j g[t, j] * y_perm[row_map[t, j]] (+ shared expert output, gate 1), the combine
// of "Scalable Training of Mixture-of-Experts Models with Megatron Core", summary page,
// "Method", first paragraph.  One wavefront per token; each lane owns 8 consecutive
// columns (16-byte loads of bf16, two 16-byte loads of fp32), accumulates in fp32 over
// j = 0..k-1 in order, and rounds once to the output dtype.  No atomics: deterministic.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokPerBlock = kThreads / kWave;

__device__ __forceinline__ void load8(const void* base, int dt, int64_t idx8, float f[8]) {
  if (dt == 0) {
    const float4* p = static_cast<const float4*>(base) + idx8 * 2;
    float4 a = p[0], b = p[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  } else {
    uint4 v = static_cast<const uint4*>(base)[idx8];
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
}

template <int YDT, int ODT>
__global__ __launch_bounds__(kThreads) void combine_kernel(const void* __restrict__ y_perm,
                                                          const int32_t* __restrict__ row_map,
                                                          const float* __restrict__ gates,
                                                          const void* __restrict__ shared_out,
                                                          int64_t T, int H, int k,
                                                          void* __restrict__ y) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  int row = 0;
  float g = 0.0f;
  if (lane < k) {
    row = row_map[t * k + lane];
    g = gates[t * k + lane];
  }
  const int n8 = H / 8;
  for (int c = lane; c < n8; c += kWave) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int j = 0; j < k; ++j) {
      int r = __shfl(row, j, kWave);
      float gj = __shfl(g, j, kWave);
      float f[8];
      load8(y_perm, YDT, static_cast<int64_t>(r) * n8 + c, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(gj, f[i], acc[i]);
    }
    if (shared_out) {
      float f[8];
      load8(shared_out, YDT, t * n8 + c, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += f[i];
    }
    if (ODT == 0) {
      float4* p = static_cast<float4*>(y) + (t * n8 + c) * 2;
      p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
      static_cast<uint4*>(y)[t * n8 + c] =
          make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    }
  }
}

}  // namespace

hipError_t launch_combine(const void* y_perm, int y_dt, const int32_t* row_map, const float* gates,
                          const void* shared_out, int64_t T, int H, int k, void* y, int out_dt,
                          hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(ceil_div(T, kTokPerBlock)));
  if (y_dt == 0 && out_dt == 0)
    hipLaunchKernelGGL((combine_kernel<0, 0>), grid, dim3(kThreads), 0, stream, y_perm, row_map, gates,
                       shared_out, T, H, k, y);
  else if (y_dt == 0 && out_dt == 1)
    hipLaunchKernelGGL((combine_kernel<0, 1>), grid, dim3(kThreads), 0, stream, y_perm, row_map, gates,
                       shared_out, T, H, k, y);
  else if (y_dt == 1 && out_dt == 0)
    hipLaunchKernelGGL((combine_kernel<1, 0>), grid, dim3(kThreads), 0, stream, y_perm, row_map, gates,
                       shared_out, T, H, k, y);
  else
    hipLaunchKernelGGL((combine_kernel<1, 1>), grid, dim3(kThreads), 0, stream, y_perm, row_map, gates,
                       shared_out, T, H, k, y);
  return hipGetLastError();
}

}  // namespace moe
