// combine.hip -- Combine stage: gate-weighted un-permute and sum.
//
// y[t] = sum_j g[t, j] * y_perm[row_map[t, j]] (+ shared expert output, gate 1), the combine
// of "Scalable Training of Mixture-of-Experts Models with Megatron Core", summary page,
// "Method", first paragraph.  Without gates (the gate folded into the experts' SwiGLU epilogue,
// so y_perm rows arrive scaled) every weight is 1: fmaf(1, v, acc) is the plain sum.  One wavefront per token; each lane owns 8 consecutive
// columns (16-byte loads of bf16, two 16-byte loads of fp32), accumulates in fp32 over
// j = 0..k-1 in order, and rounds once to the output dtype.  No atomics: deterministic.
// The sum order is the same in every variant, so results do not depend on the unrolling.
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

// KT > 0: k known at compile time, so each lane issues all k gathers of a chunk (and of the
// next chunk) before the first FMA, keeping 2 k 16-byte loads in flight per lane.
template <int YDT, int ODT, int KT>
__global__ __launch_bounds__(kThreads) void combine_kernel(const void* __restrict__ y_perm,
                                                          const int32_t* __restrict__ row_map,
                                                          const float* __restrict__ gates,
                                                          const void* __restrict__ shared_out,
                                                          int64_t T, int H, int k_rt,
                                                          void* __restrict__ y) {
  const int k = KT > 0 ? KT : k_rt;
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  int row = 0;
  float g = 0.0f;
  if (lane < k) {
    row = row_map[t * k + lane];
    // a caller's row outside [0, T k) is read as row 0: every access stays inside y_perm
    row = static_cast<uint64_t>(row) < static_cast<uint64_t>(T * k) ? row : 0;
    g = gates ? gates[t * k + lane] : 1.0f;  // no gates: rows already scaled by them
  }
  const int n8 = H / 8;
  auto store = [&](int c, const float* acc) {
    if (ODT == 0) {
      float4* p = static_cast<float4*>(y) + (t * n8 + c) * 2;
      p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
      static_cast<uint4*>(y)[t * n8 + c] =
          make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    }
  };
  if constexpr (KT > 0) {
    int rows[KT];
    float gs[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      rows[j] = __shfl(row, j, kWave);
      gs[j] = __shfl(g, j, kWave);
    }
    for (int c0 = lane; c0 < n8; c0 += 2 * kWave) {
      const int c1 = c0 + kWave;
      const bool two = c1 < n8;
      // raw 16-byte pieces (bf16: one per chunk, fp32: two), widened only at the FMA
      constexpr int NV = YDT == 0 ? 2 : 1;
      uint4 raw[2][KT][NV];
      float sh[2][8];  // the shared expert's output, loaded with the gathers
#pragma unroll
      for (int j = 0; j < KT; ++j)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const uint4* src = static_cast<const uint4*>(y_perm) + (static_cast<int64_t>(rows[j]) * n8) * NV + v;
          const u32x4_t* s4 = reinterpret_cast<const u32x4_t*>(src);
          const u32x4_t a = __builtin_nontemporal_load(s4 + static_cast<int64_t>(c0) * NV);
          raw[0][j][v] = make_uint4(a[0], a[1], a[2], a[3]);
          if (two) {
            const u32x4_t b = __builtin_nontemporal_load(s4 + static_cast<int64_t>(c1) * NV);
            raw[1][j][v] = make_uint4(b[0], b[1], b[2], b[3]);
          }
        }
      if (shared_out) {
        load8(shared_out, YDT, t * n8 + c0, sh[0]);
        if (two) load8(shared_out, YDT, t * n8 + c1, sh[1]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (u == 1 && !two) break;
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int j = 0; j < KT; ++j) {
          float f[8];
          if (YDT == 0) {
            const uint4 a = raw[u][j][0], b = raw[u][j][NV - 1];
            f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y); f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
            f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y); f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
          } else {
            const uint4 a = raw[u][j][0];
            const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              f[2 * q] = __uint_as_float(w[q] << 16);
              f[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
            }
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(gs[j], f[i], acc[i]);
        }
        if (shared_out) {
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += sh[u][i];
        }
        store(u ? c1 : c0, acc);
      }
    }
  } else {
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
      store(c, acc);
    }
  }
}

template <int YDT, int ODT>
void launch_combine_k(dim3 grid, hipStream_t stream, const void* y_perm, const int32_t* row_map, const float* gates,
                      const void* shared_out, int64_t T, int H, int k, void* y) {
  switch (k) {
    case 1: hipLaunchKernelGGL((combine_kernel<YDT, ODT, 1>), grid, dim3(kThreads), 0, stream, y_perm, row_map, gates, shared_out, T, H, k, y); break;
    case 2: hipLaunchKernelGGL((combine_kernel<YDT, ODT, 2>), grid, dim3(kThreads), 0, stream, y_perm, row_map, gates, shared_out, T, H, k, y); break;
    case 4: hipLaunchKernelGGL((combine_kernel<YDT, ODT, 4>), grid, dim3(kThreads), 0, stream, y_perm, row_map, gates, shared_out, T, H, k, y); break;
    case 8: hipLaunchKernelGGL((combine_kernel<YDT, ODT, 8>), grid, dim3(kThreads), 0, stream, y_perm, row_map, gates, shared_out, T, H, k, y); break;
    default: hipLaunchKernelGGL((combine_kernel<YDT, ODT, 0>), grid, dim3(kThreads), 0, stream, y_perm, row_map, gates, shared_out, T, H, k, y); break;
  }
}

}  // namespace

hipError_t launch_combine(const void* y_perm, int y_dt, const int32_t* row_map, const float* gates,
                          const void* shared_out, int64_t T, int H, int k, void* y, int out_dt,
                          hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(ceil_div(T, kTokPerBlock)));
  if (y_dt == 0 && out_dt == 0)
    launch_combine_k<0, 0>(grid, stream, y_perm, row_map, gates, shared_out, T, H, k, y);
  else if (y_dt == 0 && out_dt == 1)
    launch_combine_k<0, 1>(grid, stream, y_perm, row_map, gates, shared_out, T, H, k, y);
  else if (y_dt == 1 && out_dt == 0)
    launch_combine_k<1, 0>(grid, stream, y_perm, row_map, gates, shared_out, T, H, k, y);
  else
    launch_combine_k<1, 1>(grid, stream, y_perm, row_map, gates, shared_out, T, H, k, y);
  return hipGetLastError();
}

}  // namespace moe
