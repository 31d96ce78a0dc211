// bench_util.hip -- measurement helpers for the benchmark, built as a library of their own
// (libmoe_bench_util.so), apart from the layer's library:
//   * a streaming device copy (the same-run achievable-bandwidth ceiling, and the plain copy of
//     known size that scales the HBM byte counters);
//   * a fill that writes a large scratch buffer between timed repetitions, so each repetition
//     starts with the 4 MB L2 of every XCD and the 256 MB Infinity Cache holding other data;
//   * a marker: a tiny kernel launched before every measured call with `phase` workgroups of 64
//     lanes, so a profiler's dispatch trace can be cut into the benchmark's phases and steps
//     (its grid size is 64 * phase).
// The copy and the fill move 16 bytes per lane, the copy with four loads in flight per lane;
// every access is guarded by the byte count, which must be a multiple of 16 (checked on the host).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // 16-byte pieces per lane per pass

__global__ __launch_bounds__(kThreads) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                               u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads * kUnroll;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kUnroll + threadIdx.x; base < n16;
       base += stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * kThreads;
      if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * kThreads;
      if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

__global__ __launch_bounds__(kThreads) void fill_kernel(u32x4* __restrict__ dst, int64_t n16, uint32_t value) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  const u32x4 v = {value, value, value, value};
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n16; i += stride) dst[i] = v;
}

__global__ __launch_bounds__(64) void bench_mark_kernel(uint32_t* __restrict__ buf, uint32_t step) {
  if (threadIdx.x == 0) buf[blockIdx.x] = step;
}

int grid_for(int64_t n16, int per_block) {
  int64_t g = (n16 + per_block - 1) / per_block;
  const int64_t cap = 256 * 64;  // 64 workgroups per CU of a 256-CU device: enough to fill it
  return static_cast<int>(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

extern "C" {

// dst[0, bytes) = src[0, bytes) on `stream`.  bytes % 16 == 0, both pointers 16-byte aligned,
// no overlap.  Returns 0 on success, 1 for a bad argument, 2 for a failed launch.
int moe_bench_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst || bytes < 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) ||
      (reinterpret_cast<uintptr_t>(dst) & 15u))
    return 1;
  if (bytes == 0) return 0;
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(stream_copy_kernel, dim3(grid_for(n16, kThreads * kUnroll)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), static_cast<u32x4*>(dst),
                     n16);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// dst[0, bytes) = the 32-bit pattern `value` repeated.  Same argument rules as moe_bench_copy.
int moe_bench_fill(void* dst, int64_t bytes, uint32_t value, void* stream) {
  if (!dst || bytes < 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(dst) & 15u)) return 1;
  if (bytes == 0) return 0;
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(fill_kernel, dim3(grid_for(n16, kThreads)), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<u32x4*>(dst), n16, value);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Marker for phase `phase` in [1, 64]: `phase` workgroups of 64 lanes each write `step` into
// buf[workgroup] (buf holds at least 64 uint32).  Same return codes.
int moe_bench_mark(void* buf, int32_t phase, uint32_t step, void* stream) {
  if (!buf || phase < 1 || phase > 64) return 1;
  hipLaunchKernelGGL(bench_mark_kernel, dim3(phase), dim3(64), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint32_t*>(buf), step);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
