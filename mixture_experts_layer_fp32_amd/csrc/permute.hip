// permute.hip -- Dispatch stage: expert histogram, prefix sum and stable scatter.
//
// The dispatcher permutes tokens so that rows routed to the same expert are contiguous,
// which the grouped GEMM needs ("Scalable Training of Mixture-of-Experts Models with
// Megatron Core", summary page, "Method", first paragraph).  Rows of one expert follow
// increasing token index, so the permutation is a pure function of the expert ids.
//
// Three kernels, no host round trip:
//  1. perm_count: per block of 256 tokens, an LDS bitmap per expert (one bit per token,
//     set with 64-bit LDS atomic OR, which is order-independent).  A (t, j) pair's rank
//     inside its expert and block is the popcount of the bits below t; the block's count
//     for expert e is the popcount of e's bitmap.
//  2. perm_scan: one workgroup scans the [E][B] count table in expert-major order (each thread a
//     run of it, the run totals by wave shuffles), giving each (expert, block) its first
//     permuted row, expert_offsets and expert_counts.
//  3. perm_scatter: one wavefront per token resolves its k rows, writes row_map/src_token,
//     reads the token's row once (16 B per lane) and writes it to its k permuted rows,
//     optionally quantising bf16 -> e4m3 in 1x128 blocks on the way.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kBT = 256;           // tokens per count block (= threads)
constexpr int kScanThreads = 1024;
constexpr int kMaxE = 512;

// An expert id from the caller outside [0, E) is taken as expert 0 (in every kernel alike, so
// counts, ranks and rows stay consistent and every access stays in bounds; the caller's results
// are then meaningless, which the interface states).
__device__ __forceinline__ int valid_id(int e, int E) { return static_cast<unsigned>(e) < static_cast<unsigned>(E) ? e : 0; }

__global__ __launch_bounds__(kBT) void perm_count_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                         int E, int k, int nblk,
                                                         int32_t* __restrict__ blk_counts,
                                                         int32_t* __restrict__ local_rank) {
  __shared__ unsigned long long bm[kMaxE][kBT / 64];
  const int tid = threadIdx.x;
  for (int i = tid; i < E * (kBT / 64); i += kBT) bm[i / (kBT / 64)][i % (kBT / 64)] = 0ull;
  __syncthreads();
  const int b = blockIdx.x;
  const int64_t t = static_cast<int64_t>(b) * kBT + tid;
  const int w = tid / 64;
  const unsigned long long bit = 1ull << (tid % 64);
  if (t < T) {
    for (int j = 0; j < k; ++j) atomicOr(&bm[valid_id(ids[t * k + j], E)][w], bit);
  }
  __syncthreads();
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      int e = valid_id(ids[t * k + j], E);
      int r = __popcll(bm[e][w] & (bit - 1ull));
      for (int ww = 0; ww < w; ++ww) r += __popcll(bm[e][ww]);
      local_rank[t * k + j] = r;
    }
  }
  for (int e = tid; e < E; e += kBT) {
    int c = 0;
#pragma unroll
    for (int ww = 0; ww < kBT / 64; ++ww) c += __popcll(bm[e][ww]);
    blk_counts[static_cast<int64_t>(e) * nblk + b] = c;
  }
}

// Exclusive scan of blk_counts (length E * nblk, expert-major) in place -> first row of
// each (expert, block); also expert_offsets [E+1] and (optionally) expert_counts [E].
__global__ __launch_bounds__(kScanThreads) void perm_scan_kernel(int32_t* __restrict__ base, int E,
                                                                 int nblk, int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ counts) {
  __shared__ int32_t part[kScanThreads / kWave];
  const int tid = threadIdx.x;
  const int64_t n = static_cast<int64_t>(E) * nblk;
  const int64_t per = ceil_div(n, kScanThreads);
  const int64_t lo = tid * per;
  const int64_t hi = lo + per < n ? lo + per : n;
  // runs of up to kRun entries (E ceil(T / 256) <= 16384: 256 experts and up to 16384 tokens) are
  // loaded once, all at the same time, and kept in registers; longer runs take two passes over memory
  constexpr int kRun = 16;
  const bool in_regs = per <= kRun;
  int32_t rv[kRun];
  int32_t s = 0;
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < kRun; ++i) rv[i] = lo + i < hi ? base[lo + i] : 0;
#pragma unroll
    for (int i = 0; i < kRun; ++i) s += rv[i];
  } else {
    for (int64_t i = lo; i < hi; ++i) s += base[i];
  }
  // inclusive scan of the 1024 partial sums: within each wave by shuffles, then across the 16 wave
  // totals by wave 0, then each thread adds the totals of the waves before it
  const int lane = tid % kWave, wave = tid / kWave;
  constexpr int NW = kScanThreads / kWave;
  int32_t v = s;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int32_t u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  if (lane == kWave - 1) part[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int32_t w = lane < NW ? part[lane] : 0;
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) {
      const int32_t u = __shfl_up(w, o, kWave);
      if (lane >= o) w += u;
    }
    if (lane < NW) part[lane] = w;
  }
  __syncthreads();
  int32_t run = v - s + (wave > 0 ? part[wave - 1] : 0);  // exclusive prefix of this thread's chunk
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      if (lo + i < hi) base[lo + i] = run;
      run += rv[i];
    }
  } else {
    for (int64_t i = lo; i < hi; ++i) {
      int32_t c = base[i];
      base[i] = run;
      run += c;
    }
  }
  __syncthreads();
  const int32_t total = part[NW - 1];
  for (int e = tid; e <= E; e += kScanThreads) {
    int32_t o = e < E ? base[static_cast<int64_t>(e) * nblk] : total;
    offsets[e] = o;
    if (counts && e < E) {
      int32_t o1 = e + 1 < E ? base[static_cast<int64_t>(e + 1) * nblk] : total;
      counts[e] = o1 - o;
    }
  }
}

constexpr int kScatterThreads = 256;
constexpr int kTokPerBlock = kScatterThreads / kWave;

// Resolve the k permuted rows of token t in lanes 0..k-1 (others: 0) and publish the maps; with
// gate_perm, also each row's gate (gate_perm[row_map[t, j]] = gates[t, j]).
__device__ __forceinline__ int resolve_row(const int32_t* ids, const int32_t* base,
                                           const int32_t* local_rank, int64_t t, int k, int E, int nblk,
                                           int lane, int32_t* row_map, int32_t* src_token, const float* gates,
                                           float* gate_perm) {
  int row = 0;
  if (lane < k) {
    int e = valid_id(ids[t * k + lane], E);
    row = base[static_cast<int64_t>(e) * nblk + t / kBT] + local_rank[t * k + lane];
    row_map[t * k + lane] = row;
    src_token[row] = static_cast<int32_t>(t);
    if (gate_perm) gate_perm[row] = gates[t * k + lane];
  }
  return row;
}

// Bit copy: VEC = 16 bytes per lane.
__global__ __launch_bounds__(kScatterThreads) void perm_scatter_copy_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ ids, const int32_t* __restrict__ base,
    const int32_t* __restrict__ local_rank, int64_t T, int row_vecs, int k, int E, int nblk,
    uint4* __restrict__ x_perm, int32_t* __restrict__ row_map, int32_t* __restrict__ src_token,
    const float* __restrict__ gates, float* __restrict__ gate_perm) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  int row = resolve_row(ids, base, local_rank, t, k, E, nblk, lane, row_map, src_token, gates, gate_perm);
  if (!x_perm) return;
  const uint4* src = x + t * row_vecs;
  // four 16-byte loads in flight per lane before their k stores each
  // (loads past the row end re-read its last piece; only in-row pieces are stored)
  constexpr int U = 4;
  for (int c0 = lane; c0 < row_vecs; c0 += U * kWave) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave;
      v[u] = src[c < row_vecs ? c : row_vecs - 1];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)  // keep the loaded values: no re-load inside the store loop
      asm volatile("" : "+v"(v[u].x), "+v"(v[u].y), "+v"(v[u].z), "+v"(v[u].w));
    // (non-temporal stores here measured slower: 247 -> 263 us for the DeepSeek-V3-shaped rows)
    for (int j = 0; j < k; ++j) {
      uint4* dst = x_perm + static_cast<int64_t>(__shfl(row, j, kWave)) * row_vecs;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (c0 + u * kWave < row_vecs) dst[c0 + u * kWave] = v[u];
    }
  }
}

// 8 bf16 values of a lane -> 8 e4m3 codes, with one power-of-two scale per 1x128 block shared by
// the 16 lanes that hold the block (lanes 16g .. 16g+15 of the wave).  Lanes with live == false
// contribute zeros to the block maximum.
__device__ __forceinline__ uint2 quant_e4m3_x8(uint4 v, float& scale) {
  uint32_t wv[4] = {v.x, v.y, v.z, v.w};
  float f[8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(wv[i] << 16);
    f[2 * i + 1] = __uint_as_float(wv[i] & 0xFFFF0000u);
    amax = fmaxf(amax, fmaxf(fabsf(f[2 * i]), fabsf(f[2 * i + 1])));
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
  const float s = e4m3_block_scale(amax);  // a power of two
  const float inv = pow2_inverse(s);        // x * inv is x / s rounded once
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = fminf(fmaxf(f[i] * inv, -448.0f), 448.0f);
  scale = s;
  return make_uint2(pack_e4m3x4(r[0], r[1], r[2], r[3]), pack_e4m3x4(r[4], r[5], r[6], r[7]));
}

// bf16 -> e4m3 with one fp32 scale per 1x128 block (16 lanes x 8 values).
__global__ __launch_bounds__(kScatterThreads) void perm_scatter_fp8_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ ids, const int32_t* __restrict__ base,
    const int32_t* __restrict__ local_rank, int64_t T, int H, int k, int E, int nblk,
    uint2* __restrict__ x_perm, float* __restrict__ scales, int32_t* __restrict__ row_map,
    int32_t* __restrict__ src_token, const float* __restrict__ gates, float* __restrict__ gate_perm) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  int row = resolve_row(ids, base, local_rank, t, k, E, nblk, lane, row_map, src_token, gates, gate_perm);
  if (!x_perm) return;
  const int row_vecs = H / 8;
  const int nsb = H / 128;
  const uint4* src = x + t * row_vecs;
  // two 16-byte loads in flight per lane; H % 128 == 0: whole 16-lane groups stay together
  for (int c0 = 0; c0 < row_vecs; c0 += 2 * kWave) {
    uint4 v[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = c0 + u * kWave + lane;
      v[u] = c < row_vecs ? src[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = c0 + u * kWave + lane;
      const bool live = c < row_vecs;
      float s;
      const uint2 packed = quant_e4m3_x8(v[u], s);
      for (int j = 0; j < k; ++j) {
        int r = __shfl(row, j, kWave);
        if (live) {
          x_perm[static_cast<int64_t>(r) * row_vecs + c] = packed;
          if ((lane & 15) == 0) scales[static_cast<int64_t>(r) * nsb + c / 16] = s;
        }
      }
    }
  }
}

// 8 bf16 values of a lane -> 8 E2M1 codes (4 bytes, value i in nibble i), with one E8M0 scale per
// 32 values shared by the 4 lanes that hold them (lanes 4g .. 4g+3; a group is wholly in or out).
__device__ __forceinline__ uint32_t quant_fp4_x8(uint4 v, int& e8) {
  const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
  float f[8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(wv[i] << 16);
    f[2 * i + 1] = __uint_as_float(wv[i] & 0xFFFF0000u);
    amax = fmaxf(amax, fmaxf(fabsf(f[2 * i]), fabsf(f[2 * i + 1])));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
  e8 = fp4_block_e8m0(amax);
  const float inv = e8m0_inverse(e8);  // f * inv is f / scale rounded once (exact: a power of two)
  return pack_fp4x8(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv, f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
}

// bf16 -> MXFP4 rows scattered to their permuted positions (codes [R, H / 2], scales [R, H / 32]).
__global__ __launch_bounds__(kScatterThreads) void perm_scatter_fp4_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ ids, const int32_t* __restrict__ base,
    const int32_t* __restrict__ local_rank, int64_t T, int H, int k, int E, int nblk,
    uint32_t* __restrict__ x_perm, uint8_t* __restrict__ scales, int32_t* __restrict__ row_map,
    int32_t* __restrict__ src_token, const float* __restrict__ gates, float* __restrict__ gate_perm) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  int row = resolve_row(ids, base, local_rank, t, k, E, nblk, lane, row_map, src_token, gates, gate_perm);
  if (!x_perm) return;
  const int row_vecs = H / 8;
  const int nsb = H / 32;
  const uint4* src = x + t * row_vecs;
  for (int c0 = 0; c0 < row_vecs; c0 += 2 * kWave) {
    uint4 v[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = c0 + u * kWave + lane;
      v[u] = c < row_vecs ? src[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = c0 + u * kWave + lane;
      int e8;
      const uint32_t packed = quant_fp4_x8(v[u], e8);
      for (int j = 0; j < k; ++j) {
        const int r = __shfl(row, j, kWave);
        if (c < row_vecs) {
          x_perm[static_cast<int64_t>(r) * row_vecs + c] = packed;
          if ((lane & 3) == 0) scales[static_cast<int64_t>(r) * nsb + c / 4] = static_cast<uint8_t>(e8);
        }
      }
    }
  }
}

// Dense per-row MXFP4 quantisation (each token once, for the fused forward and the shared expert).
__global__ __launch_bounds__(kScatterThreads) void quant_rows_fp4_kernel(const uint4* __restrict__ x, int64_t T,
                                                                          int H, uint32_t* __restrict__ codes,
                                                                          uint8_t* __restrict__ scales) {
  constexpr int U = 4;
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  const int row_vecs = H / 8;
  const int nsb = H / 32;
  const uint4* src = x + t * row_vecs;
  for (int c0 = 0; c0 < row_vecs; c0 += U * kWave) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave + lane;
      v[u] = c < row_vecs ? src[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave + lane;
      int e8;
      const uint32_t packed = quant_fp4_x8(v[u], e8);  // H % 32 == 0: a 4-lane group is wholly in or out
      if (c < row_vecs) {
        codes[t * row_vecs + c] = packed;
        if ((lane & 3) == 0) scales[t * nsb + c / 4] = static_cast<uint8_t>(e8);
      }
    }
  }
}

// Dense per-row quantisation (each token once, for the fused forward and the shared expert):
// one wavefront per row, four 16-byte loads per lane in flight before any is quantised.
__global__ __launch_bounds__(kScatterThreads) void quant_rows_fp8_kernel(const uint4* __restrict__ x, int64_t T,
                                                                          int H, uint2* __restrict__ codes,
                                                                          float* __restrict__ scales) {
  constexpr int U = 4;
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  const int row_vecs = H / 8;
  const int nsb = H / 128;
  const uint4* src = x + t * row_vecs;
  for (int c0 = 0; c0 < row_vecs; c0 += U * kWave) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave + lane;
      v[u] = c < row_vecs ? src[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave + lane;
      float s;
      const uint2 packed = quant_e4m3_x8(v[u], s);  // H % 128 == 0: a 16-lane group is wholly in or out
      if (c < row_vecs) {
        codes[t * row_vecs + c] = packed;
        if ((lane & 15) == 0) scales[t * nsb + c / 16] = s;
      }
    }
  }
}

}  // namespace

size_t permute_scratch_bytes(int64_t T, int E, int k) {
  const int64_t nblk = ceil_div(T, kBT);
  size_t a = static_cast<size_t>(E) * nblk * sizeof(int32_t);
  a = (a + 255) & ~static_cast<size_t>(255);
  return a + static_cast<size_t>(T) * k * sizeof(int32_t);
}

hipError_t launch_permute(const void* x, int x_dt, const int32_t* ids, int64_t T, int H, int E, int k,
                          void* x_perm, int perm_dt, void* x_perm_scales, int32_t* row_map,
                          int32_t* src_token, int32_t* counts, int32_t* offsets, void* scratch,
                          hipStream_t stream, const float* gates, float* gate_perm) {
  if ((gates == nullptr) != (gate_perm == nullptr)) return hipErrorInvalidValue;
  const int nblk = static_cast<int>(ceil_div(T, kBT));
  int32_t* blk = static_cast<int32_t*>(scratch);
  size_t a = static_cast<size_t>(E) * nblk * sizeof(int32_t);
  a = (a + 255) & ~static_cast<size_t>(255);
  int32_t* local_rank = reinterpret_cast<int32_t*>(static_cast<char*>(scratch) + a);

  hipLaunchKernelGGL(perm_count_kernel, dim3(nblk), dim3(kBT), 0, stream, ids, T, E, k, nblk, blk,
                     local_rank);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, blk, E, nblk, offsets,
                     counts);
  dim3 grid(static_cast<unsigned>(ceil_div(T, kTokPerBlock)));
  if (perm_dt == 2) {
    hipLaunchKernelGGL(perm_scatter_fp8_kernel, grid, dim3(kScatterThreads), 0, stream,
                       static_cast<const uint4*>(x), ids, blk, local_rank, T, H, k, E, nblk,
                       static_cast<uint2*>(x_perm), static_cast<float*>(x_perm_scales), row_map, src_token, gates,
                       gate_perm);
  } else if (perm_dt == 3) {
    hipLaunchKernelGGL(perm_scatter_fp4_kernel, grid, dim3(kScatterThreads), 0, stream,
                       static_cast<const uint4*>(x), ids, blk, local_rank, T, H, k, E, nblk,
                       static_cast<uint32_t*>(x_perm), static_cast<uint8_t*>(x_perm_scales), row_map, src_token,
                       gates, gate_perm);
  } else {
    const int elt = (x_dt == 0) ? 4 : 2;
    const int row_vecs = H * elt / 16;
    hipLaunchKernelGGL(perm_scatter_copy_kernel, grid, dim3(kScatterThreads), 0, stream,
                       static_cast<const uint4*>(x), ids, blk, local_rank, T, row_vecs, k, E, nblk,
                       static_cast<uint4*>(x_perm), row_map, src_token, gates, gate_perm);
  }
  return hipGetLastError();
}

hipError_t launch_quant_rows_fp8(const void* x, int x_dt, int64_t T, int H, uint8_t* codes, float* scales,
                                 hipStream_t stream) {
  if (x_dt != 1 || H % 128 != 0) return hipErrorInvalidValue;
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_fp8_kernel, dim3(static_cast<unsigned>(ceil_div(T, kTokPerBlock))),
                     dim3(kScatterThreads), 0, stream, static_cast<const uint4*>(x), T, H,
                     reinterpret_cast<uint2*>(codes), scales);
  return hipGetLastError();
}

hipError_t launch_quant_rows_fp4(const void* x, int64_t T, int H, uint8_t* codes, uint8_t* scales,
                                 hipStream_t stream) {
  if (H % 32 != 0) return hipErrorInvalidValue;
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_fp4_kernel, dim3(static_cast<unsigned>(ceil_div(T, kTokPerBlock))),
                     dim3(kScatterThreads), 0, stream, static_cast<const uint4*>(x), T, H,
                     reinterpret_cast<uint32_t*>(codes), scales);
  return hipGetLastError();
}

}  // namespace moe
