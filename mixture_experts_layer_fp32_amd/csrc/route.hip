// route.hip -- Route stage: fp32 router projection, selection key, top-k and gates.
//
// The router is a learned linear projection optionally evaluated in FP32, followed by
// softmax or sigmoid scores and top-k selection ("Scalable Training of Mixture-of-Experts
// Models with Megatron Core", summary page, "Method", first paragraph; the router stays
// in higher precision per the same page's [§5] key claim).
//
// Two kernels:
//  1. route_logits: logits[T, E] = x[T, H] . W_r[H, E] in fp32 FMA (x widened exactly from
//     bf16).  A register-tiled skinny GEMM: a workgroup owns BT tokens x BE experts and
//     walks H in KC-wide chunks staged in LDS; each thread accumulates a TM x TN tile.
//  2. route_topk: one wavefront per token.  Lane l holds experts l, l+64, ...; k rounds of a
//     wave-wide arg-max (larger key wins, equal keys -> lower index) pick the slots in key
//     order; softmax statistics come from wave reductions over all E logits.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kKC = 32;  // H chunk staged per iteration

template <typename XT>
__device__ __forceinline__ float load_x(const XT* p);
template <>
__device__ __forceinline__ float load_x<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_x<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

// TN experts per thread along E (TX = BE / TN threads), TM tokens per thread (TY = 256 / TX).
template <typename XT, int BE, int TN, int TM>
__global__ __launch_bounds__(kRouteThreads) void route_logits_kernel(
    const XT* __restrict__ x, const float* __restrict__ w, float* __restrict__ logits, int64_t T,
    int H, int E) {
  constexpr int TX = BE / TN;
  constexpr int TY = kRouteThreads / TX;
  constexpr int BT = TY * TM;
  __shared__ float xs[kKC][BT + 1];
  __shared__ float ws[kKC][BE];

  const int tid = threadIdx.x;
  const int tx = tid % TX, ty = tid / TX;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * BT;
  const int e0 = blockIdx.y * BE;

  float acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;

  for (int h0 = 0; h0 < H; h0 += kKC) {
    // stage x[t0 .. t0+BT, h0 .. h0+KC) transposed (rows past T and columns past H read as 0)
    for (int i = tid; i < BT * kKC; i += kRouteThreads) {
      int tt = i / kKC, hh = i % kKC;
      int64_t t = t0 + tt;
      int h = h0 + hh;
      xs[hh][tt] = (t < T && h < H) ? load_x<XT>(x + t * H + h) : 0.0f;
    }
    for (int i = tid; i < kKC * BE; i += kRouteThreads) {
      int hh = i / BE, ee = i % BE;
      int h = h0 + hh, e = e0 + ee;
      ws[hh][ee] = (h < H && e < E) ? w[static_cast<int64_t>(h) * E + e] : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kKC; ++kk) {
      float a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = xs[kk][ty + i * TY];
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = ws[kk][tx + j * TX];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    int64_t t = t0 + ty + i * TY;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int e = e0 + tx + j * TX;
      if (e < E) logits[t * E + e] = acc[i][j];
    }
  }
}

constexpr int kMaxPerLane = 8;  // E <= 512 = 8 x 64 lanes

// larger key wins; equal keys -> lower index
__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int64_t T, int E, int k,
    int score, int norm, int32_t* __restrict__ ids, float* __restrict__ gates) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (kRouteThreads / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // whole wave exits together
  const float* lt = logits + t * E;

  float lg[kMaxPerLane], key[kMaxPerLane];
  float lmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    int e = lane + i * kWave;
    if (e < E) {
      lg[i] = lt[e];
      key[i] = bias ? lg[i] + bias[e] : lg[i];  // one fp32 add
      lmax = fmaxf(lmax, lg[i]);
    } else {
      lg[i] = 0.0f;
      key[i] = -INFINITY;
    }
  }
  float denom = 0.0f, m = 0.0f;
  if (score == 0) {
    m = wave_max(lmax);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
      if (lane + i * kWave < E) s += expf(lg[i] - m);
    denom = wave_sum(s);
  }

  uint32_t taken = 0;
  float my_gate = 0.0f;
  int my_id = 0;
  float gsum = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bk = -INFINITY, bl = 0.0f;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      int e = lane + i * kWave;
      if (e < E && !(taken & (1u << i)) && better(key[i], e, bk, bi)) {
        bk = key[i];
        bi = e;
        bl = lg[i];
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      float ok = __shfl_xor(bk, o, kWave);
      int oi = __shfl_xor(bi, o, kWave);
      float ol = __shfl_xor(bl, o, kWave);
      if (better(ok, oi, bk, bi)) {
        bk = ok;
        bi = oi;
        bl = ol;
      }
    }
    // every lane now holds the winner (bi, its logit bl)
    if ((bi % kWave) == lane) taken |= 1u << (bi / kWave);
    float g = (score == 0) ? expf(bl - m) / denom : 1.0f / (1.0f + expf(-bl));
    gsum += g;
    if (lane == j) {
      my_gate = g;
      my_id = bi;
    }
  }
  if (lane < k) {
    ids[t * k + lane] = my_id;
    gates[t * k + lane] = norm ? my_gate / gsum : my_gate;
  }
}

template <typename XT>
hipError_t launch_logits(const XT* x, const float* w, float* logits, int64_t T, int H, int E,
                         hipStream_t stream) {
  if (E >= 64) {
    constexpr int BE = 64, TN = 4, TM = 4;
    constexpr int BT = (kRouteThreads / (BE / TN)) * TM;
    dim3 grid(static_cast<unsigned>(ceil_div(T, BT)), static_cast<unsigned>(ceil_div(E, BE)));
    hipLaunchKernelGGL((route_logits_kernel<XT, BE, TN, TM>), grid, dim3(kRouteThreads), 0, stream,
                       x, w, logits, T, H, E);
  } else if (E > 16) {
    constexpr int BE = 32, TN = 2, TM = 2;
    constexpr int BT = (kRouteThreads / (BE / TN)) * TM;
    dim3 grid(static_cast<unsigned>(ceil_div(T, BT)), 1);
    hipLaunchKernelGGL((route_logits_kernel<XT, BE, TN, TM>), grid, dim3(kRouteThreads), 0, stream,
                       x, w, logits, T, H, E);
  } else {
    constexpr int BE = 16, TN = 2, TM = 1;
    constexpr int BT = (kRouteThreads / (BE / TN)) * TM;
    dim3 grid(static_cast<unsigned>(ceil_div(T, BT)), 1);
    hipLaunchKernelGGL((route_logits_kernel<XT, BE, TN, TM>), grid, dim3(kRouteThreads), 0, stream,
                       x, w, logits, T, H, E);
  }
  return hipGetLastError();
}

}  // namespace

size_t route_scratch_bytes(int64_t T, int E) { return static_cast<size_t>(T) * E * sizeof(float); }

hipError_t launch_route(const void* x, int x_dt, const float* w_router, const float* bias, int64_t T,
                        int H, int E, int k, int score, int norm, float* logits, int32_t* ids,
                        float* gates, float* logits_scratch, hipStream_t stream) {
  float* lg = logits ? logits : logits_scratch;
  hipError_t err = (x_dt == 0)
                       ? launch_logits(static_cast<const float*>(x), w_router, lg, T, H, E, stream)
                       : launch_logits(static_cast<const bf16_t*>(x), w_router, lg, T, H, E, stream);
  if (err != hipSuccess) return err;
  dim3 grid(static_cast<unsigned>(ceil_div(T, kRouteThreads / kWave)));
  hipLaunchKernelGGL(route_topk_kernel, grid, dim3(kRouteThreads), 0, stream, lg, bias, T, E, k, score,
                     norm, ids, gates);
  return hipGetLastError();
}

}  // namespace moe
