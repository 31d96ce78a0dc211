// route.hip -- Route stage: fp32 router projection, selection key, top-k and gates.
//
// The router is a learned linear projection optionally evaluated in FP32, followed by
// softmax or sigmoid scores and top-k selection ("Scalable Training of Mixture-of-Experts
// Models with Megatron Core", summary page, "Method", first paragraph; the router stays
// in higher precision per the same page's [§5] key claim).
//
// Kernels:
//  1. logits, bf16 x (the usual case): W_r is split once per call into three bf16 matrices
//     W_r = W_hi + W_mid + W_lo (each the bf16 rounding of what the previous ones leave; the
//     remainder is below 2^-24 |w|), stored K-contiguous per expert.  x is exactly bf16, so
//     three bf16 MFMAs (v_mfma_f32_16x16x32_bf16, fp32 accumulate, exact products) give the
//     fp32 projection at MFMA speed: the stage is then bound by streaming x from HBM.
//     Fragments come straight from global memory in MFMA layout (16 B per lane); the small
//     split weight stays in L2.
//  1'. logits, fp32 x: a register-tiled fp32 FMA skinny GEMM (a workgroup owns BT tokens x
//     BE experts and walks H in KC-wide chunks staged in LDS).
//  2. route_topk: one wavefront per token.  Lane l holds experts l, l+64, ...; k rounds, each a
//     wave-wide maximum of the free keys and ballots for its lowest expert index (larger key
//     wins, equal keys -> lower index), pick the slots in key order; softmax statistics come
//     from wave reductions over all E logits.
//  3. For <= 16 experts and long batches, 1 and 2 in one kernel (route_fused_few_kernel): the
//     three weight parts packed as MFMA columns, the logits and the top k of 16 tokens per
//     workgroup.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;

struct RouterGemmPlan {
  int bm;      // tile rows of the router GEMM (128 or 256)
  int ksplit;  // K slices
};
constexpr int kKC = 32;  // H chunk staged per iteration

template <typename XT>
__device__ __forceinline__ float load_x(const XT* p);
template <>
__device__ __forceinline__ float load_x<float>(const float* p) { return *p; }

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

// W_r [H, E] fp32 -> ws [3][Ep][H] bf16 (Ep = E rounded up to 16, padded experts are 0).
__global__ __launch_bounds__(kRouteThreads) void route_split_kernel(const float* __restrict__ w, int H,
                                                                   int E, int Ep,
                                                                   bf16_t* __restrict__ ws) {
  const int64_t n = static_cast<int64_t>(Ep) * H;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kRouteThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kRouteThreads) {
    const int e = static_cast<int>(i / H), h = static_cast<int>(i % H);
    float v = e < E ? w[static_cast<int64_t>(h) * E + e] : 0.0f;
    bf16_t p0 = f32_to_bf16(v);
    float r1 = v - bf16_to_f32(p0);  // exact: v and its bf16 rounding share the leading bits
    bf16_t p1 = f32_to_bf16(r1);
    float r2 = r1 - bf16_to_f32(p1);
    bf16_t p2 = f32_to_bf16(r2);
    ws[i] = p0;
    ws[n + i] = p1;
    ws[2 * n + i] = p2;
  }
}

// The same split, stored [H][3 Ep] (N-contiguous, plane-major columns) for the grouped-GEMM
// kernel used when there are many experts: column p * Ep + e holds part p of W_r[:, e].
__global__ __launch_bounds__(kRouteThreads) void route_split_kn_kernel(const float* __restrict__ w, int H, int E,
                                                                      int Ep, bf16_t* __restrict__ wkn) {
  const int64_t n = static_cast<int64_t>(Ep) * H;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kRouteThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kRouteThreads) {
    const int h = static_cast<int>(i / Ep), e = static_cast<int>(i % Ep);
    float v = e < E ? w[static_cast<int64_t>(h) * E + e] : 0.0f;
    bf16_t p0 = f32_to_bf16(v);
    float r1 = v - bf16_to_f32(p0);
    bf16_t p1 = f32_to_bf16(r1);
    float r2 = r1 - bf16_to_f32(p1);
    bf16_t p2 = f32_to_bf16(r2);
    bf16_t* row = wkn + static_cast<int64_t>(h) * 3 * Ep;
    row[e] = p0;
    row[Ep + e] = p1;
    row[2 * Ep + e] = p2;
  }
}

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4v;

// A workgroup computes 16*TM tokens x 16*TN experts with v_mfma_f32_16x16x32_bf16 over the
// blockIdx.z-th of gridDim.z slices of H; its NW waves split the slice NW ways (each keeping U
// k-steps of loads in flight) and their partial sums are added in LDS.  With one slice the
// workgroup writes the logits; with several, `logits` is a [slices][T][E] scratch array and the
// workgroup writes its slice's partial logits there (summed by the top-k kernel in slice order).  Operand layout: lane l holds row (l % 16), k = 8*(l/16) .. +8 of a 32-wide
// k-step (A: token rows of x; B: expert rows of the split weight); accumulator slot r of lane l
// is token 4*(l/16) + r, expert l % 16.
template <int TM, int TN, int U, int NW = 4>
__global__ __launch_bounds__(NW * 64) void route_logits_mfma_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ ws, float* __restrict__ logits, int64_t T,
    int H, int E, int Ep) {
  __shared__ float part[NW][TM][TN][4][kWave];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * (16 * TM);
  const int e0 = blockIdx.y * (16 * TN);
  const int64_t plane = static_cast<int64_t>(Ep) * H;
  const int kq = 8 * (lane / 16);
  const bf16_t* xa[TM];
  bool live[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    int64_t t = t0 + i * 16 + lane % 16;
    live[i] = t < T;
    xa[i] = x + (live[i] ? t : 0) * H + kq;
  }
  const bf16_t* wb[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) wb[j] = ws + static_cast<int64_t>(e0 + j * 16 + lane % 16) * H + kq;
  f32x4v acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};
  // this wave's share of this slice's 32-wide k-steps
  const int steps = (H + 31) / 32, nz = static_cast<int>(gridDim.z), z = static_cast<int>(blockIdx.z);
  const int z0 = z * steps / nz, z1 = (z + 1) * steps / nz;
  const int s0 = z0 + wave * (z1 - z0) / NW, s1 = z0 + (wave + 1) * (z1 - z0) / NW;
  logits += static_cast<int64_t>(z) * T * E;
  for (int sb = s0; sb < s1; sb += U) {
    bf16x8_t a[U][TM], b[U][TN][3];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = (sb + u) * 32;
      const bool kin = (sb + u) < s1 && k0 + kq < H;  // H % 8 == 0: an 8-wide chunk is wholly in or out
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        uint4 v = (live[i] && kin) ? *reinterpret_cast<const uint4*>(xa[i] + k0) : make_uint4(0, 0, 0, 0);
        a[u][i] = *reinterpret_cast<bf16x8_t*>(&v);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int sp = 0; sp < 3; ++sp) {
          uint4 v = kin ? *reinterpret_cast<const uint4*>(wb[j] + sp * plane + k0) : make_uint4(0, 0, 0, 0);
          b[u][j][sp] = *reinterpret_cast<bf16x8_t*>(&v);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          // smallest parts first
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][i], b[u][j][2], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][i], b[u][j][1], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][i], b[u][j][0], acc[i][j], 0, 0, 0);
        }
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[wave][i][j][r][lane] = acc[i][j][r];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int e = e0 + j * 16 + lane % 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = part[0][i][j][r][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += part[w][i][j][r][lane];
        const int64_t t = t0 + i * 16 + 4 * (lane / 16) + r;
        if (t < T && e < E) logits[t * E + e] = v;
      }
    }
}

constexpr int kMaxPerLane = 8;  // E <= 512 = 8 x 64 lanes

// larger key wins; equal keys -> lower index
__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Where the logits come from: with slices > 1, `parts` holds the few-expert kernel's partial
// logits of `slices` H slices ([slices][T][E]), added in slice order; with slices == 1 and
// `parts`, it holds the router GEMM's [ksplit][T][3 Ep] products of x with the three weight
// parts, each part summed over the K slices in order and the logit taken as (lo + mid) + hi;
// either way the logit is also written to `logits`.  Without `parts` the logits are read from
// `logits`.
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(
    float* __restrict__ logits, const float* __restrict__ parts, int Ep, int ksplit, int slices,
    const float* __restrict__ bias, int64_t T, int E, int k, int score, int norm, int32_t* __restrict__ ids,
    float* __restrict__ gates) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (kRouteThreads / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // whole wave exits together
  float* lt = logits + t * E;
  const float* pt = parts && slices == 1 ? parts + t * 3 * Ep : nullptr;

  float lg[kMaxPerLane], key[kMaxPerLane];
  float lmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    int e = lane + i * kWave;
    if (e < E) {
      if (slices > 1) {
        // partial logits of the H slices ([slices][T][E] in `parts`), added in slice order
        const float* ps = parts + t * E + e;
        float v = ps[0];
        for (int s = 1; s < slices; ++s) v += ps[s * T * E];
        lg[i] = v;
        lt[e] = v;
      } else if (pt) {
        // each part summed over the K slices in order, then smallest part first
        const int64_t slice = T * 3 * Ep;
        float p0 = pt[e], p1 = pt[Ep + e], p2 = pt[2 * Ep + e];
        for (int s = 1; s < ksplit; ++s) {
          p0 += pt[s * slice + e];
          p1 += pt[s * slice + Ep + e];
          p2 += pt[s * slice + 2 * Ep + e];
        }
        lg[i] = (p2 + p1) + p0;
        lt[e] = lg[i];
      } else {
        lg[i] = lt[e];
      }
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
    // the largest key still free, then its lowest expert index: expert e = lane + 64 i, so the
    // first slot i whose ballot of "free and equal to the maximum" is non-empty, and in it the
    // lowest lane (larger key wins, equal keys -> lower index; +0 and -0 compare equal)
    float lk = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
      if (lane + i * kWave < E && !(taken & (1u << i))) lk = fmaxf(lk, key[i]);
    const float mk = wave_max(lk);
    int bi = -1;
    float bl = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      if (bi < 0) {  // wave-uniform
        const uint64_t b = __ballot(lane + i * kWave < E && !(taken & (1u << i)) && key[i] == mk);
        if (b) {
          const int ln = __builtin_ctzll(b);
          bi = i * kWave + ln;
          bl = __shfl(lg[i], ln, kWave);
        }
      }
    }
    if (bi < 0) {  // only NaN keys left: the lowest free expert
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) {
        if (bi < 0) {
          const uint64_t b = __ballot(lane + i * kWave < E && !(taken & (1u << i)));
          if (b) {
            const int ln = __builtin_ctzll(b);
            bi = i * kWave + ln;
            bl = __shfl(lg[i], ln, kWave);
          }
        }
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

// Few experts and enough tokens: the whole route stage in one kernel.  A workgroup owns 16 TM
// tokens and all of H, which its NW waves split.  The B operand packs the three bf16 parts side
// by side: column c = p E + e holds part p of expert e (the split weight stored [3E][H], row c
// K-contiguous), columns from 3E on are zero, so 16 TN >= 3E columns take one MFMA per token
// block and k-step instead of one per part.  Lane layout as in route_logits_mfma_kernel.  The
// waves' partial sums are added in LDS in wave order, then one lane per token forms the logit
// (hi + mid + lo summed smallest part first, as the router GEMM does), writes it, and takes the
// top k with the same key, tie and gate rules as route_topk_kernel.
template <int TM, int TN, int NW, int U>
__global__ __launch_bounds__(NW * 64) void route_fused_few_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ ws, const float* __restrict__ bias, int64_t T,
    int H, int E, int k, int score, int norm, float* __restrict__ logits, int32_t* __restrict__ ids,
    float* __restrict__ gates) {
  extern __shared__ float fsm[];
  float* part = fsm;                              // [NW][TM][TN][4][64]
  float* S = fsm + NW * TM * TN * 4 * kWave;      // [16 TM][16 TN] summed products
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * (16 * TM);
  const int kq = 8 * (lane / 16);
  const bf16_t* xa[TM];
  bool live[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t t = t0 + i * 16 + lane % 16;
    live[i] = t < T;
    xa[i] = x + (live[i] ? t : 0) * H + kq;
  }
  const bf16_t* wb[TN];
  bool col[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int c = j * 16 + lane % 16;
    col[j] = c < 3 * E;
    wb[j] = ws + static_cast<int64_t>(col[j] ? c : 0) * H + kq;
  }
  f32x4v acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};
  const int steps = (H + 31) / 32;
  const int s0 = wave * steps / NW, s1 = (wave + 1) * steps / NW;
  for (int sb = s0; sb < s1; sb += U) {
    bf16x8_t a[U][TM], b[U][TN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = (sb + u) * 32;
      const bool kin = (sb + u) < s1 && k0 + kq < H;  // H % 8 == 0: an 8-wide chunk is wholly in or out
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        uint4 v = (live[i] && kin) ? *reinterpret_cast<const uint4*>(xa[i] + k0) : make_uint4(0, 0, 0, 0);
        a[u][i] = *reinterpret_cast<bf16x8_t*>(&v);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        uint4 v = (col[j] && kin) ? *reinterpret_cast<const uint4*>(wb[j] + k0) : make_uint4(0, 0, 0, 0);
        b[u][j] = *reinterpret_cast<bf16x8_t*>(&v);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][i], b[u][j], acc[i][j], 0, 0, 0);
  }
  // accumulator slot r of lane l: token 4 (l / 16) + r of its 16-token block, column l % 16
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[(((wave * TM + i) * TN + j) * 4 + r) * kWave + lane] = acc[i][j][r];
  __syncthreads();
  constexpr int NTOK = 16 * TM, NCOL = 16 * TN;
  for (int idx = threadIdx.x; idx < NTOK * NCOL; idx += NW * kWave) {
    const int tok = idx / NCOL, c = idx % NCOL;
    const int i = tok / 16, rr = tok % 16, j = c / 16;
    const int l = 16 * (rr / 4) + c % 16, r = rr % 4;
    float v = part[((i * TN + j) * 4 + r) * kWave + l];
    for (int w = 1; w < NW; ++w) v += part[(((w * TM + i) * TN + j) * 4 + r) * kWave + l];
    S[tok * NCOL + c] = v;
  }
  __syncthreads();
  if (threadIdx.x >= NTOK) return;
  const int64_t t = t0 + threadIdx.x;
  if (t >= T) return;
  float* st = S + threadIdx.x * NCOL;  // this token's row; its first k entries later hold the gates
  float lg[16], key[16];
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    if (e < E) {
      lg[e] = (st[2 * E + e] + st[E + e]) + st[e];
      key[e] = bias ? lg[e] + bias[e] : lg[e];  // one fp32 add
      m = fmaxf(m, lg[e]);
      logits[t * E + e] = lg[e];
    } else {
      lg[e] = 0.0f;
      key[e] = -INFINITY;
    }
  }
  float denom = 0.0f;
  if (score == 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (e < E) denom += expf(lg[e] - m);
  }
  uint32_t taken = 0;
  float gsum = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bk = -INFINITY, bl = 0.0f;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (e < E && !(taken & (1u << e)) && better(key[e], e, bk, bi)) {
        bk = key[e];
        bi = e;
        bl = lg[e];
      }
    }
    taken |= 1u << bi;
    const float gj = (score == 0) ? expf(bl - m) / denom : 1.0f / (1.0f + expf(-bl));
    gsum += gj;
    ids[t * k + j] = bi;
    st[j] = gj;  // k <= E <= 16 <= NCOL
  }
  for (int j = 0; j < k; ++j) gates[t * k + j] = norm ? st[j] / gsum : st[j];
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

int padded_experts(int E) { return (E + 15) / 16 * 16; }

size_t split_bytes(int H, int E) { return static_cast<size_t>(3) * padded_experts(E) * H * sizeof(bf16_t); }

// Many experts (>= 64): the projection is a dense GEMM x [T, H] . W_split [H, 3 Ep] on the
// grouped-GEMM kernel (fp32 output, one row band per 128 tokens), summed per expert by top-k.
bool logits_by_gemm(int H, int E) { return padded_experts(E) >= 64 && H % 64 == 0; }

// Tile height and K slices of the router GEMM.  With few output tiles (T/bm x 3Ep/256 of them)
// the projection leaves CUs idle, but every slice writes a [T][3Ep] fp32 partial product that the
// top-k kernel reads back.  Estimated cost, in 64-deep K steps of a 128-row tile: rounds of 256
// single-workgroup CUs x K steps per slice x the tile's step cost (a 256-row step costs 1.3
// 128-row steps: its weight loads and fragment reads serve twice the rows), plus the partial
// products at about 8 MB of HBM traffic per K step.  Measured GEMM times of the candidates
// (DeepSeek-V3-shaped router, T=8192 H=7168 3Ep=768: 128-row tiles 1 slice 132 us, 2 slices
// 131, 4 slices 130; 256-row tiles 1 slice 169, 2 slices 114, 4 slices 119.  Qwen3-235B-shaped,
// T=8192 H=4096 3Ep=384: 128-row 1/2/4 slices 74/52/55 us, 256-row 2/4 slices 63/46 us).  Powers
// of two up to 8 that keep >= 8 K steps per slice; ties go to 128-row tiles, then fewer slices.
// A pure function of (T, H, E): the workspace size and the launch must agree.
RouterGemmPlan router_gemm_plan(int64_t T, int H, int E) {
  const int64_t ntiles = ceil_div(3 * padded_experts(E), 256);
  const int nk = H / 64;
  const double slice_steps = static_cast<double>(T) * 3 * padded_experts(E) * 8 / 8.0e6;
  RouterGemmPlan best{128, 1};
  double best_cost = -1.0;
  for (int bm : {128, 256}) {
    const int64_t tiles = ceil_div(T, bm) * ntiles;
    const double step = bm == 256 ? 1.3 : 1.0;
    for (int ks = 1; ks <= 8; ks *= 2) {
      if (nk % ks != 0 || (ks > 1 && nk / ks < 8)) break;
      const double cost =
          static_cast<double>(ceil_div(tiles * ks, 256)) * (nk / ks) * step + ks * slice_steps;
      if (best_cost < 0.0 || cost < best_cost) {
        best = RouterGemmPlan{bm, ks};
        best_cost = cost;
      }
    }
  }
  return best;
}

// H slices of the few-expert (Ep <= 16) router kernel: 64 tokens per workgroup would leave CUs
// idle for short batches and, with one slice, every workgroup streams the whole split weight
// for only 64 tokens; H is cut until there are >= 256 workgroups, each wave keeping >= 1 k-step.
int router_hslices(int64_t T, int H, int E) {
  if (padded_experts(E) > 16) return 1;
  const int64_t chunks = ceil_div(T, 64);
  const int steps = (H + 31) / 32;
  int hs = 1;
  while (hs < 8 && chunks * hs < 256 && steps / (2 * hs) >= 16) hs *= 2;
  return hs;
}

// The fused few-expert kernel (16 tokens per workgroup, four k-steps of loads in flight per
// wave) when it gives at least 192 workgroups; shorter batches take the H-sliced logits kernel
// and the separate top-k.  Measured on the Mixtral-shaped route (split + fused kernel): 25 us
// against 30 us for the sliced path; 32-token workgroups (half the CUs busy) 32 us.
bool route_fused(int64_t T, int E) { return padded_experts(E) <= 16 && ceil_div(T, 16) >= 192; }

template <int TN>
hipError_t launch_fused_few(const bf16_t* x, const bf16_t* ws, const float* bias, int64_t T, int H, int E, int k,
                            int score, int norm, float* logits, int32_t* ids, float* gates, hipStream_t stream) {
  constexpr int TM = 1, NW = 16, U = 4;
  constexpr size_t smem = (static_cast<size_t>(NW) * TM * TN * 4 * kWave + 16 * TM * 16 * TN) * sizeof(float);
  auto kern = route_fused_few_kernel<TM, TN, NW, U>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(ceil_div(T, 16 * TM))), dim3(NW * kWave), smem, stream, x, ws,
                     bias, T, H, E, k, score, norm, logits, ids, gates);
  return hipGetLastError();
}

size_t hslice_bytes(int64_t T, int H, int E) {
  const int hs = router_hslices(T, H, E);
  return hs > 1 ? ((static_cast<size_t>(hs) * T * E * sizeof(float) + 255) & ~static_cast<size_t>(255)) : 0;
}

size_t parts_bytes(int64_t T, int H, int E) {
  return (static_cast<size_t>(router_gemm_plan(T, H, E).ksplit) * T * 3 * padded_experts(E) * sizeof(float) + 255) &
         ~static_cast<size_t>(255);
}

hipError_t launch_logits_bf16(const bf16_t* x, const float* w, float* logits, float* parts, float* hparts,
                              int64_t T, int H, int E, bf16_t* wsplit, hipStream_t stream) {
  const int Ep = padded_experts(E);
  const int64_t n = static_cast<int64_t>(Ep) * H;
  const unsigned gs = static_cast<unsigned>(ceil_div(n, kRouteThreads) < 2048 ? ceil_div(n, kRouteThreads) : 2048);
  if (parts) {
    hipLaunchKernelGGL(route_split_kn_kernel, dim3(gs), dim3(kRouteThreads), 0, stream, w, H, E, Ep, wsplit);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const RouterGemmPlan plan = router_gemm_plan(T, H, E);
    return launch_dense_gemm_f32out(x, wsplit, T, H, 3 * Ep, parts, stream, plan.ksplit, plan.bm);
  }
  hipLaunchKernelGGL(route_split_kernel, dim3(gs), dim3(kRouteThreads), 0, stream, w, H, E, Ep, wsplit);
  if (Ep <= 16) {
    // few experts: 64 tokens per workgroup, 16 waves split the workgroup's slice of H so that each
    // CU keeps many x loads in flight; with several slices the partial logits go to hparts
    const int hs = router_hslices(T, H, E);
    dim3 grid(static_cast<unsigned>(ceil_div(T, 64)), 1, static_cast<unsigned>(hs));
    hipLaunchKernelGGL((route_logits_mfma_kernel<4, 1, 2, 16>), grid, dim3(16 * kWave), 0, stream, x, wsplit,
                       hs > 1 ? hparts : logits, T, H, E, Ep);
  } else if (Ep % 64 == 0) {
    dim3 grid(static_cast<unsigned>(ceil_div(T, 32)), static_cast<unsigned>(Ep / 64));
    hipLaunchKernelGGL((route_logits_mfma_kernel<2, 4, 2>), grid, dim3(kRouteThreads), 0, stream, x, wsplit,
                       logits, T, H, E, Ep);
  } else {
    dim3 grid(static_cast<unsigned>(ceil_div(T, 32)), static_cast<unsigned>(Ep / 16));
    hipLaunchKernelGGL((route_logits_mfma_kernel<2, 1, 4>), grid, dim3(kRouteThreads), 0, stream, x, wsplit,
                       logits, T, H, E, Ep);
  }
  return hipGetLastError();
}

}  // namespace

size_t route_scratch_bytes(int64_t T, int H, int E, bool logits_given) {
  size_t a = logits_given ? 0 : (static_cast<size_t>(T) * E * sizeof(float) + 255) & ~static_cast<size_t>(255);
  a += (split_bytes(H, E) + 255) & ~static_cast<size_t>(255);
  if (logits_by_gemm(H, E)) a += parts_bytes(T, H, E);
  a += hslice_bytes(T, H, E);
  return a;
}

hipError_t launch_route(const void* x, int x_dt, const float* w_router, const float* bias, int64_t T,
                        int H, int E, int k, int score, int norm, float* logits, int32_t* ids,
                        float* gates, void* scratch, hipStream_t stream) {
  float* lg = logits;
  char* sp = static_cast<char*>(scratch);
  if (!lg) {
    lg = reinterpret_cast<float*>(sp);
    sp += (static_cast<size_t>(T) * E * sizeof(float) + 255) & ~static_cast<size_t>(255);
  }
  bf16_t* wsplit = reinterpret_cast<bf16_t*>(sp);
  sp += (split_bytes(H, E) + 255) & ~static_cast<size_t>(255);
  if (x_dt != 0 && route_fused(T, E)) {
    // the split weight as [3E][H]: row p E + e is part p of expert e
    const int64_t n = static_cast<int64_t>(E) * H;
    const unsigned gs = static_cast<unsigned>(ceil_div(n, kRouteThreads) < 2048 ? ceil_div(n, kRouteThreads) : 2048);
    hipLaunchKernelGGL(route_split_kernel, dim3(gs), dim3(kRouteThreads), 0, stream, w_router, H, E, E, wsplit);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const int tn = (3 * E + 15) / 16;
    if (tn == 1) return launch_fused_few<1>(xb, wsplit, bias, T, H, E, k, score, norm, lg, ids, gates, stream);
    if (tn == 2) return launch_fused_few<2>(xb, wsplit, bias, T, H, E, k, score, norm, lg, ids, gates, stream);
    return launch_fused_few<3>(xb, wsplit, bias, T, H, E, k, score, norm, lg, ids, gates, stream);
  }
  float* parts = (x_dt != 0 && logits_by_gemm(H, E)) ? reinterpret_cast<float*>(sp) : nullptr;
  if (logits_by_gemm(H, E)) sp += parts_bytes(T, H, E);
  const int hs = x_dt != 0 ? router_hslices(T, H, E) : 1;
  float* hparts = hs > 1 ? reinterpret_cast<float*>(sp) : nullptr;
  hipError_t err = (x_dt == 0)
                       ? launch_logits(static_cast<const float*>(x), w_router, lg, T, H, E, stream)
                       : launch_logits_bf16(static_cast<const bf16_t*>(x), w_router, lg, parts, hparts, T, H, E,
                                            wsplit, stream);
  if (err != hipSuccess) return err;
  dim3 grid(static_cast<unsigned>(ceil_div(T, kRouteThreads / kWave)));
  hipLaunchKernelGGL(route_topk_kernel, grid, dim3(kRouteThreads), 0, stream, lg, hs > 1 ? hparts : parts,
                     padded_experts(E), parts ? router_gemm_plan(T, H, E).ksplit : 1, hs, bias, T, E, k, score, norm, ids,
                     gates);
  return hipGetLastError();
}

}  // namespace moe
