// backward.hip -- gradients of the MoE layer: the forward's stages differentiated in reverse.
//
// The pages measure this layer in training ("Scalable Training of Mixture-of-Experts Models
// with Megatron Core": abstract; summary page, "Method", second paragraph, which counts
// fine-grained activation recomputation among the memory recipes).  Given dy = dL/dy:
//   combine:  dyp[p] = g_p dy[t_p],  dg_p = <dy[t_p], yp[p]>        (p = row_map(t, j), t_p = t)
//   experts:  u = xp W1 (recomputed here, not kept from the forward), a | b = u, h = SiLU(a) b,
//             dh = dyp W2^T, dW2 = h^T dyp, du = [dh b SiLU'(a) | dh SiLU(a)],
//             dxp = du W1^T, dW1 = xp^T du
//   dispatch: dx[t] = sum_j dxp[row_map(t, j)]
//   route:    dlogits from dg through the gate function; dx += dlogits W_r^T, dW_r = x^T dlogits
// Two rewrites keep y_perm and the gate-weighted rows g_p dy[t_p] out of memory: dh' = dy[t_p] W2^T
// is formed once without the gate, so dg_p = <dh'_p, h_p> (= <dy[t_p], h_p W2>) and dh = g_p dh'_p;
// and dW2 = (g h)^T dy[t_p] takes the gate on the h side.  Every GEMM reads the token rows of x and
// dy through src_token (the dispatch permutation fused into the loads), so neither x_perm nor a
// permuted dy is materialised.
//
// Kernels:
//  * bwd_gemm_kernel<layout, TA, TB>: one grouped GEMM for the three operand layouts the chain
//    needs, 128 x 128 output tiles, 4 waves of 64 x 64, v_mfma_f32_32x32x16_bf16 (both operands
//    bf16) or v_mfma_f32_32x32x2f32 (an fp32 operand), fp32 accumulate and output.  Operands are
//    staged through registers into k-contiguous LDS tiles, two buffers, one barrier per K step:
//      NN  C[p, n]   = sum_k A[g(p), k] B_e[k, n]      p over expert e's rows   (u)
//      NT  C[p, n]   = sum_k A[g(p), k] B_e[n, k]      p over expert e's rows   (dh', dxp)
//      TN  C_e[m, n] = sum_p A[g(p), m] B[g'(p), n]    contraction over e's rows (dW1, dW2)
//    An expert without rows gets a zero weight gradient (its TN tiles have no K steps).
//  * bwd_swiglu_kernel: per permuted row, the SwiGLU backward and the gate gradient dg_p.
//  * bwd_gate_kernel: per token, the softmax / sigmoid (+ renormalisation) Jacobian.
//  * bwd_dx_kernel: per token, dx = sum_j dxp[row_map(t, j)] + shared expert + router terms.
// With bf16 operands the expert GEMMs run on the forward's grouped-GEMM kernel instead (gemm.hip):
// u as there, dh' and dxp with the weight read as stored ([N, K]), and dW1, dW2 as independent
// per-expert products over the expert's rows padded to a multiple of 64: dW1_e = (x[src]^T)_e du_e
// and dW2_e = ((g h)^T)_e dy[src]_e, the transposed operands written by bwd_transpose_pad_kernel
// (zeros in the padding columns) and dy gathered into row order by bwd_gather_rows_kernel.
#include "gemm_common.hpp"

namespace moe {
namespace {

using namespace gemm;

enum Layout { kNN = 0, kNT = 1, kTN = 2 };

constexpr int kTile = 128;  // output tile columns (rows: 256 or 128)

template <typename T>
struct Elt;
template <>
struct Elt<float> {
  static constexpr int kVec = 4;  // elements per 16-byte chunk
};
template <>
struct Elt<bf16_t> {
  static constexpr int kVec = 8;
};

template <typename TA, typename TB>
struct BwdCfg {
  static constexpr bool kBf16 = std::is_same<TA, bf16_t>::value && std::is_same<TB, bf16_t>::value;
  using CT = typename std::conditional<kBf16, bf16_t, float>::type;  // LDS / MFMA operand type
  static constexpr int BK = kBf16 ? 32 : 16;                         // K per LDS tile
  static constexpr int LD = BK + (kBf16 ? 8 : 4);                    // LDS row pitch: 80 bytes
};

template <typename TA, typename TB>
struct GemmArgs {
  const TA* A;
  int64_t lda;
  const int32_t* gA;  // row gather of A (NN / NT: output rows; TN: contraction rows) or null
  int64_t gA_rows;    // rows of A a gathered index may name (indices are clamped into it)
  const TB* B;
  int64_t ldb;
  int64_t sB;         // NN / NT: element stride between experts' B matrices
  const int32_t* gB;  // TN: row gather of B or null
  int64_t gB_rows;
  const int32_t* offsets;  // [G + 1] in device memory, or null: one group of `rows` rows
  int64_t rows;            // host bound of the grouped rows (T * k, or T)
  int G;
  int M, N, K;             // TN: M x N per group; NN / NT: N output columns, K contraction
  float* C;
  int64_t ldc;
  int64_t sC;              // TN: element stride between groups' outputs
  int vecA, vecB;          // 16-byte loads allowed: base 16-byte aligned, strides multiples of a chunk
};

// bf16 LDS tiles: the four 16-byte k-chunks of row r sit at chunk ^ ((r >> 4) & 3), so the
// transposing stores (a wave's lanes write rows 4 apart) spread over the banks; every read and
// write of a bf16 tile goes through it.
__device__ __forceinline__ int swz(int row, int k) { return (((k >> 3) ^ ((row >> 4) & 3)) << 3) | (k & 7); }

__device__ __forceinline__ int64_t clamp_row(int64_t r, int64_t n) { return r < 0 ? 0 : (r >= n ? n - 1 : r); }

// One 16-byte chunk (4 fp32 or 8 bf16) starting at p, of which the first n_ok elements exist;
// the rest read as zero.  p is dereferenced only for existing elements.
template <typename T>
__device__ __forceinline__ u32x4_t load_chunk(const T* p, int n_ok, int vec) {
  constexpr int V = Elt<T>::kVec;
  if (vec && n_ok == V) return *reinterpret_cast<const u32x4_t*>(p);
  u32x4_t r = {0u, 0u, 0u, 0u};
  if constexpr (V == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < n_ok) r[i] = __float_as_uint(p[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < n_ok) r[i / 2] |= static_cast<uint32_t>(p[i]) << (16 * (i % 2));
  }
  return r;
}

template <typename T>
__device__ __forceinline__ float chunk_f32(const u32x4_t& c, int i) {
  if constexpr (Elt<T>::kVec == 4) return __uint_as_float(c[i]);
  else return bf16_to_f32(static_cast<bf16_t>((c[i / 2] >> (16 * (i % 2))) & 0xFFFFu));
}

// Chunk of source type TS to LDS row `row`, columns kc.. (k-contiguous in both).
template <typename TS, typename CT, int LD>
__device__ __forceinline__ void store_k(CT* s, const u32x4_t& c, int row, int kc) {
  if constexpr (std::is_same<TS, CT>::value) {
    *reinterpret_cast<u32x4_t*>(s + row * LD + (std::is_same<CT, bf16_t>::value ? swz(row, kc) : kc)) = c;
  } else {  // bf16 source, fp32 tile: 8 floats
    u32x4_t lo, hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = __float_as_uint(chunk_f32<TS>(c, i));
      hi[i] = __float_as_uint(chunk_f32<TS>(c, 4 + i));
    }
    *reinterpret_cast<u32x4_t*>(s + row * LD + kc) = lo;
    *reinterpret_cast<u32x4_t*>(s + row * LD + kc + 4) = hi;
  }
}

// Chunk of source type TS holding consecutive rows mc.. of LDS column k (a transposed store).
template <typename TS, typename CT, int LD>
__device__ __forceinline__ void store_t(CT* s, const u32x4_t& c, int mc, int k) {
  constexpr int V = Elt<TS>::kVec;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    if constexpr (std::is_same<CT, bf16_t>::value)
      s[(mc + i) * LD + swz(mc + i, k)] = static_cast<bf16_t>((c[i / 2] >> (16 * (i % 2))) & 0xFFFFu);
    else
      s[(mc + i) * LD + k] = chunk_f32<TS>(c, i);
  }
}

// Four bf16 at p (8 bytes), of which the first n_ok exist; the rest read as zero.
__device__ __forceinline__ uint2 load8(const bf16_t* p, int n_ok, int vec) {
  if (vec && n_ok == 4) return *reinterpret_cast<const uint2*>(p);
  uint2 r = make_uint2(0u, 0u);
  if (n_ok > 0) r.x = p[0];
  if (n_ok > 1) r.x |= static_cast<uint32_t>(p[1]) << 16;
  if (n_ok > 2) r.y = p[2];
  if (n_ok > 3) r.y |= static_cast<uint32_t>(p[3]) << 16;
  return r;
}

__device__ __forceinline__ uint32_t half_of(const uint2& q, int j) {
  return ((j < 2 ? q.x : q.y) >> (16 * (j % 2))) & 0xFFFFu;
}

template <int LAY, typename TA, typename TB, int BM, int BN>
__global__ __launch_bounds__(BM * BN / 64, BM * BN == 32768 ? 4 : 1) void bwd_gemm_kernel(const GemmArgs<TA, TB> g) {
  using Cfg = BwdCfg<TA, TB>;
  using CT = typename Cfg::CT;
  constexpr int NTH = BM * BN / 64;  // (BM / 64) x (BN / 64) waves, each 64 x 64
  constexpr int WN = BN / 64;
  constexpr int BK = Cfg::BK, LD = Cfg::LD;
  constexpr int VA = Elt<TA>::kVec, VB = Elt<TB>::kVec;
  constexpr int RA = BM * BK / VA / NTH, RB = BN * BK / VB / NTH;  // chunks per thread
  static_assert(RA >= 1 && RB >= 1 && RA * VA * NTH == BM * BK && RB * VB * NTH == BN * BK, "tile split");
  __shared__ __align__(16) CT sA[2][BM * LD];
  __shared__ __align__(16) CT sB[2][BN * LD];
  __shared__ int s_pref[kMaxExpertsLds];

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;
  int e = 0, m0 = 0, n0 = 0;
  int64_t row0 = 0, row_end = 0, kbeg = 0, kend = 0;
  if constexpr (LAY == kTN) {
    // Workgroups go round-robin to the 8 XCDs; tile L = (w % 8) per + w / 8 gives each XCD a
    // contiguous range of tiles, m-major, so the tiles sharing an A block run on one XCD's L2.
    const int tiles_n = static_cast<int>(ceil_div(g.N, BN));
    const int tiles = static_cast<int>(ceil_div(g.M, BM)) * tiles_n;
    const int per = (tiles + 7) / 8;
    const int w = static_cast<int>(blockIdx.x);
    const int L = (w % 8) * per + w / 8;
    if (L >= tiles) return;  // whole workgroup, before any barrier
    // inside that range, groups of 8 m-tiles walked n-major: the tiles running together form
    // ~8 x 8 blocks that share their A and B blocks in L2
    const int tiles_m = tiles / tiles_n;
    const int grp = L / (8 * tiles_n), idx = L % (8 * tiles_n);
    const int gm = tiles_m - grp * 8 < 8 ? tiles_m - grp * 8 : 8;
    e = static_cast<int>(blockIdx.y);
    m0 = (grp * 8 + idx % gm) * BM;
    n0 = idx / gm * BN;
    if (g.offsets != nullptr) {
      int64_t base, cnt;
      expert_rows(g.offsets, e, g.rows, base, cnt);
      kbeg = base;
      kend = base + cnt;
    } else {  // one dense group: blockIdx.y cuts its rows into gridDim.y slices (C + y sC each)
      const int64_t S = gridDim.y;
      kbeg = g.rows * e / S;
      kend = g.rows * (e + 1) / S;
    }
  } else {
    TileMap tm;
    if (!map_tile<BM>(g.offsets, g.rows, g.G, static_cast<int>(ceil_div(g.N, BN)), s_pref, tm)) return;
    e = tm.expert;
    row0 = tm.row0;
    row_end = tm.row_end;
    n0 = tm.nt * BN;
    kend = g.K;
  }
  const TB* Bg = g.B + (LAY == kTN ? 0 : static_cast<int64_t>(e) * g.sB);

  // bf16 operands laid out n- (or m-) contiguous in memory (TN: A and B; NN: B): a thread takes
  // a 4 (k) x 4 (n) block as four 8-byte loads, transposes it in registers and writes four
  // 8-byte k-contiguous LDS rows, instead of eight 2-byte LDS stores per 16-byte chunk.
  constexpr bool kTrA = Cfg::kBf16 && LAY == kTN;
  constexpr bool kTrB = Cfg::kBf16 && LAY != kNT;
  // The source rows (gathered or not) of the tile fetched next are read one K step ahead of its
  // data, so a data load never waits on the index load issued just before it (ix = -1: no row).
  // An operand tile of COLS columns: COLS / 4 column groups of 4; each thread takes TR k rows of
  // its group (TR = BK COLS / 4 / NTH: 4 for A, 4 or 2 for B).
  using CGA = std::integral_constant<int, BM / 4>;
  using CGB = std::integral_constant<int, BN / 4>;
  constexpr int TRA = BK * CGA::value / NTH, TRB = BK * CGB::value / NTH;
  static_assert(TRA % 2 == 0 && TRB % 2 == 0 && TRA <= 4 && TRB <= 4, "transpose blocks");
  uint2 qa[TRA], qb[TRB];
  int64_t ia[TRA], ib[TRB];
  auto load_idx = [&](auto cg, const int32_t* gat, int64_t glim, int64_t kb, auto& ix) {
    constexpr int CG = decltype(cg)::value;
    constexpr int TR = std::extent<std::remove_reference_t<decltype(ix)>>::value;
#pragma unroll
    for (int r = 0; r < TR; ++r) {
      const int64_t row = kb + (tid / CG) * TR + r;
      ix[r] = row < kend ? (gat ? clamp_row(gat[row], glim) : row) : -1;
    }
  };
  auto load_tr = [&](auto cg, const bf16_t* base, int64_t ld, const auto& ix, int col0, int ncols, int vec,
                     auto& q) {
    constexpr int CG = decltype(cg)::value;
    constexpr int TR = std::extent<std::remove_reference_t<decltype(q)>>::value;
    const int c = col0 + (tid % CG) * 4;
#pragma unroll
    for (int r = 0; r < TR; ++r) {
      q[r] = make_uint2(0u, 0u);
      if (ix[r] >= 0 && c < ncols) q[r] = load8(base + ix[r] * ld + c, ncols - c < 4 ? ncols - c : 4, vec);
    }
  };
  auto store_tr = [&](auto cg, bf16_t* sm, const auto& q) {
    constexpr int CG = decltype(cg)::value;
    constexpr int TR = std::extent<std::remove_reference_t<decltype(q)>>::value;
    const int nb = (tid % CG) * 4, kq = (tid / CG) * TR;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w0 = half_of(q[0], j) | (half_of(q[1], j) << 16);
      if constexpr (TR == 4) {
        uint2 v;
        v.x = w0;
        v.y = half_of(q[2], j) | (half_of(q[3], j) << 16);
        *reinterpret_cast<uint2*>(sm + (nb + j) * LD + swz(nb + j, kq)) = v;
      } else {
        *reinterpret_cast<uint32_t*>(sm + (nb + j) * LD + swz(nb + j, kq)) = w0;
      }
    }
  };

  u32x4_t ra[RA], rb[RB];
  auto load_a = [&](int64_t kb) {
    if constexpr (kTrA) {
      load_tr(CGA{}, g.A, g.lda, ia, m0, g.M, g.vecA, qa);
      load_idx(CGA{}, g.gA, g.gA_rows, kb + BK, ia);
      return;
    }
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      const int c = tid + i * NTH;
      const TA* p = g.A;
      int n_ok = 0;
      if constexpr (LAY == kTN) {  // A [rows, M]: m contiguous, the contraction runs over rows
        const int kr = c / (BM / VA), m = m0 + c % (BM / VA) * VA;
        const int64_t r = kb + kr;
        if (r < kend && m < g.M) {
          const int64_t src = g.gA ? clamp_row(g.gA[r], g.gA_rows) : r;
          p = g.A + src * g.lda + m;
          n_ok = g.M - m < VA ? g.M - m : VA;
        }
      } else {  // A [rows, K]: k contiguous
        const int r = c / (BK / VA);
        const int64_t grow = row0 + r, kk = kb + c % (BK / VA) * VA;
        if (grow < row_end && kk < kend) {
          const int64_t src = g.gA ? clamp_row(g.gA[grow], g.gA_rows) : grow;
          p = g.A + src * g.lda + kk;
          n_ok = kend - kk < VA ? static_cast<int>(kend - kk) : VA;
        }
      }
      ra[i] = load_chunk(p, n_ok, g.vecA);
    }
  };
  auto load_b = [&](int64_t kb) {
    if constexpr (kTrB) {
      load_tr(CGB{}, LAY == kTN ? g.B : Bg, g.ldb, ib, n0, g.N, g.vecB, qb);
      load_idx(CGB{}, LAY == kTN ? g.gB : nullptr, g.gB_rows, kb + BK, ib);
      return;
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int c = tid + i * NTH;
      const TB* p = g.B;
      int n_ok = 0;
      if constexpr (LAY == kNT) {  // B_e [N, K]: k contiguous
        const int n = n0 + c / (BK / VB);
        const int64_t kk = kb + c % (BK / VB) * VB;
        if (n < g.N && kk < kend) {
          p = Bg + static_cast<int64_t>(n) * g.ldb + kk;
          n_ok = kend - kk < VB ? static_cast<int>(kend - kk) : VB;
        }
      } else {  // NN: B_e [K, N]; TN: B [rows, N] (gathered rows): n contiguous
        const int64_t r = kb + c / (BN / VB);
        const int n = n0 + c % (BN / VB) * VB;
        if (r < kend && n < g.N) {
          const int64_t src = (LAY == kTN && g.gB) ? clamp_row(g.gB[r], g.gB_rows) : r;
          p = Bg + src * g.ldb + n;
          n_ok = g.N - n < VB ? g.N - n : VB;
        }
      }
      rb[i] = load_chunk(p, n_ok, g.vecB);
    }
  };
  auto store_a = [&](int buf) {
    if constexpr (kTrA) {
      store_tr(CGA{}, sA[buf], qa);
      return;
    }
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      const int c = tid + i * NTH;
      if constexpr (LAY == kTN)
        store_t<TA, CT, LD>(sA[buf], ra[i], c % (BM / VA) * VA, c / (BM / VA));
      else
        store_k<TA, CT, LD>(sA[buf], ra[i], c / (BK / VA), c % (BK / VA) * VA);
    }
  };
  auto store_b = [&](int buf) {
    if constexpr (kTrB) {
      store_tr(CGB{}, sB[buf], qb);
      return;
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int c = tid + i * NTH;
      if constexpr (LAY == kNT)
        store_k<TB, CT, LD>(sB[buf], rb[i], c / (BK / VB), c % (BK / VB) * VB);
      else
        store_t<TB, CT, LD>(sB[buf], rb[i], c % (BN / VB) * VB, c / (BN / VB));
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto compute = [&](int buf) {
    const CT* as = sA[buf] + (wm * 64 + lane % 32) * LD;
    const CT* bs = sB[buf] + (wn * 64 + lane % 32) * LD;
    if constexpr (Cfg::kBf16) {
#pragma unroll
      for (int ks = 0; ks < BK; ks += 16) {
        bf16x8_t af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int k = ks + (lane / 32) * 8;
          af[i] = *reinterpret_cast<const bf16x8_t*>(as + i * 32 * LD + swz(wm * 64 + i * 32 + lane % 32, k));
          bfr[i] = *reinterpret_cast<const bf16x8_t*>(bs + i * 32 * LD + swz(wn * 64 + i * 32 + lane % 32, k));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < BK; ks += 2) {
        float af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          af[i] = as[i * 32 * LD + ks + lane / 32];
          bfr[i] = bs[i * 32 * LD + ks + lane / 32];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  if (kbeg < kend) {
    if constexpr (kTrA) load_idx(CGA{}, g.gA, g.gA_rows, kbeg, ia);
    if constexpr (kTrB) load_idx(CGB{}, LAY == kTN ? g.gB : nullptr, g.gB_rows, kbeg, ib);
    load_a(kbeg);
    load_b(kbeg);
    store_a(0);
    store_b(0);
    __syncthreads();
    int buf = 0;
    for (int64_t kb = kbeg; kb < kend; kb += BK) {
      const bool more = kb + BK < kend;
      if (more) {  // next tile's global loads overlap this tile's MFMAs
        load_a(kb + BK);
        load_b(kb + BK);
      }
      compute(buf);
      if (more) {  // the other buffer was last read before the previous barrier
        store_a(buf ^ 1);
        store_b(buf ^ 1);
      }
      __syncthreads();
      buf ^= 1;
    }
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + i * 32 + (r / 4) * 8 + (lane / 32) * 4 + r % 4;
        const int col = wn * 64 + j * 32 + lane % 32;
        if constexpr (LAY == kTN) {
          const int m = m0 + row, n = n0 + col;
          if (m < g.M && n < g.N) g.C[e * g.sC + static_cast<int64_t>(m) * g.ldc + n] = acc[i][j][r];
        } else {
          const int64_t grow = row0 + row;
          const int n = n0 + col;
          if (grow < row_end && n < g.N) g.C[grow * g.ldc + n] = acc[i][j][r];
        }
      }
}

// bf16 operands: 8 waves, 128 x 256 tiles for NT (the activation rows, re-read once per column
// tile, are the larger stream) and 256 x 128 otherwise; an fp32 operand: 128 x 128 (4 waves).
template <int LAY, typename TA, typename TB>
hipError_t launch_bwd_gemm(const GemmArgs<TA, TB>& g, hipStream_t stream) {
  constexpr bool bf = BwdCfg<TA, TB>::kBf16;
  constexpr int BM = bf ? (LAY == kNT ? 128 : 256) : 128;
  constexpr int BN = bf ? (LAY == kNT ? 256 : 128) : 128;
  const int64_t tiles_n = ceil_div(g.N, BN);
  dim3 grid;
  if (LAY == kTN)
    grid = dim3(static_cast<unsigned>(8 * ceil_div(ceil_div(g.M, BM) * tiles_n, 8)), static_cast<unsigned>(g.G));
  else
    grid = dim3(grid_for(max_tiles<BM>(g.rows, g.G, g.offsets == nullptr), static_cast<int>(tiles_n)));
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_gemm_kernel<LAY, TA, TB, BM, BN>), grid, dim3(BM * BN / 64), 0, stream, g);
  return hipGetLastError();
}

template <typename T>
bool vec_ok(const T* p, int64_t ld, int64_t stride) {
  constexpr int V = Elt<T>::kVec;
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0 && ld % V == 0 && stride % V == 0;
}

template <typename TA, typename TB>
GemmArgs<TA, TB> args(const TA* A, int64_t lda, const int32_t* gA, int64_t gA_rows, const TB* B, int64_t ldb,
                      int64_t sB, const int32_t* gB, int64_t gB_rows, const int32_t* offsets, int64_t rows, int G,
                      int M, int N, int K, float* C, int64_t ldc, int64_t sC) {
  GemmArgs<TA, TB> g{A, lda, gA, gA_rows, B, ldb, sB, gB, gB_rows, offsets, rows, G, M, N, K, C, ldc, sC, 0, 0};
  g.vecA = vec_ok(A, lda, 0);
  g.vecB = vec_ok(B, ldb, sB);
  return g;
}

// ------------------------------------------------------------------- elementwise backward
template <typename CT>
__device__ __forceinline__ void store4(CT* p, float a, float b, float c, float d) {
  if constexpr (std::is_same<CT, float>::value) {
    f32x4_t v = {a, b, c, d};
    *reinterpret_cast<f32x4_t*>(p) = v;
  } else {
    uint2 v;
    v.x = pack_bf16x2(a, b);
    v.y = pack_bf16x2(c, d);
    *reinterpret_cast<uint2*>(p) = v;
  }
}

// One workgroup per row p of u [rows, 2F] (fp32) and dh' [rows, F] (fp32, no gate).  The gate of
// row p is that of the (t, j) pair with row_map(t, j) = p, t = src[p]; without src (the shared
// expert) it is 1 and dg is not written.  SiLU'(a) = s (1 + a (1 - s)), s = 1 / (1 + e^-a).
template <typename CT>
__global__ __launch_bounds__(256) void bwd_swiglu_kernel(const float* __restrict__ u, const float* __restrict__ dhp,
                                                         const float* __restrict__ gates,
                                                         const int32_t* __restrict__ row_map,
                                                         const int32_t* __restrict__ src, int64_t T, int k, int F,
                                                         CT* __restrict__ du, CT* __restrict__ gh,
                                                         float* __restrict__ dg) {
  __shared__ float s_gate;
  __shared__ float s_part[256 / kWave];
  const int64_t p = blockIdx.x;
  const int tid = threadIdx.x;
  float gate = 1.0f;
  if (src != nullptr) {
    if (tid == 0) {
      const int64_t t = clamp_row(src[p], T);
      float gg = 0.0f;
      for (int j = 0; j < k; ++j)
        if (row_map[t * k + j] == p) gg = gates[t * k + j];
      s_gate = gg;
    }
    __syncthreads();
    gate = s_gate;
  }
  const float* up = u + p * 2 * F;
  const float* dp = dhp + p * F;
  CT* dup = du + p * 2 * F;
  CT* ghp = gh + p * F;
  float part = 0.0f;
  for (int f = tid * 4; f < F; f += 256 * 4) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(up + f);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(up + F + f);
    const f32x4_t d = *reinterpret_cast<const f32x4_t*>(dp + f);
    float da[4], db[4], hg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s = 1.0f / (1.0f + expf(-a[i]));
      const float sl = a[i] * s;
      const float h = sl * b[i];
      part += d[i] * h;
      const float dh = gate * d[i];
      da[i] = dh * b[i] * (s * (1.0f + a[i] * (1.0f - s)));
      db[i] = dh * sl;
      hg[i] = gate * h;
    }
    store4(dup + f, da[0], da[1], da[2], da[3]);
    store4(dup + F + f, db[0], db[1], db[2], db[3]);
    store4(ghp + f, hg[0], hg[1], hg[2], hg[3]);
  }
  if (dg != nullptr) {
    part = wave_sum(part);
    if (tid % kWave == 0) s_part[tid / kWave] = part;
    __syncthreads();
    if (tid == 0) dg[p] = ((s_part[0] + s_part[1]) + s_part[2]) + s_part[3];
  }
}

// One wave per token: dlogits [T, E] from dg_perm (the gate gradients in permuted-row order).
// Scores s_j: softmax over all E at the selected experts, or the logistic function of the
// selected logit; with `norm` the gates are s_j / S.  Unselected experts get p_e (0 - B) under
// softmax and 0 under sigmoid.
__global__ __launch_bounds__(256) void bwd_gate_kernel(const float* __restrict__ logits,
                                                       const int32_t* __restrict__ ids,
                                                       const float* __restrict__ dg_perm,
                                                       const int32_t* __restrict__ row_map, int64_t T, int E, int k,
                                                       int score, int norm, int64_t R, float* __restrict__ dl) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (256 / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // whole waves; no barriers below
  const float* lt = logits + t * E;
  int id = 0;
  float dgj = 0.0f;
  if (lane < k) {
    const int v = ids[t * k + lane];
    id = v < 0 ? 0 : (v >= E ? E - 1 : v);
    dgj = dg_perm[clamp_row(row_map[t * k + lane], R)];
  }
  float m = -INFINITY, z = 0.0f, sj = 0.0f;
  if (score == 0) {
    for (int e = lane; e < E; e += kWave) m = fmaxf(m, lt[e]);
    m = wave_max(m);
    for (int e = lane; e < E; e += kWave) z += expf(lt[e] - m);
    z = wave_sum(z);
    if (lane < k) sj = expf(lt[id] - m) / z;
  } else if (lane < k) {
    sj = 1.0f / (1.0f + expf(-lt[id]));
  }
  float dsj = dgj;
  if (norm) {
    const float S = wave_sum(sj);
    const float A = wave_sum(dgj * (sj / S));
    dsj = lane < k ? (dgj - A) / S : 0.0f;
  }
  const float B = score == 0 ? wave_sum(dsj * sj) : 0.0f;
  int idj[kMaxTopk];
  float dsk[kMaxTopk];
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) {
    idj[j] = __shfl(id, j, kWave);
    dsk[j] = __shfl(dsj, j, kWave);
  }
  for (int e = lane; e < E; e += kWave) {
    float d = 0.0f;
    bool sel = false;
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j)
      if (j < k && idj[j] == e) {
        d = dsk[j];
        sel = true;
      }
    float v;
    if (score == 0) {
      v = expf(lt[e] - m) / z * (d - B);
    } else {
      const float s = 1.0f / (1.0f + expf(-lt[e]));
      v = sel ? d * (s * (1.0f - s)) : 0.0f;
    }
    dl[t * E + e] = v;
  }
}

// out[i] = sum_s part[s n + i], slices in order.
__global__ __launch_bounds__(256) void bwd_sum_slices_kernel(const float* __restrict__ part, int S, int64_t n,
                                                             float* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float acc = part[i];
  for (int s = 1; s < S; ++s) acc += part[s * n + i];
  out[i] = acc;
}

// 4 consecutive values as fp32 (fp32 or bf16 storage, 16- or 8-byte aligned).
template <typename T>
__device__ __forceinline__ f32x4_t load4(const T* p) {
  if constexpr (std::is_same<T, float>::value) {
    return *reinterpret_cast<const f32x4_t*>(p);
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return f32x4_t{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                   __uint_as_float(v.y & 0xffff0000u)};
  }
}

// One workgroup per token: dx[t] = sum_j dxp[row_map(t, j)] (j ascending) + extra0[t] + extra1[t], in
// fp32; dxp and extra0 (the shared expert's term) are stored in the layer's dtype, as the forward
// keeps y_perm and sums it in fp32 in combine.
template <typename XT>
__global__ __launch_bounds__(256) void bwd_dx_kernel(const XT* __restrict__ dxp, const int32_t* __restrict__ row_map,
                                                     int64_t R, int k, const XT* __restrict__ extra0,
                                                     const float* __restrict__ extra1, int H, XT* __restrict__ dx) {
  __shared__ int64_t s_rows[kMaxTopk];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < k) s_rows[threadIdx.x] = clamp_row(row_map[t * k + threadIdx.x], R);
  __syncthreads();
  for (int h = threadIdx.x * 4; h < H; h += 256 * 4) {
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < k; ++j) acc += load4(dxp + s_rows[j] * H + h);
    if (extra0) acc += load4(extra0 + t * H + h);
    if (extra1) acc += *reinterpret_cast<const f32x4_t*>(extra1 + t * H + h);
    store4(dx + t * H + h, acc[0], acc[1], acc[2], acc[3]);
  }
}

// The padded contraction table of the per-expert weight-gradient products: kinfo[0 .. E] the
// exclusive prefix of the experts' row counts rounded up to 64, kinfo[E + 1 .. 2E + 1] the
// experts' row offsets (clamped like the forward's tile map; offsets null: one group of `rows`).
// One workgroup of 256 threads, E <= 512.
__global__ __launch_bounds__(256) void bwd_kinfo_kernel(const int32_t* __restrict__ offsets, int64_t rows, int E,
                                                        int32_t* __restrict__ kinfo) {
  __shared__ int s[kMaxExpertsLds];
  for (int e = static_cast<int>(threadIdx.x); e < E; e += static_cast<int>(blockDim.x)) {
    int64_t base = 0, M = rows;
    if (offsets) expert_rows(offsets, e, rows, base, M);
    s[e + 1] = static_cast<int>((M + 63) / 64 * 64);
    kinfo[E + 1 + e] = static_cast<int32_t>(base);
    if (e == E - 1) kinfo[2 * E + 1] = static_cast<int32_t>(base + M);
  }
  scan_prefix(s, E);
  for (int e = static_cast<int>(threadIdx.x); e <= E; e += static_cast<int>(blockDim.x)) kinfo[e] = s[e];
}

// dst [C, ld] (bf16) = the per-expert transposes of the rows of src [*, C]: padded column
// kinfo[e] + i holds row kinfo[E + 1 + e] + i of expert e (read at gather[row] when gather is
// given), the padding columns up to kinfo[e + 1] hold zeros; columns past kinfo[E] are not
// written.  Tiles of 64 columns x 64 rows of dst staged through LDS; grid (ld / 64, C / 64),
// C % 64 == 0.
__global__ __launch_bounds__(256) void bwd_transpose_pad_kernel(const bf16_t* __restrict__ src,
                                                                const int32_t* __restrict__ gather, int C,
                                                                const int32_t* __restrict__ kinfo, int E,
                                                                bf16_t* __restrict__ dst, int64_t ld) {
  __shared__ uint32_t tile[64][33];  // [padded column q][pairs of source columns], odd pitch
  const int64_t q0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int c0 = static_cast<int>(blockIdx.y) * 64;
  if (q0 >= kinfo[E]) return;
  int lo = 0, hi = E - 1;  // the expert whose padded range holds q0 (ranges are multiples of 64)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (kinfo[mid] <= q0) lo = mid; else hi = mid - 1;
  }
  const int64_t off = q0 - kinfo[lo];
  const int64_t first = kinfo[E + 1 + lo] + off;
  const int64_t valid = kinfo[E + 2 + lo] - kinfo[E + 1 + lo] - off;  // >= 1
  const int tid = static_cast<int>(threadIdx.x);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = tid / 8 + 32 * j, cc = (tid % 8) * 8;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (i < valid) {
      int64_t r = first + i;
      if (gather) r = gather[r];
      v = *reinterpret_cast<const u32x4_t*>(src + r * C + c0 + cc);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) tile[i][cc / 2 + t] = v[t];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ci = tid / 8 + 32 * j, qq = (tid % 8) * 8;
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t a = tile[qq + 2 * t][ci / 2], b = tile[qq + 2 * t + 1][ci / 2];
      w[t] = (ci % 2) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    *reinterpret_cast<u32x4_t*>(dst + static_cast<int64_t>(c0 + ci) * ld + q0 + qq) = u32x4_t{w[0], w[1], w[2], w[3]};
  }
}

// dst [rows + pad, C] (bf16): row p = src[gather ? gather[p] : p] for p < rows, zeros after.
// One workgroup per row, C % 8 == 0.
__global__ __launch_bounds__(256) void bwd_gather_rows_kernel(const bf16_t* __restrict__ src,
                                                              const int32_t* __restrict__ gather, int64_t rows, int C,
                                                              bf16_t* __restrict__ dst) {
  const int64_t p = blockIdx.x;
  u32x4_t* d = reinterpret_cast<u32x4_t*>(dst + p * C);
  if (p < rows) {
    const u32x4_t* sp = reinterpret_cast<const u32x4_t*>(src + (gather ? static_cast<int64_t>(gather[p]) : p) * C);
    for (int c = static_cast<int>(threadIdx.x); c < C / 8; c += 256) d[c] = sp[c];
  } else {
    for (int c = static_cast<int>(threadIdx.x); c < C / 8; c += 256) d[c] = u32x4_t{0u, 0u, 0u, 0u};
  }
}

constexpr int kRouterPadRows = 64;  // zero rows after the last token of dW_r's B operand

// The router's products of a bf16 layer on the bf16 MFMA kernel, as accurate as fp32: dlogits dl
// (fp32) is split into three bf16 parts d1 + d2 + d3 (each the bf16 rounding, to nearest even, of
// what the parts before it leave; the remainders are exact in fp32) and so is W_r (w1 + w2 + w3);
// x is bf16 already.
//   dx_r = dl W_r^T: the six products d_a w_b with a + b <= 4 -- the three left out are below
//          2^-24 of the terms -- as one product over a 6E-deep contraction, the parts paired
//          [d3 d2 d1 d2 d1 d1] . [w1 w2 w3 w1 w2 w1], the smallest first;
//   dW_r = x^T dl = x^T d3 + x^T d2 + x^T d1: one per-slice product of x^T with [d3 d2 d1] over S
//          row slices of the tokens, then summed over the slices and the parts.
__device__ __forceinline__ void split_bf16x3(float v, bf16_t& p1, bf16_t& p2, bf16_t& p3) {
  p1 = f32_to_bf16(v);
  const float r1 = v - bf16_to_f32(p1);
  p2 = f32_to_bf16(r1);
  p3 = f32_to_bf16(r1 - bf16_to_f32(p2));
}

// a6 [T, 6E] = [d3 d2 d1 d2 d1 d1]; d3 [T + 64, 3E] = [d3 d2 d1], its last 64 rows zero.
__global__ __launch_bounds__(256) void bwd_split_dl_kernel(const float* __restrict__ dl, int64_t T, int E,
                                                           bf16_t* __restrict__ a6, bf16_t* __restrict__ d3) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= (T + kRouterPadRows) * E) return;
  const int64_t t = i / E;
  const int e = static_cast<int>(i % E);
  bf16_t* d = d3 + t * 3 * E + e;
  if (t >= T) {
    d[0] = d[E] = d[2 * E] = 0;
    return;
  }
  bf16_t p1, p2, p3;
  split_bf16x3(dl[t * E + e], p1, p2, p3);
  bf16_t* a = a6 + t * 6 * E + e;
  a[0] = p3; a[E] = p2; a[2 * E] = p1; a[3 * E] = p2; a[4 * E] = p1; a[5 * E] = p1;
  d[0] = p3; d[E] = p2; d[2 * E] = p1;
}

// b6 [H, 6E] = [w1 w2 w3 w1 w2 w1] of W_r [H, E] (row h of b6 is weight row h: the [N, K] operand).
__global__ __launch_bounds__(256) void bwd_split_wr_kernel(const float* __restrict__ wr, int H, int E,
                                                           bf16_t* __restrict__ b6) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(H) * E) return;
  const int64_t h = i / E;
  const int e = static_cast<int>(i % E);
  bf16_t p1, p2, p3;
  split_bf16x3(wr[i], p1, p2, p3);
  bf16_t* b = b6 + h * 6 * E + e;
  b[0] = p1; b[E] = p2; b[2 * E] = p3; b[3 * E] = p1; b[4 * E] = p2; b[5 * E] = p1;
}

// off[s] = T s / S, s = 0 .. S: the row slices of dW_r's contraction.
__global__ void bwd_slice_offsets_kernel(int64_t T, int S, int32_t* __restrict__ off) {
  const int s = static_cast<int>(threadIdx.x);
  if (s <= S) off[s] = static_cast<int32_t>(T * s / S);
}

// dW_r[h][e] = sum over the parts d3, d2, d1 (the smallest first) and, inside each, the slices in
// order of part[s][h][p E + e].
__global__ __launch_bounds__(256) void bwd_router_dw_sum_kernel(const float* __restrict__ part, int S, int H, int E,
                                                                float* __restrict__ dw) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(H) * E) return;
  const int64_t h = i / E;
  const int e = static_cast<int>(i % E);
  float acc = 0.0f;
  for (int p = 0; p < 3; ++p)
    for (int sl = 0; sl < S; ++sl) acc += part[(static_cast<int64_t>(sl) * H + h) * 3 * E + p * E + e];
  dw[i] = acc;
}

// Rows a per-expert product's B operand may read past the group's last row (its padding).
constexpr int kPadRows = 64;

// Padded contraction columns of the weight-gradient products: sum_e roundup(M_e, 64) <= rows + 64 E.
int64_t padded_cols(int64_t rows, int E) { return rows + static_cast<int64_t>(kPadRows) * E; }

// dW_e = (A^T)_e B_e for the groups of offsets (null: one group): the padded table, the transposed
// activation, the product.  B holds rows + kPadRows rows (the last kPadRows finite).
hipError_t wgrad_bf16(const bf16_t* act, const int32_t* act_gather, int C, const bf16_t* B, int N,
                      const int32_t* offsets, int64_t rows, int G, int32_t* kinfo, bf16_t* at, int64_t ld_t,
                      float* dw, hipStream_t s) {
  hipLaunchKernelGGL(bwd_kinfo_kernel, dim3(1), dim3(256), 0, s, offsets, rows, G, kinfo);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ld = padded_cols(rows, G);
  if (ld > ld_t) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_transpose_pad_kernel, dim3(static_cast<unsigned>(ceil_div(ld, 64)), C / 64), dim3(256), 0,
                     s, act, act_gather, C, kinfo, G, at, ld_t);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_batched_gemm_f32out(at, ld_t, B, kinfo, G, C, N, dw, s);
}

// The backward of one SwiGLU expert group (routed: offsets/src/gates given; shared: all null).
template <typename WT>
hipError_t expert_group_backward(const WT* x, const WT* dy, const WT* w1, const WT* w2, const int32_t* offsets,
                                 const int32_t* src, const float* gates, const int32_t* row_map, int64_t T, int k,
                                 int64_t rows, int G, int H, int F, float* u, float* dhp, WT* du, WT* gh, float* dg,
                                 WT* dxp, float* dw1, float* dw2, int32_t* kinfo, void* xt, void* dyp,
                                 int64_t ld_t, hipStream_t s, hipEvent_t const* ev) {
  auto mark = [&](int i) -> hipError_t { return ev && ev[i] ? hipEventRecord(ev[i], s) : hipSuccess; };
  const int64_t gx = src ? T : rows;
  if (rows == 0) {  // no rows: every weight gradient is zero (TN tiles without K steps), nothing else runs
    hipError_t e = launch_bwd_gemm<kTN>(args(gh, F, static_cast<const int32_t*>(nullptr), 0, dy, H, 0,
                                             static_cast<const int32_t*>(nullptr), 0, nullptr, 0, G, F, H, 0, dw2,
                                             H, int64_t{F} * H),
                                        s);
    if (e == hipSuccess)
      e = launch_bwd_gemm<kTN>(args(x, H, static_cast<const int32_t*>(nullptr), 0, static_cast<const WT*>(du), 2 * F,
                                    0, static_cast<const int32_t*>(nullptr), 0, nullptr, 0, G, H, 2 * F, 0, dw1,
                                    2 * F, int64_t{H} * 2 * F),
                               s);
    for (int i = 1; i <= 6 && e == hipSuccess; ++i) e = mark(i);
    return e;
  }
  // u = x[src] W1: bf16 on the forward's grouped-GEMM kernel (no SwiGLU epilogue, fp32 out)
  hipError_t e;
  if constexpr (std::is_same<WT, bf16_t>::value)
    e = launch_grouped_gemm_f32out(x, w1, offsets, rows, G, H, 2 * F, u, s, src);
  else
    e = launch_bwd_gemm<kNN>(args(x, H, src, gx, w1, 2 * F, int64_t{H} * 2 * F, nullptr, 0, offsets, rows, G, 0,
                                  2 * F, H, u, 2 * F, 0),
                             s);
  if (e == hipSuccess) e = mark(1);
  // dh' = dy[src] W2^T: bf16 on the forward's kernel with the weight read as stored ([F, H] = [N, K])
  if (e == hipSuccess) {
    if constexpr (std::is_same<WT, bf16_t>::value)
      e = launch_grouped_gemm_nt_f32out(dy, w2, offsets, rows, G, H, F, dhp, s, src);
    else
      e = launch_bwd_gemm<kNT>(args(dy, H, src, gx, w2, H, int64_t{F} * H, nullptr, 0, offsets, rows, G, 0, F, H,
                                    dhp, F, 0),
                               s);
  }
  if (e == hipSuccess) e = mark(2);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_swiglu_kernel<WT>, dim3(static_cast<unsigned>(rows)), dim3(256), 0, s, u, dhp, gates,
                     row_map, src, T, k, F, du, gh, dg);
  e = hipGetLastError();
  if (e == hipSuccess) e = mark(3);
  // dW2 = (g h)^T dy[src]: bf16 per expert on the forward's kernel (dy gathered into row order first)
  if (e == hipSuccess) {
    if constexpr (std::is_same<WT, bf16_t>::value) {
      hipLaunchKernelGGL(bwd_gather_rows_kernel, dim3(static_cast<unsigned>(rows + kPadRows)), dim3(256), 0, s, dy,
                         src, rows, H, static_cast<bf16_t*>(dyp));
      e = hipGetLastError();
      if (e == hipSuccess)
        e = wgrad_bf16(gh, nullptr, F, static_cast<const bf16_t*>(dyp), H, offsets, rows, G, kinfo,
                       static_cast<bf16_t*>(xt), ld_t, dw2, s);
    } else {
      e = launch_bwd_gemm<kTN>(args(gh, F, static_cast<const int32_t*>(nullptr), rows, dy, H, 0, src, gx, offsets,
                                    rows, G, F, H, 0, dw2, H, int64_t{F} * H),
                               s);
    }
  }
  if (e == hipSuccess) e = mark(4);
  // dx_perm = du W1^T (W1 [H, 2F] = [N, K] as stored); bf16 rows, like the forward's y_perm
  if (e == hipSuccess) {
    if constexpr (std::is_same<WT, bf16_t>::value)
      e = launch_grouped_gemm_nt_bf16out(du, w1, offsets, rows, G, 2 * F, H, dxp, s, nullptr);
    else
      e = launch_bwd_gemm<kNT>(args(static_cast<const WT*>(du), 2 * F, static_cast<const int32_t*>(nullptr), rows,
                                    w1, 2 * F, int64_t{H} * 2 * F, nullptr, 0, offsets, rows, G, 0, H, 2 * F, dxp, H,
                                    0),
                               s);
  }
  if (e == hipSuccess) e = mark(5);
  // dW1 = x[src]^T du: bf16 per expert on the forward's kernel (du's kPadRows rows after its end zeroed)
  if (e == hipSuccess) {
    if constexpr (std::is_same<WT, bf16_t>::value) {
      hipLaunchKernelGGL(bwd_gather_rows_kernel, dim3(kPadRows), dim3(256), 0, s, du, nullptr, int64_t{0}, 2 * F,
                         du + rows * 2 * F);
      e = hipGetLastError();
      if (e == hipSuccess)
        e = wgrad_bf16(x, src, H, du, 2 * F, offsets, rows, G, kinfo, static_cast<bf16_t*>(xt), ld_t, dw1, s);
    } else {
      e = launch_bwd_gemm<kTN>(args(x, H, src, gx, static_cast<const WT*>(du), 2 * F, 0,
                                    static_cast<const int32_t*>(nullptr), rows, offsets, rows, G, H, 2 * F, 0, dw1,
                                    2 * F, int64_t{H} * 2 * F),
                               s);
    }
  }
  if (e == hipSuccess) e = mark(6);
  return e;
}

template <typename WT>
hipError_t layer_backward(const BackwardShape& sh, const BackwardIO& io, const BackwardScratch& ws, hipStream_t s,
                          hipEvent_t const* ev) {
  auto mark = [&](int i) -> hipError_t { return ev && ev[i] ? hipEventRecord(ev[i], s) : hipSuccess; };
  const int64_t T = sh.T, R = T * sh.k;
  const WT* x = static_cast<const WT*>(io.x);
  const WT* dy = static_cast<const WT*>(io.dy);
  hipError_t e = mark(0);
  if (e == hipSuccess)
    e = expert_group_backward<WT>(x, dy, static_cast<const WT*>(io.w1), static_cast<const WT*>(io.w2), io.offsets,
                                  io.src_token, io.gates, io.row_map, T, sh.k, R, sh.E, sh.H, sh.F, ws.u, ws.dhp,
                                  static_cast<WT*>(ws.du), static_cast<WT*>(ws.gh), ws.dg, static_cast<WT*>(ws.dxp),
                                  io.dw1, io.dw2,
                                  ws.kinfo, ws.xt, ws.dyp, ws.ld_t, s, ev);
  if (e == hipSuccess && sh.Fs > 0)
    e = expert_group_backward<WT>(x, dy, static_cast<const WT*>(io.ws1), static_cast<const WT*>(io.ws2), nullptr,
                                  nullptr, nullptr, nullptr, T, 1, T, 1, sh.H, sh.Fs, ws.us, ws.dhs,
                                  static_cast<WT*>(ws.dus), static_cast<WT*>(ws.ghs), nullptr, static_cast<WT*>(ws.dxs),
                                  io.dws1,
                                  io.dws2, ws.kinfo_s, ws.xt, ws.dyp, ws.ld_t, s, nullptr);
  if (e == hipSuccess) e = mark(7);
  if (e != hipSuccess) return e;
  if (T > 0) {
    hipLaunchKernelGGL(bwd_gate_kernel, dim3(static_cast<unsigned>(ceil_div(T, 256 / kWave))), dim3(256), 0, s,
                       io.logits, io.ids, ws.dg, io.row_map, T, sh.E, sh.k, sh.score, sh.norm, R, ws.dl);
    e = hipGetLastError();
  }
  // dx_router = dl W_r^T (W_r [H, E] read as [N = H, K = E]); dW_r = x^T dl
  if constexpr (std::is_same<WT, bf16_t>::value) {
    if (ws.ra6 != nullptr) {  // router_split: split bf16 products on the grouped-GEMM kernel
      const int E = sh.E, H = sh.H, S = ws.rS;
      const int64_t n = int64_t{H} * E;
      if (e == hipSuccess) {
        hipLaunchKernelGGL(bwd_split_dl_kernel, dim3(static_cast<unsigned>(ceil_div((T + kRouterPadRows) * E, 256))),
                           dim3(256), 0, s, static_cast<const float*>(ws.dl), T, E, static_cast<bf16_t*>(ws.ra6),
                           static_cast<bf16_t*>(ws.rd3));
        e = hipGetLastError();
      }
      if (e == hipSuccess) {
        hipLaunchKernelGGL(bwd_split_wr_kernel, dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, s,
                           io.w_router, H, E, static_cast<bf16_t*>(ws.rb6));
        e = hipGetLastError();
      }
      if (e == hipSuccess)
        e = launch_grouped_gemm_nt_f32out(ws.ra6, ws.rb6, nullptr, T, 1, 6 * E, H, ws.dxr, s, nullptr);
      if (e == hipSuccess) {
        hipLaunchKernelGGL(bwd_slice_offsets_kernel, dim3(1), dim3(64), 0, s, T, S, ws.roff);
        e = hipGetLastError();
      }
      if (e == hipSuccess)
        e = wgrad_bf16(x, nullptr, H, static_cast<const bf16_t*>(ws.rd3), 3 * E, ws.roff, T, S, ws.kinfo,
                       static_cast<bf16_t*>(ws.xt), ws.ld_t, ws.rpart, s);
      if (e == hipSuccess) {
        hipLaunchKernelGGL(bwd_router_dw_sum_kernel, dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, s,
                           ws.rpart, S, H, E, io.dw_router);
        e = hipGetLastError();
      }
    }
  }
  if (ws.ra6 == nullptr) {
    if (e == hipSuccess)
      e = launch_bwd_gemm<kNT>(args(static_cast<const float*>(ws.dl), sh.E, static_cast<const int32_t*>(nullptr), T,
                                    io.w_router, sh.E, 0, nullptr, 0, nullptr, T, 1, 0, sh.H, sh.E, ws.dxr, sh.H, 0),
                               s);
    const int S = router_slices(T, sh.H, sh.E);
    if (e == hipSuccess)
      e = launch_bwd_gemm<kTN>(args(x, sh.H, static_cast<const int32_t*>(nullptr), T,
                                    static_cast<const float*>(ws.dl), sh.E, 0, static_cast<const int32_t*>(nullptr), T,
                                    nullptr, T, S, sh.H, sh.E, 0, S > 1 ? ws.dwr_part : io.dw_router, sh.E,
                                    int64_t{sh.H} * sh.E),
                               s);
    if (e == hipSuccess && S > 1) {
      const int64_t n = int64_t{sh.H} * sh.E;
      hipLaunchKernelGGL(bwd_sum_slices_kernel, dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, s,
                         ws.dwr_part, S, n, io.dw_router);
      e = hipGetLastError();
    }
  }
  if (e == hipSuccess && T > 0) {
    hipLaunchKernelGGL(bwd_dx_kernel<WT>, dim3(static_cast<unsigned>(T)), dim3(256), 0, s,
                       static_cast<const WT*>(ws.dxp), io.row_map, R, sh.k,
                       sh.Fs > 0 ? static_cast<const WT*>(ws.dxs) : nullptr,
                       static_cast<const float*>(ws.dxr), sh.H, static_cast<WT*>(io.dx));
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = mark(8);
  return e;
}

}  // namespace

bool router_split(const BackwardShape& sh, int dt) { return dt != 0 && sh.E % 32 == 0 && sh.H % 64 == 0 && sh.T > 0; }

int router_split_slices(int64_t T) {
  // about 1024 tokens per slice, at most 6 (the [H, 3E] product then has enough tiles)
  const int64_t S = T / 1024;
  return S < 1 ? 1 : (S > 6 ? 6 : static_cast<int>(S));
}

int router_slices(int64_t T, int H, int E) {
  // enough slices for ~512 workgroups, each of at least 64 rows, at most 32
  const int64_t tiles = ceil_div(H, kTile) * ceil_div(E, kTile);
  int64_t S = ceil_div(512, tiles);
  if (S > T / 64) S = T / 64;
  if (S > 32) S = 32;
  return S < 1 ? 1 : static_cast<int>(S);
}

BackwardScratch carve_backward(const BackwardShape& sh, int dt, void* base, size_t* bytes) {
  const size_t cts = dt == 0 ? 4 : 2;
  const int64_t T = sh.T, R = T * sh.k;
  char* b = static_cast<char*>(base);
  size_t used = 0;
  auto take = [&](size_t n) -> void* {
    void* p = b ? b + used : nullptr;
    used += (n + 255) & ~static_cast<size_t>(255);
    return p;
  };
  BackwardScratch w{};
  if (router_split(sh, dt)) {
    const int64_t E = sh.E;
    w.rS = router_split_slices(T);
    w.ra6 = take(T * 6 * E * 2);
    w.rb6 = take(int64_t{sh.H} * 6 * E * 2);
    w.rd3 = take((T + kRouterPadRows) * 3 * E * 2);
    w.rpart = static_cast<float*>(take(static_cast<size_t>(w.rS) * sh.H * 3 * E * 4));
    w.roff = static_cast<int32_t*>(take(static_cast<size_t>(w.rS + 1) * 4));
  } else {
    const int S = router_slices(T, sh.H, sh.E);
    w.dwr_part = S > 1 ? static_cast<float*>(take(static_cast<size_t>(S) * sh.H * sh.E * 4)) : nullptr;
  }
  const bool bf16 = dt != 0;
  const int64_t pad = bf16 ? kPadRows : 0;  // zero rows after du and dy's row-order copy (bf16 weight gradients)
  w.u = static_cast<float*>(take(R * 2 * sh.F * 4));
  w.dhp = static_cast<float*>(take(R * sh.F * 4));
  w.du = take((R + pad) * 2 * sh.F * cts);
  w.gh = take(R * sh.F * cts);
  w.dg = static_cast<float*>(take(R * 4));
  w.dxp = take(R * sh.H * cts);
  w.dl = static_cast<float*>(take(T * sh.E * 4));
  w.dxr = static_cast<float*>(take(T * sh.H * 4));
  if (sh.Fs > 0) {
    w.us = static_cast<float*>(take(T * 2 * sh.Fs * 4));
    w.dhs = static_cast<float*>(take(T * sh.Fs * 4));
    w.dus = take((T + pad) * 2 * sh.Fs * cts);
    w.ghs = take(T * sh.Fs * cts);
    w.dxs = take(T * sh.H * cts);
  }
  if (bf16) {
    // one transposed activation at a time ([H or F or Fs][ld_t]); ld_t covers both groups' padding
    const int64_t ld_r = padded_cols(R, sh.E), ld_s = sh.Fs > 0 ? padded_cols(T, 1) : 0;
    w.ld_t = ((ld_r > ld_s ? ld_r : ld_s) + 63) / 64 * 64;
    const int64_t cmax_ = sh.H > sh.F ? (sh.H > sh.Fs ? sh.H : sh.Fs) : (sh.F > sh.Fs ? sh.F : sh.Fs);
    w.kinfo = static_cast<int32_t*>(take(static_cast<size_t>(2 * (sh.E + 1)) * 4));
    w.kinfo_s = static_cast<int32_t*>(take(4 * 4));
    w.xt = take(static_cast<size_t>(cmax_) * w.ld_t * 2);
    w.dyp = take(static_cast<size_t>((R > T ? R : T) + pad) * sh.H * 2);
  }
  if (bytes) *bytes = used;
  return w;
}

hipError_t launch_layer_backward(const BackwardShape& sh, int dt, const BackwardIO& io, const BackwardScratch& ws,
                                 hipStream_t stream, hipEvent_t const* events) {
  if (dt == 0) return layer_backward<float>(sh, io, ws, stream, events);
  if (dt == 1) return layer_backward<bf16_t>(sh, io, ws, stream, events);
  return hipErrorNotSupported;
}

}  // namespace moe
