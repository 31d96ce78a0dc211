// gemm_common.hpp -- pieces shared by the grouped GEMM kernels (bf16 and fp8): the device-side
// tile scheduler and the LDS-DMA / wait-count helpers.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace moe {
namespace gemm {

constexpr int kBN = 256;              // N per tile (SwiGLU: 128 gate + 128 up columns)
constexpr int kMaxExpertsLds = 520;   // >= E + 1 for E <= 512
constexpr int kGemmThreads = 512;     // 8 waves, two per SIMD

// Per-workgroup tile lookup built from the device-resident expert offsets.
struct TileMap {
  int expert, mt, nt;
  int64_t row0, row_end;  // this tile's first row and the expert's end row
};

// Words of the prefix buffer past E + 1 (E <= 512) where the scan leaves two statistics of
// the scanned values: their maximum and how many are non-zero.
constexpr int kStatMax = kMaxExpertsLds - 2, kStatNonzero = kMaxExpertsLds - 1;

// Rows [base, base + M) of expert e: the caller's offsets clamped into [0, rows] and made
// non-decreasing, so that offsets breaking the contract (not monotone, or past `rows`, the
// bound the launch was sized for) can drop or repeat work but never address rows outside
// [0, rows).
__device__ __forceinline__ void expert_rows(const int32_t* offsets, int e, int64_t rows, int64_t& base,
                                            int64_t& M) {
  int64_t lo = offsets[e], hi = offsets[e + 1];
  lo = lo < 0 ? 0 : (lo > rows ? rows : lo);
  hi = hi < lo ? lo : (hi > rows ? rows : hi);
  base = lo;
  M = hi - lo;
}

// In-place inclusive scan of s_pref[1..E] by one wave (E <= 512, chunks of 64), s_pref[0] = 0,
// and the statistics above; every thread of the workgroup calls it after writing s_pref[1..E].
__device__ void scan_prefix(int* s_pref, int E) {
  const int tid = threadIdx.x;
  if (tid == 0) s_pref[0] = 0;
  __syncthreads();
  if (tid < kWave) {
    int carry = 0, mx = 0, nz = 0;
    for (int base = 1; base <= E; base += kWave) {
      int i = base + tid;
      int v = i <= E ? s_pref[i] : 0;
      mx = v > mx ? v : mx;
      nz += v != 0;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        int u = __shfl_up(v, o, kWave);
        if (tid >= o) v += u;
      }
      if (i <= E) s_pref[i] = v + carry;
      carry += __shfl(v, kWave - 1, kWave);
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int m2 = __shfl_xor(mx, o, kWave);
      mx = m2 > mx ? m2 : mx;
      nz += __shfl_xor(nz, o, kWave);
    }
    if (tid == 0) {
      s_pref[kStatMax] = mx;
      s_pref[kStatNonzero] = nz;
    }
  }
  __syncthreads();
}

// Tile count (m-tiles summed over experts, times NT); builds the m-tile prefix in s_pref.
template <int BM>
__device__ int count_tiles(const int32_t* offsets, int64_t rows, int E, int NT, int* s_pref) {
  if (offsets == nullptr) return static_cast<int>(ceil_div(rows, BM)) * NT;
  const int tid = threadIdx.x;
  // m-tiles per expert, exclusive prefix in s_pref[0..E]
  for (int e = tid; e < E; e += static_cast<int>(blockDim.x)) {
    int64_t base, c;
    expert_rows(offsets, e, rows, base, c);
    s_pref[e + 1] = static_cast<int>((c + BM - 1) / BM);
  }
  scan_prefix(s_pref, E);
  return s_pref[E] * NT;
}


// Tiles that do not fill the last wave of `ncu` workgroups when run whole (at most `ncu` - 1): with
// S > 1 each of them is cut into up to S row bands (so the last wave holds several times as many
// pieces, each with a fraction of the MFMA work).
__device__ __forceinline__ int whole_tiles(int total, int ncu, int S) {
  return S > 1 ? total - total % ncu : total;
}

// Rows per m-tile when an expert's M rows are spread evenly over its ceil(M / BM) m-tiles, in
// whole 32-row blocks (<= BM).  Equal tiles run at equal speed (a tile computes only its live
// row blocks), so the m-tiles that share a weight tile stay in step and share it through L2.
// The last tile takes the remainder, which can be empty when rounding up overshoots.
template <int BM>
__device__ __forceinline__ int64_t balanced_rows(int64_t M, int mtiles) {
  const int64_t per = (M + mtiles - 1) / mtiles;
  return (per + 31) / 32 * 32;
}

// Linear tile L -> (expert, m-tile, n-tile); n-major inside an expert so the m-tiles of one
// weight tile are adjacent.  A tile covers rows [row0, row_end): at most BM of its expert.
template <int BM>
__device__ void locate_tile(const int32_t* offsets, int64_t rows, int E, int NT, const int* s_pref, int L,
                            TileMap& tm) {
  if (offsets == nullptr) {  // one dense expert over rows [0, rows)
    const int mtiles = static_cast<int>(ceil_div(rows, BM));
    tm.expert = 0;
    tm.nt = L / mtiles;
    tm.mt = L % mtiles;
    const int64_t rpt = balanced_rows<BM>(rows, mtiles);
    tm.row0 = static_cast<int64_t>(tm.mt) * rpt;
    tm.row_end = tm.row0 + rpt < rows ? tm.row0 + rpt : rows;
    return;
  }
  // expert whose tile range [s_pref[e]*NT, s_pref[e+1]*NT) holds L (binary search in LDS)
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_pref[mid] * NT <= L) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int me = s_pref[e + 1] - s_pref[e];
  const int idx = L - s_pref[e] * NT;
  tm.expert = e;
  tm.nt = idx / me;
  tm.mt = idx % me;
  int64_t base, M;
  expert_rows(offsets, e, rows, base, M);
  const int64_t rpt = balanced_rows<BM>(M, me);
  tm.row0 = base + static_cast<int64_t>(tm.mt) * rpt;
  tm.row_end = tm.row0 + rpt < base + M ? tm.row0 + rpt : base + M;
}

// Returns false if this workgroup has no tile.  `s_pref` is LDS of >= E+1 ints.  Workgroups
// [0, 8 ceil(W / 8)) take the W whole tiles, XCD-remapped (consecutive tiles on one XCD share
// weights and rows in its L2); the following ones take the S row bands of each tail tile.
template <int BM>
__device__ bool map_tile_counted(const int32_t* offsets, int64_t rows, int E, int NT, const int* s_pref,
                                 int total, TileMap& tm, int ncu, int S) {
  const int whole = whole_tiles(total, ncu, S);
  const int per = (whole + 7) / 8;
  const int w = blockIdx.x;
  if (w < 8 * per) {
    const int L = (w % 8) * per + w / 8;
    if (L >= whole) return false;
    locate_tile<BM>(offsets, rows, E, NT, s_pref, L, tm);
    return tm.row0 < tm.row_end;  // an even split can leave the last m-tile empty
  }
  // Tail: as many bands per tile as still fit one wave (at most S; bands are whole 32-row
  // blocks).  Pieces P = tile * SB + band are XCD-remapped like the whole tiles, whole tiles'
  // worth of pieces per XCD, so the bands of one tile (which stream the same weight tile) run on
  // one XCD.
  const int tail = total - whole;
  int SB = ncu / (tail > 0 ? tail : 1);
  SB = SB < 1 ? 1 : (SB > S ? S : SB);
  const int band_rows = (BM / SB + 31) / 32 * 32;
  const int pieces = tail * SB;
  const int per_t = (tail + 7) / 8 * SB;
  const int q = w - 8 * per;
  if (q >= 8 * per_t) return false;
  const int P = (q % 8) * per_t + q / 8;
  if (P >= pieces) return false;
  locate_tile<BM>(offsets, rows, E, NT, s_pref, whole + P / SB, tm);
  tm.row0 += static_cast<int64_t>(P % SB) * band_rows;
  const int64_t band_end = tm.row0 + band_rows;
  if (band_end < tm.row_end) tm.row_end = band_end;
  return tm.row0 < tm.row_end;  // band past the tile's last row, or an empty tile
}

template <int BM>
__device__ bool map_tile(const int32_t* offsets, int64_t rows, int E, int NT, int* s_pref, TileMap& tm,
                         int ncu = 0, int S = 1) {
  const int total = count_tiles<BM>(offsets, rows, E, NT, s_pref);
  return map_tile_counted<BM>(offsets, rows, E, NT, s_pref, total, tm, ncu, S);
}

// Alternative whole-tile map that spreads every expert's work evenly over the 8 XCDs: the NT m_e
// tiles of expert e, in n-tile -> m-tile order, are cut into 8 contiguous ranges of equal size
// (+-1), range x for XCD x.  On its XCD, workgroup w / 8 takes that XCD's tiles expert by expert,
// so the m-tiles sharing a weight tile stay adjacent and share it through that XCD's L2 (only a
// weight tile cut by a range boundary is fetched by two XCDs).  With skewed loads (a few experts
// with many m-tiles) the map above gives each XCD a contiguous range of equal tile count but very
// unequal work; here each XCD gets the same share of every expert.  On entry `s_pref` holds the
// m-tile prefix (count_tiles).  The launch needs grid_for_spread workgroups.
template <int BM>
__device__ bool map_tile_spread(const int32_t* offsets, int64_t rows, int E, int NT, int* s_pref, TileMap& tm) {
  const int x = static_cast<int>(blockIdx.x % 8), i = static_cast<int>(blockIdx.x / 8);
  auto range_start = [&](int me, int xx) { return static_cast<int>(static_cast<int64_t>(xx) * me * NT / 8); };
  // A thread owns experts tid and tid + blockDim (blockDim >= 256, E <= 512).
  const int e0 = static_cast<int>(threadIdx.x), e1 = e0 + static_cast<int>(blockDim.x);
  const int me0 = e0 < E ? s_pref[e0 + 1] - s_pref[e0] : 0;
  const int me1 = e1 < E ? s_pref[e1 + 1] - s_pref[e1] : 0;
  __syncthreads();
  if (e0 < E) s_pref[e0 + 1] = range_start(me0, x + 1) - range_start(me0, x);  // this XCD's tiles of e0
  if (e1 < E) s_pref[e1 + 1] = range_start(me1, x + 1) - range_start(me1, x);
  scan_prefix(s_pref, E);
  if (i >= s_pref[E]) return false;
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_pref[mid] <= i) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  int64_t base, M;
  expert_rows(offsets, e, rows, base, M);
  const int me = static_cast<int>(ceil_div(M, BM));
  const int j = range_start(me, x) + (i - s_pref[e]);  // tile of expert e, n-major
  tm.expert = e;
  tm.nt = j / me;
  tm.mt = j % me;
  const int64_t rpt = balanced_rows<BM>(M, me);
  tm.row0 = base + static_cast<int64_t>(tm.mt) * rpt;
  tm.row_end = tm.row0 + rpt < base + M ? tm.row0 + rpt : base + M;
  return tm.row0 < tm.row_end;
}

// Picks the tile map: map_tile_spread when the expert loads are skewed (the busiest expert has
// more than 3x the mean m-tile count of the experts with rows), else map_tile.  The statistics
// come out of the m-tile prefix scan, so every workgroup reaches the same decision from the
// same offsets at no extra cost.  The grid must cover both maps (grid_for_any).  `s_pref` is
// LDS of kMaxExpertsLds ints (E <= 512).
template <int BM>
__device__ bool map_tile_auto(const int32_t* offsets, int64_t rows, int E, int NT, int* s_pref, TileMap& tm,
                              int ncu = 0, int S = 1) {
  const int total = count_tiles<BM>(offsets, rows, E, NT, s_pref);
  if (offsets != nullptr) {
    const int64_t mtiles = s_pref[E];
    if (static_cast<int64_t>(s_pref[kStatMax]) * s_pref[kStatNonzero] > 3 * mtiles)
      return map_tile_spread<BM>(offsets, rows, E, NT, s_pref, tm);
  }
  return map_tile_counted<BM>(offsets, rows, E, NT, s_pref, total, tm, ncu, S);
}

// Operand modes of the bf16 grouped GEMM (gemm.hip): weights [K, N]; weights [N, K]; independent
// per-expert GEMMs with contractions of their own (the weight gradients).
constexpr int kModeNN = 0, kModeNT = 1, kModeBatchK = 2;

// Tile map of the batched mode: E independent [M, N] outputs of MT x NT tiles each.  The tiles of
// one expert are walked in groups of 8 m-tiles, n-major inside a group (the tiles running together
// then share 8 row blocks of A and a few column blocks of B in L2), and every XCD takes a
// contiguous range of this order (workgroup w runs on XCD w % 8).  The launch has
// 8 ceil(E MT NT / 8) workgroups.
template <int BM>
__device__ bool map_tile_batched(int64_t M, int E, int NT, TileMap& tm) {
  const int MT = static_cast<int>(ceil_div(M, BM));
  const int per_e = MT * NT;
  const int total = E * per_e;
  const int per = (total + 7) / 8;
  const int w = blockIdx.x;
  const int L = (w % 8) * per + w / 8;
  if (L >= total) return false;
  const int e = L / per_e, idx = L % per_e;
  const int g = idx / (8 * NT);
  const int gm = MT - 8 * g < 8 ? MT - 8 * g : 8;
  const int r = idx - g * 8 * NT;
  tm.expert = e;
  tm.nt = r / gm;
  tm.mt = 8 * g + r % gm;
  tm.row0 = static_cast<int64_t>(e) * M + static_cast<int64_t>(tm.mt) * BM;
  tm.row_end = static_cast<int64_t>(e) * M + M;
  return true;
}

constexpr int cmax(int a, int b) { return a > b ? a : b; }

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// 16 bytes per lane from global memory straight into LDS at lds_addr + 16 * lane
// (global_load_lds_dwordx4).  Issued through asm so the compiler does not insert its own
// conservative vmcnt waits before unrelated LDS reads; completion is tracked explicitly with
// wait_vmcnt (vmcnt retires loads in issue order, so the compiler's own counts stay safe).
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_addr) {
  // an SALU write of M0 needs one wait state before an LDS-DMA load reads it
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt encoding: vmcnt [3:0] + [15:14], expcnt [6:4] (7 = no wait), lgkmcnt [11:8] (15)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Wait (vmcnt) until at most N - STEP * d loads are still in flight, d in [0, D] (wave-uniform):
// the count of a wave that skips d loads in each of STEP load groups issued after the awaited one.
template <int N, int STEP, int D>
__device__ __forceinline__ void wait_vmcnt_less(int d) {
  if constexpr (STEP == 0 || D == 0) {
    wait_vmcnt<N>();
  } else {
    if (d >= D) wait_vmcnt<N - STEP * D>();
    else wait_vmcnt_less<N, STEP, D - 1>(d);
  }
}

// Wait (vmcnt) until at most `tiles` (<= MAXT) tiles of RPT loads each are still in flight.
template <int RPT, int MAXT>
__device__ __forceinline__ void wait_tiles(int tiles) {
  if constexpr (MAXT >= 2) {
    if (tiles >= 2) { wait_vmcnt<2 * RPT>(); return; }
  }
  if constexpr (MAXT >= 1) {
    if (tiles >= 1) { wait_vmcnt<RPT>(); return; }
  }
  wait_vmcnt<0>();
}

__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14)); }

// SiLU for the epilogue: z * 1 / (1 + 2^(-z log2 e)) with the hardware exp2 and reciprocal
// (about 1e-6 relative error, far below the bf16 rounding of h).
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}


// Calls f(std::integral_constant<int, n>) for the runtime n in [0, MAXN] (wave-uniform).
template <int MAXN, typename Fn>
__device__ __forceinline__ void dispatch_live(int n, Fn&& f) {
  if constexpr (MAXN > 0) {
    if (n >= MAXN) { f(std::integral_constant<int, MAXN>{}); return; }
    dispatch_live<MAXN - 1>(n, f);
  } else {
    f(std::integral_constant<int, 0>{});
  }
}

template <int BM>
inline int64_t max_tiles(int64_t rows, int E, bool dense) {
  return dense ? ceil_div(rows, BM) : (rows + static_cast<int64_t>(E) * (BM - 1)) / BM;
}

inline unsigned grid_for_spread(int64_t mtiles, int NT, int E) {
  return static_cast<unsigned>(8 * (ceil_div(mtiles * NT, 8) + E));  // per XCD: sum_e ceil(NT m_e / 8)
}

inline unsigned grid_for(int64_t mtiles, int NT, int ncu = 0, int S = 1) {
  int64_t g = mtiles * NT;
  if (S > 1) g += 7 + 7 * S + static_cast<int64_t>(ncu - 1) * (S - 1);  // roundings to 8 + tail bands
  return static_cast<unsigned>(ceil_div(g, 8) * 8);
}

// Workgroups for map_tile_auto: enough for either map.
inline unsigned grid_for_any(int64_t mtiles, int NT, int E, bool dense, int ncu = 0, int S = 1) {
  const unsigned a = grid_for(mtiles, NT, ncu, S);
  if (dense) return a;  // one expert: always the contiguous map
  const unsigned b = grid_for_spread(mtiles, NT, E);
  return a > b ? a : b;
}

}  // namespace gemm
}  // namespace moe
