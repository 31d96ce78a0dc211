// gemm_fp8.hip -- Compute stage with FP8 (OCP E4M3) expert GEMMs and fp32 block scales.
//
// Selective FP8 on the expert GEMMs with the router kept in higher precision ("Scalable Training
// of Mixture-of-Experts Models with Megatron Core", summary page, "Key claims" [§5] and "Method"
// second paragraph).  Operands: x_perm codes with one fp32 scale per row and 128-wide K block,
// weights [K, N] codes with one fp32 scale per 128 x 128 block.  The SwiGLU activation h is
// quantised to E4M3 in 1 x 128 blocks inside the path (scale: the smallest power of two that
// maps the block's amax into +-448).
//
// Tile 128 x 256 x 128 (K step = one scale block), 8 waves in a 2 (M) x 4 (N) grid, each wave
// 64 x 64 = 2 x 2 blocks of v_mfma_scale_f32_32x32x64_f8f6f4 issued with unit (E8M0 = 127)
// scales.  Per K step the two 64-deep MFMAs of a block accumulate into a temporary, then
//     acc += tmp * s_a[row] * s_b[block]
// on the VALU.  Operands stream global -> LDS (global_load_lds_dwordx4; the row scales of the
// step with global_load_lds_dword) through a ring of three LDS stages, so a tile's loads have
// two iterations to land:
//   A stage: 128 rows x 128 B, chunk c of row r at c ^ ((r >> 1) & 7) (as the bf16 kernel);
//   B stage: 128 k-rows x 256 B (untransposed), chunk c of k-row k at c ^ 2 (k & 7).
// The weight block scales are wave-uniform and come through the scalar cache.
// B fragments come from ds_read_b64_tr_b8: within a group of 16 lanes, lane 16g + 8a + b
// receives byte b of the 8-byte pieces addressed by lanes 16g + a + 2e (e = 0..7), so source
// lane s addresses k-row 8 q + (s % 16) / 2 (+ 32 (s / 32)) at column 16 ((s / 16) % 2) + 8 (s % 2)
// of the fragment and destination lane d collects column d % 32 for 8 consecutive k.
#include "gemm_common.hpp"

namespace moe {
namespace {

using namespace gemm;

constexpr int kF8BM = 128;    // rows per tile
constexpr int kF8BK = 128;    // K per iteration = one scale block
constexpr int kF8BRow = kBN;  // bytes per B k-row (256 fp8 columns)
constexpr int kF8Stages = 3;
constexpr int kF8Stage = kF8BM * kF8BK + kF8BK * kF8BRow;  // A + B of one K tile
constexpr int kF8ScaleSlots = kF8Stages + 1;                // row-scale ring, one slot longer
constexpr int kF8Smem = kF8Stages * kF8Stage + kF8ScaleSlots * kF8BM * 4;

typedef int v2i32_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i32_t lds_v2i32_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4_t;

// 4 bytes per lane from global memory straight into LDS at lds_addr + 4 * lane.
__device__ __forceinline__ void lds_dma4(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gptr), "s"(lds_addr)
               : "memory", "m0");
}

template <bool SWIGLU, bool OUT_F32>
__global__ __launch_bounds__(kGemmThreads) void gemm_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ A_scales, const uint8_t* __restrict__ B,
    const float* __restrict__ B_scales, const int32_t* __restrict__ offsets, int64_t rows, int E, int K,
    int ldb, int NT, void* __restrict__ out, float* __restrict__ out_scales, const int32_t* __restrict__ gather) {
  constexpr int NWAVE = kGemmThreads / kWave;  // 8
  constexpr int BM = kF8BM;
  constexpr int FM = 2, FN = 2;
  constexpr int A_BYTES = BM * kF8BK;           // 16 KB
  constexpr int B_BYTES = kF8BK * kF8BRow;      // 32 KB
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int NS = kF8Stages;
  constexpr int A_ROUNDS = A_BYTES / 1024 / NWAVE;  // 2
  constexpr int B_ROUNDS = B_BYTES / 1024 / NWAVE;  // 4
  constexpr int RPT = A_ROUNDS + B_ROUNDS;          // loads per wave per tile (+1 on waves 0, 1)
  static_assert(STAGE == kF8Stage && NS * STAGE + kF8ScaleSlots * BM * 4 == kF8Smem, "LDS layout");

  extern __shared__ __attribute__((aligned(1024))) char smem[];
  __shared__ int s_pref[kMaxExpertsLds];

  TileMap tm;
  if (!map_tile<BM>(offsets, rows, E, NT, s_pref, tm)) return;
  const int t_expert = __builtin_amdgcn_readfirstlane(tm.expert);  // uniform: scalar address math
  const int t_nt = __builtin_amdgcn_readfirstlane(tm.nt);

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 4, wn = wave % 4;
  const int khalf = lane / 32;
  lds_void_t* lds = (lds_void_t*)smem;  // address-space cast: generic -> LDS
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
  const int nkb = K / kF8BK;

  // ---- global sources of the direct loads
  const uint8_t* a_src[A_ROUNDS];
#pragma unroll
  for (int p = 0; p < A_ROUNDS; ++p) {
    const int r = (NWAVE * p + wave) * 8 + lane / 8;
    int64_t grow = tm.row0 + r;
    if (grow >= tm.row_end) grow = tm.row_end - 1;
    if (gather) grow = gather[grow];  // fused dispatch: row p of the tile is token gather[p]
    a_src[p] = A + grow * K + (((lane % 8) ^ ((r >> 1) & 7)) * 16);
  }
  // row scales of the step: waves 0 and 1 gather 64 rows each (one dword per lane)
  const float* as_src;
  {
    int64_t grow = tm.row0 + (wave % 2) * 64 + lane;
    if (grow >= tm.row_end) grow = tm.row_end - 1;
    if (gather) grow = gather[grow];
    as_src = A_scales + grow * nkb;
  }
  // B round p of wave w covers k-rows 4 (8p + w) + lane / 16 (1 KB = 4 k-rows x 256 B); stored
  // chunk lane % 16 holds logical chunk (lane % 16) ^ 2 ((4w + lane / 16) & 7).
  const int b_lchunk = (lane % 16) ^ (2 * ((4 * wave + lane / 16) & 7));
  int64_t b_col;
  if (SWIGLU) {
    const int F = ldb / 2;
    b_col = (b_lchunk < 8) ? static_cast<int64_t>(tm.nt) * 128 + b_lchunk * 16
                           : F + static_cast<int64_t>(tm.nt) * 128 + (b_lchunk - 8) * 16;
  } else {
    b_col = static_cast<int64_t>(tm.nt) * kBN + b_lchunk * 16;
  }
  if (b_col >= ldb) b_col = 0;  // ldb % 128 == 0: a 16-column group is wholly in or out
  const uint8_t* b_src = B + static_cast<int64_t>(tm.expert) * K * ldb +
                         static_cast<int64_t>(4 * wave + lane / 16) * ldb + b_col;
  const int64_t b_round = static_cast<int64_t>(4 * NWAVE) * ldb;
  // weight block scales of this wave's two column blocks
  const int nbn = ldb / 128;
  int blk[FN];
  if (SWIGLU) {
    blk[0] = t_nt;
    blk[1] = ldb / 256 + t_nt;
  } else {
    const int c0 = t_nt * 2 + wn / 2;
    blk[0] = blk[1] = c0 < nbn ? c0 : 0;
  }
  const float* bs_src = B_scales + static_cast<int64_t>(t_expert) * nkb * nbn;

  auto stage_base = [&](int kt) { return lds_base + static_cast<uint32_t>(kt % NS) * STAGE; };
  // row scales of tile kt live in their own ring slot, which the loads issued at the barrier of
  // iteration kt (tile kt + NS) do not touch, so they can be read after that barrier
  auto scale_base = [&](int kt) {
    return lds_base + NS * STAGE + static_cast<uint32_t>(kt % kF8ScaleSlots) * (BM * 4);
  };
  auto issue_loads = [&](int kt) {
    const uint32_t sbase = stage_base(kt);
#pragma unroll
    for (int p = 0; p < A_ROUNDS; ++p)
      lds_dma16(a_src[p] + static_cast<int64_t>(kt) * kF8BK, sbase + (NWAVE * p + wave) * 1024);
    if (wave < 2) lds_dma4(as_src + kt, scale_base(kt) + wave * 256);
    const uint8_t* bs = b_src + static_cast<int64_t>(kt) * kF8BK * ldb;
#pragma unroll
    for (int p = 0; p < B_ROUNDS; ++p)
      lds_dma16(bs + p * b_round, sbase + A_BYTES + (NWAVE * p + wave) * 1024);
  };

  // ---- fragment addresses
  uint32_t a_row_off[FM], a_sw[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = wm * 64 + i * 32 + lane % 32;
    a_row_off[i] = r * 128;
    a_sw[i] = (r >> 1) & 7;
  }
  uint32_t b_off[FN];
  {
    const int g = lane / 16, a2 = lane % 2, e = (lane % 16) / 2;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int cb = SWIGLU ? j * 128 + wn * 32 : wn * 64 + j * 32;
      const int col = cb + 16 * (g % 2) + 8 * a2;
      b_off[j] = (32 * (g / 2) + e) * kF8BRow + (((col / 16) ^ (2 * e)) << 4) + (col % 16);
    }
  }

  f32x16_t acc[FM][FN], tmp[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const f32x16_t zero16 = {};

  // Only the 32-row blocks of this wave that hold rows of the expert are computed (wave-uniform).
  int nl_rows = static_cast<int>((tm.row_end - tm.row0 < BM ? tm.row_end - tm.row0 : BM)) - wm * 64;
  nl_rows = nl_rows < 0 ? 0 : nl_rows;
  const int nlive = __builtin_amdgcn_readfirstlane(nl_rows >= 64 ? FM : (nl_rows + 31) / 32);

  const int nk = nkb;
  auto run = [&](auto nl_c) {
    constexpr int NL = decltype(nl_c)::value;
    constexpr int NLA = NL > 0 ? NL : 1;
    i32x8_t af[2][NLA], bfr[2][FN];
    auto read_a = [&](uint32_t sbase, int s, int buf, int i) {
      const uint32_t c0 = 4 * s + 2 * khalf;
      u32x4_t lo = *reinterpret_cast<const lds_u32x4_t*>(
          static_cast<uintptr_t>(sbase + a_row_off[i] + ((c0 ^ a_sw[i]) << 4)));
      u32x4_t hi = *reinterpret_cast<const lds_u32x4_t*>(
          static_cast<uintptr_t>(sbase + a_row_off[i] + (((c0 + 1) ^ a_sw[i]) << 4)));
      af[buf][i] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    auto read_b = [&](uint32_t sbase, int s, int buf, int j) {
      const uint32_t bbase = sbase + A_BYTES + s * 64 * kF8BRow;
      v2i32_t q[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        q[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            reinterpret_cast<lds_v2i32_t*>(static_cast<uintptr_t>(bbase + b_off[j] + r * 8 * kF8BRow)));
      bfr[buf][j] = i32x8_t{q[0][0], q[0][1], q[1][0], q[1][1], q[2][0], q[2][1], q[3][0], q[3][1]};
    };
    // sub-step s (0, 1) of tile kt: 64 K bytes; A lane l holds k 32 (l / 32) .. +32 of it.
    // Read in the order the MFMAs (i-major) consume them: B0, A0, B1, A1.
    auto read_frags = [&](int kt, int s, int buf) {
      if constexpr (NL > 0) {
        const uint32_t sbase = stage_base(kt);
        read_b(sbase, s, buf, 0);
        read_a(sbase, s, buf, 0);
#pragma unroll
        for (int j = 1; j < FN; ++j) read_b(sbase, s, buf, j);
#pragma unroll
        for (int i = 1; i < NL; ++i) read_a(sbase, s, buf, i);
      }
    };
    auto mfmas = [&](int buf, bool first) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          tmp[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[buf][i], bfr[buf][j],
                                                                       first ? zero16 : tmp[i][j], 0, 0, 0, 127, 0, 127);
    };
    // row scales of this lane's 16 accumulator rows per block i: 4 runs of 4 consecutive rows
    f32x4_t sa[NLA][4];
    auto read_row_scales = [&](int kt) {
      const uint32_t sbase = scale_base(kt);
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = wm * 64 + i * 32 + q * 8 + khalf * 4;
          sa[i][q] = *reinterpret_cast<const lds_f32x4_t*>(static_cast<uintptr_t>(sbase + row * 4));
        }
    };

    float sb[FN], sb_next[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) sb[j] = bs_src[blk[j]];
    const int pro = nk < NS ? nk : NS;  // tiles in flight before the loop
    for (int t = 0; t < pro; ++t) issue_loads(t);
    if (wave < 2) wait_tiles<RPT + 1, NS - 1>(pro - 1); else wait_tiles<RPT, NS - 1>(pro - 1);  // tile 0 landed
    lds_barrier();
    read_frags(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int ktn = kt + 1 < nk ? kt + 1 : kt;
#pragma unroll
      for (int j = 0; j < FN; ++j) sb_next[j] = bs_src[static_cast<int64_t>(ktn) * nbn + blk[j]];
      mfmas(0, true);
      read_frags(kt, 1, 1);
      if (kt + 1 < nk) {
        wait_lgkm0();  // this wave's reads of tile kt are complete
        // this wave's loads of tile kt + 1 have landed; tiles kt + 2 .. kt + NS - 1 may be in flight
        const int later = nk - 2 - kt < NS - 2 ? nk - 2 - kt : NS - 2;
        if (wave < 2) wait_tiles<RPT + 1, NS - 2>(later); else wait_tiles<RPT, NS - 2>(later);
        lds_barrier();  // for every wave: tile kt + 1 readable, tile kt's stage free
        if (kt + NS < nk) issue_loads(kt + NS);
      }
      mfmas(1, false);
      read_frags(kt + 1, 0, 0);  // past the last tile this reads a stale stage (in bounds, unused)
      read_row_scales(kt);
      // promote the block: acc += tmp * s_a[row] * s_b[column block]
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(tmp[i][j][r], sa[i][r / 4][r % 4] * sb[j], acc[i][j][r]);
#pragma unroll
      for (int j = 0; j < FN; ++j) sb[j] = sb_next[j];
    }
  };
  dispatch_live<FM>(nlive, run);

  // ---- epilogue.  32x32 accumulator layout: slot r of lane l is
  //      row (r / 4) * 8 + (l / 32) * 4 + (r % 4), column l % 32.
  if (SWIGLU) {
    // h = SiLU(gate) * up for this lane's 2 x 16 rows, then E4M3 in 1 x 128 blocks: the tile's
    // 128 h columns are one block, spread over the 4 N-waves (32 columns each).
    const int F = ldb / 2;
    float h[FM][16];
    float amax[FM][16];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        h[i][r] = silu_fast(acc[i][0][r]) * acc[i][1][r];
        float m = fabsf(h[i][r]);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
        amax[i][r] = m;
      }
    wait_lgkm0();
    __syncthreads();  // every wave is done with the LDS stages
    float* red = reinterpret_cast<float*>(smem);  // [BM rows][4 N-waves]
    if (lane % 32 == 0) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row_t = wm * 64 + i * 32 + (r / 4) * 8 + khalf * 4 + (r % 4);
          red[row_t * 4 + wn] = amax[i][r];
        }
    }
    __syncthreads();
    uint8_t* hq = static_cast<uint8_t*>(out);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row_t = wm * 64 + i * 32 + (r / 4) * 8 + khalf * 4 + (r % 4);
        const int64_t grow = tm.row0 + row_t;
        if (grow >= tm.row_end) continue;
        const float m = fmaxf(fmaxf(red[row_t * 4 + 0], red[row_t * 4 + 1]), fmaxf(red[row_t * 4 + 2], red[row_t * 4 + 3]));
        const float sc = e4m3_block_scale(m);  // a power of two
        const float v = fminf(fmaxf(h[i][r] / sc, -448.0f), 448.0f);
        const int64_t col = static_cast<int64_t>(tm.nt) * 128 + wn * 32 + lane % 32;
        hq[grow * F + col] = static_cast<uint8_t>(f32_to_e4m3(v));
        if (wn == 0 && lane % 32 == 0) out_scales[grow * (F / 128) + tm.nt] = sc;
      }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row_t = wm * 64 + i * 32 + (r / 4) * 8 + khalf * 4 + (r % 4);
        const int64_t grow = tm.row0 + row_t;
        if (grow >= tm.row_end) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t col = static_cast<int64_t>(tm.nt) * kBN + wn * 64 + j * 32 + lane % 32;
          if (col >= ldb) continue;
          if (OUT_F32)
            static_cast<float*>(out)[grow * ldb + col] = acc[i][j][r];
          else
            static_cast<bf16_t*>(out)[grow * ldb + col] = f32_to_bf16(acc[i][j][r]);
        }
      }
  }
}

template <bool SWIGLU, bool OUT_F32>
hipError_t launch_fp8(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs, const int32_t* offsets,
                      int64_t rows, int E, int K, int ldb, int NT, void* out, float* out_scales,
                      hipStream_t stream, const int32_t* gather = nullptr) {
  constexpr int smem = kF8Smem;
  auto kern = gemm_fp8_kernel<SWIGLU, OUT_F32>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (attr != hipSuccess) return attr;
  const unsigned grid = grid_for(max_tiles<kF8BM>(rows, E, offsets == nullptr), NT);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kGemmThreads), smem, stream, A, As, B, Bs, offsets, rows, E, K, ldb,
                     NT, out, out_scales, gather);
  return hipGetLastError();
}

}  // namespace

size_t fp8_hidden_bytes(int64_t rows, int F) {
  return (static_cast<size_t>(rows) * F + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_grouped_swiglu_fp8(const void* x_perm, const float* x_scales, const int32_t* offsets,
                                     int64_t rows, int E, int H, int F, const void* w1, const float* w1_scales,
                                     const void* w2, const float* w2_scales, void* y_perm, int out_dt,
                                     void* scratch, hipStream_t stream, hipEvent_t between, const int32_t* gather) {
  uint8_t* hq = static_cast<uint8_t*>(scratch);
  float* hs = reinterpret_cast<float*>(static_cast<char*>(scratch) + fp8_hidden_bytes(rows, F));
  hipError_t err = launch_fp8<true, false>(static_cast<const uint8_t*>(x_perm), x_scales,
                                           static_cast<const uint8_t*>(w1), w1_scales, offsets, rows, E, H, 2 * F,
                                           F / 128, hq, hs, stream, gather);
  if (err != hipSuccess) return err;
  if (between && (err = hipEventRecord(between, stream)) != hipSuccess) return err;
  const int nt2 = static_cast<int>(ceil_div(H, kBN));
  if (out_dt == 0)
    return launch_fp8<false, true>(hq, hs, static_cast<const uint8_t*>(w2), w2_scales, offsets, rows, E, F, H, nt2,
                                   y_perm, nullptr, stream);
  return launch_fp8<false, false>(hq, hs, static_cast<const uint8_t*>(w2), w2_scales, offsets, rows, E, F, H, nt2,
                                  y_perm, nullptr, stream);
}

}  // namespace moe
