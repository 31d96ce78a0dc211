// gemm_fp8.hip -- Compute stage with FP8 (OCP E4M3) expert GEMMs and fp32 block scales.
//
// Selective FP8 on the expert GEMMs with the router kept in higher precision ("Scalable Training
// of Mixture-of-Experts Models with Megatron Core", summary page, "Key claims" [§5] and "Method"
// second paragraph).  Operands: x_perm codes with one fp32 scale per row and 128-wide K block,
// weights [K, N] codes with one fp32 scale per 128 x 128 block.  The SwiGLU activation h is
// quantised to E4M3 in 1 x 128 blocks inside the path (scale: the smallest power of two that
// maps the block's amax into +-448).
//
// Tiles BM x 256 x 128 (K step = one scale block), 8 waves in a 2 (M) x 4 (N) grid, each wave
// (BM / 2) x 64 in 32 x 32 blocks of v_mfma_scale_f32_32x32x64_f8f6f4.  Operands stream
// global -> LDS (global_load_lds_dwordx4) through two rings of LDS stages:
//   A stage: BM rows x 128 B, chunk c of row r at c ^ ((r >> 1) & 7) (as the bf16 kernel);
//   B stage: 128 k-rows x 256 B (untransposed), chunk c of k-row k at c ^ 2 (k & 7);
// and, loaded with each A stage (global_load_lds_dword), a slot of scales: the row scales of
// the step and the tile's two weight block scales.
// B fragments come from ds_read_b64_tr_b8: within a group of 16 lanes, lane 16g + 8a + b
// receives byte b of the 8-byte pieces addressed by lanes 16g + a + 2e (e = 0..7), so source
// lane s addresses k-row 8 q + (s % 16) / 2 (+ 32 (s / 32)) at column 16 ((s / 16) % 2) + 8 (s % 2)
// of the fragment and destination lane d collects column d % 32 for 8 consecutive k.
#include "gemm_common.hpp"

namespace moe {
namespace {

using namespace gemm;

constexpr int kF8BK = 128;    // K per iteration = one scale block
constexpr int kF8BRow = kBN;  // bytes per B k-row (256 fp8 columns)

// Two variants share the kernel below:
//  * general (BM = 128): any fp32 weight block scales.  Each 128-deep K block's two MFMAs go to a
//    temporary with unit scales, then acc += tmp * s_a[row] * s_b[block] on the VALU; three
//    LDS stages of A and of B.
//  * MX (BM = 192): every weight block scale is a power of two (as the activation scales always
//    are), so the scaled MFMA applies both as E8M0 exponents and accumulates straight into acc:
//    no temporary, no promotion, 96 x 64 wave tiles (128 x 64 would need more than the 256
//    registers a wave has at two waves per SIMD); two LDS stages of A and three of B (the
//    weights, which miss L2 more often, get the deeper ring).
// A device flag (set by fp8_scale_check_kernel) tells which variant runs; the other exits.
template <int BM>
struct F8Cfg {
  static constexpr bool MX = BM != 128;
  static constexpr int NA = MX ? 2 : 3;                      // LDS stages of A (activation rows)
  static constexpr int NB = 3;                               // LDS stages of B (weights)
  static constexpr int A_BYTES = BM * kF8BK;
  static constexpr int B_BYTES = kF8BK * kF8BRow;
  static constexpr int SLOTS = NA + 1;                       // scale ring (travels with A), one longer
  static constexpr int SLOT = BM * 4 + 256;                  // row scales + the tile's 2 weight scales
  static constexpr int B_RING = NA * A_BYTES;
  static constexpr int S_RING = B_RING + NB * B_BYTES;
  static constexpr int SMEM = S_RING + SLOTS * SLOT;
};

typedef int v2i32_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i32_t lds_v2i32_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4_t;

// 4 bytes per lane from global memory straight into LDS at lds_addr + 4 * lane.
__device__ __forceinline__ void lds_dma4(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gptr),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// flag = 1 unless every scale of the three arrays is a power of two 2^q, q in [-127, 127].
__global__ __launch_bounds__(256) void fp8_scale_check_kernel(const float* __restrict__ s0, int64_t n0,
                                                              const float* __restrict__ s1, int64_t n1,
                                                              const float* __restrict__ s2, int64_t n2,
                                                              int* __restrict__ flag) {
  bool bad = false;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n0 + n1 + n2;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const float v = i < n0 ? s0[i] : (i < n0 + n1 ? s1[i - n0] : s2[i - n0 - n1]);
    const uint32_t u = __float_as_uint(v);
    const uint32_t e = (u >> 23) & 0xFFu;
    const bool pow2 = ((u & 0x807FFFFFu) == 0u && e != 0u && e != 0xFFu) || u == 0x00400000u;
    bad = bad || !pow2;
  }
  if (__any(bad) && threadIdx.x % kWave == 0) atomicOr(flag, 1);
}

__global__ void fp8_flag_clear_kernel(int* flag) { *flag = 0; }

template <int BM, bool SWIGLU, bool OUT_F32>
__global__ __launch_bounds__(kGemmThreads) void gemm_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ A_scales, const uint8_t* __restrict__ B,
    const float* __restrict__ B_scales, const int32_t* __restrict__ offsets, int64_t rows, int E, int K,
    int ldb, int NT, void* __restrict__ out, float* __restrict__ out_scales, const int32_t* __restrict__ gather,
    const float* __restrict__ row_scale,
    const int* __restrict__ mx_flag) {
  using C = F8Cfg<BM>;
  constexpr bool MX = C::MX;
  constexpr int NWAVE = kGemmThreads / kWave;  // 8: 2 along M x 4 along N
  constexpr int WROWS = BM / 2;                // rows per wave
  constexpr int FM = WROWS / 32, FN = 2;
  constexpr int A_BYTES = C::A_BYTES, B_BYTES = C::B_BYTES;
  constexpr int NA = C::NA, NB = C::NB;
  constexpr int SW = BM / 64;                       // waves gathering the row scales (64 rows each)
  static_assert(BM % 64 == 0 && A_BYTES % (1024 * NWAVE) == 0, "tile height");
  static_assert(NA >= 2 && NB >= 2 && SW < NWAVE, "ring depths");
  constexpr int A_ROUNDS = A_BYTES / 1024 / NWAVE;  // 2 or 3
  constexpr int B_ROUNDS = B_BYTES / 1024 / NWAVE;  // 4
  // loads per wave per group: A part A_ROUNDS (+1 scale load on waves <= SW), B part B_ROUNDS
  constexpr int RPT = A_ROUNDS + B_ROUNDS;

  // the variant the scales allow runs; the other exits before touching anything
  if (mx_flag && ((*mx_flag == 0) != MX)) return;

  extern __shared__ __attribute__((aligned(1024))) char smem[];
  __shared__ int s_pref[kMaxExpertsLds];

  TileMap tm;
  // skewed loads: the SwiGLU GEMM spreads every expert over the XCDs (the second GEMM, whose
  // activation rows are as large as its weights, measured better on the contiguous map)
  if (SWIGLU ? !map_tile_auto<BM>(offsets, rows, E, NT, s_pref, tm) : !map_tile<BM>(offsets, rows, E, NT, s_pref, tm))
    return;
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
  // row scales of the step: waves 0 .. SW-1 gather 64 rows each (one dword per lane)
  const float* as_src;
  {
    int64_t grow = tm.row0 + (wave % SW) * 64 + lane;
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
  // The tile's two weight column blocks (SwiGLU: the gate and the up block; else columns 0-127
  // and 128-255 of the tile).  Wave SW loads their scales into the scale slot (lane l: block
  // l % 2); the wave's block j uses slot entry wslot[j].
  const int nbn = ldb / 128;
  int wslot[FN];
  int64_t ws_off;
  {
    int b0, b1;
    if (SWIGLU) {
      b0 = t_nt;
      b1 = ldb / 256 + t_nt;
    } else {
      b0 = t_nt * 2;
      b1 = t_nt * 2 + 1 < nbn ? t_nt * 2 + 1 : 0;  // past the last column: unused
    }
    ws_off = static_cast<int64_t>(t_expert) * nkb * nbn + (lane % 2 ? b1 : b0);
#pragma unroll
    for (int j = 0; j < FN; ++j) wslot[j] = SWIGLU ? j : wn / 2;
  }
  const float* ws_src = B_scales + ws_off;

  auto a_stage = [&](int kt) { return lds_base + static_cast<uint32_t>(kt % NA) * A_BYTES; };
  auto b_stage = [&](int kt) { return lds_base + C::B_RING + static_cast<uint32_t>(kt % NB) * B_BYTES; };
  // The scales of tile kt (loaded with A tile kt) live in their own ring slot, which the loads
  // issued at the barriers of iterations kt - 1 and kt (A tiles kt - 1 + NA, kt + NA) do not touch.
  auto scale_base = [&](int kt) {
    return lds_base + C::S_RING + static_cast<uint32_t>(kt % C::SLOTS) * C::SLOT;
  };
  // Load group j: A tile j + NA with its scales and B tile j + NB, each if it exists.  Group j is
  // issued at iteration j (the prologue issues groups -max(NA, NB) .. -1).
  auto issue_a = [&](int j) {
    const int ta = j + NA;
    if (ta >= 0 && ta < nkb) {
      const uint32_t abase = a_stage(ta);
#pragma unroll
      for (int p = 0; p < A_ROUNDS; ++p)
        lds_dma16(a_src[p] + static_cast<int64_t>(ta) * kF8BK, abase + (NWAVE * p + wave) * 1024);
      if (wave < SW) lds_dma4(as_src + ta, scale_base(ta) + wave * 256);
      if (wave == SW) lds_dma4(ws_src + static_cast<int64_t>(ta) * nbn, scale_base(ta) + BM * 4);
    }
  };
  auto b_load = [&](int tb, int p) {
    lds_dma16(b_src + static_cast<int64_t>(tb) * kF8BK * ldb + p * b_round, b_stage(tb) + (NWAVE * p + wave) * 1024);
  };
  auto issue_group = [&](int j) {
    issue_a(j);
    const int tb = j + NB;
    if (tb >= 0 && tb < nkb) {
#pragma unroll
      for (int p = 0; p < B_ROUNDS; ++p) b_load(tb, p);
    }
  };
  // vmcnt waits (per wave: RPTW = RPT, +1 on waves <= SW).  In the loop group j goes out at the
  // barrier of iteration j; with power-of-two scales (MX) only its A part (with the scales) does,
  // one load after each MFMA and fragment read of the second sub-step, and its B part follows in
  // the first sub-step of iteration j + 1 in the same way (a direct load issued ahead of a wave's
  // LDS reads delays them).  The prologue issues whole groups.  Tile t
  // is complete once the later of its A and B parts has landed: loads issued after that part are
  // the B part of its group (when NB > NA) and then whole groups -- min(NA, NB) - 1 after the
  // prologue (tile 0), and min(NA, NB) - 2 at iteration t (tile t + 1) -- when every tile those
  // groups name exists (max(NA, NB) <= nk, t + max(NA, NB) <= nk).  Otherwise wait for all.
  constexpr int NM = NA > NB ? NA : NB, GM = NA < NB ? NA : NB;
  constexpr int AFTER = NB > NA ? B_ROUNDS : 0;
  auto wait_tile = [&](bool full, auto groups_c) {
    constexpr int G = decltype(groups_c)::value;
    if (!full) wait_vmcnt<0>();
    else if (wave <= SW) wait_vmcnt<AFTER + G * (RPT + 1)>();
    else wait_vmcnt<AFTER + G * RPT>();
  };

  // ---- fragment addresses
  uint32_t a_row_off[FM], a_sw[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = wm * WROWS + i * 32 + lane % 32;
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

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Only the 32-row blocks of this wave that hold rows of the expert are computed (wave-uniform).
  int nl_rows = static_cast<int>((tm.row_end - tm.row0 < BM ? tm.row_end - tm.row0 : BM)) - wm * WROWS;
  nl_rows = nl_rows < 0 ? 0 : nl_rows;
  const int nlive = __builtin_amdgcn_readfirstlane(nl_rows >= WROWS ? FM : (nl_rows + 31) / 32);

  const int nk = nkb;
  auto run = [&](auto nl_c) {
    constexpr int NL = decltype(nl_c)::value;
    constexpr int NLA = NL > 0 ? NL : 1;
    i32x8_t af[2][NLA], bfr[2][FN];
    auto read_a = [&](uint32_t abase, int s, int buf, int i) {
      const uint32_t c0 = 4 * s + 2 * khalf;
      u32x4_t lo = *reinterpret_cast<const lds_u32x4_t*>(
          static_cast<uintptr_t>(abase + a_row_off[i] + ((c0 ^ a_sw[i]) << 4)));
      u32x4_t hi = *reinterpret_cast<const lds_u32x4_t*>(
          static_cast<uintptr_t>(abase + a_row_off[i] + (((c0 + 1) ^ a_sw[i]) << 4)));
      af[buf][i] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    auto read_b = [&](uint32_t bstage, int s, int buf, int j) {
      const uint32_t bbase = bstage + s * 64 * kF8BRow;
      v2i32_t q[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        q[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            reinterpret_cast<lds_v2i32_t*>(static_cast<uintptr_t>(bbase + b_off[j] + r * 8 * kF8BRow)));
      bfr[buf][j] = i32x8_t{q[0][0], q[0][1], q[1][0], q[1][1], q[2][0], q[2][1], q[3][0], q[3][1]};
    };
    // sub-step s (0, 1) of tile kt: 64 K bytes; A lane l holds k 32 (l / 32) .. +32 of it.
    // Read in the order the MFMAs (i-major) consume them: B0, A0, B1, A1, ...
    auto read_frags = [&](int kt, int s, int buf) {
      if constexpr (NL > 0) {
        const uint32_t abase = a_stage(kt), bbase = b_stage(kt);
        read_b(bbase, s, buf, 0);
        read_a(abase, s, buf, 0);
#pragma unroll
        for (int j = 1; j < FN; ++j) read_b(bbase, s, buf, j);
#pragma unroll
        for (int i = 1; i < NL; ++i) read_a(abase, s, buf, i);
      }
    };

    // The first groups of loads, then the loop.
    for (int j = -NM; j < 0; ++j) issue_group(j);
    wait_tile(NM <= nk, std::integral_constant<int, GM - 1>{});  // tile 0 landed
    lds_barrier();
    read_frags(0, 0, 0);

    if constexpr (MX) {
      // E8M0 exponents: per lane its A row's scale (one per 32-row block), per block j the weight
      // block scale.  Tile kt + 1's are read from the scale ring right after the barrier that
      // makes that tile readable, a sub-step before they are needed.
      int sae[NLA], sbe[FN], sae_n[NLA], sbe_n[FN];
      auto read_exps = [&](int kt) {
        const uint32_t sbase = scale_base(kt);
#pragma unroll
        for (int i = 0; i < NL; ++i)
          sae_n[i] = e8m0_of(*reinterpret_cast<const __attribute__((address_space(3))) float*>(
              static_cast<uintptr_t>(sbase + (wm * WROWS + i * 32 + lane % 32) * 4)));
#pragma unroll
        for (int j = 0; j < FN; ++j)
          sbe_n[j] = e8m0_of(*reinterpret_cast<const __attribute__((address_space(3))) float*>(
              static_cast<uintptr_t>(sbase + BM * 4 + wslot[j] * 4)));
      };
      auto take_exps = [&]() {
#pragma unroll
        for (int i = 0; i < NL; ++i) sae[i] = sae_n[i];
#pragma unroll
        for (int j = 0; j < FN; ++j) sbe[j] = sbe_n[j];
      };
      read_exps(0);
      take_exps();
      constexpr int NR = NL > 0 ? NL + FN : 0;  // read units: B0, A0, B1, A1, A2, ...
      // read unit q of sub-step s of tile kt into buffer buf
      auto read_unit = [&](int kt, int s, int buf, int q) {
        if constexpr (NL > 0) {
          if (q < NR) {
            if (q == 0) read_b(b_stage(kt), s, buf, 0);
            else if (q == 1) read_a(a_stage(kt), s, buf, 0);
            else if (q < 2 + FN - 1) read_b(b_stage(kt), s, buf, q - 1);
            else read_a(a_stage(kt), s, buf, q - FN);
          }
        }
      };
      for (int kt = 0; kt < nk; ++kt) {
        // First sub-step: MFMA q, fragment read q of the second sub-step, then load q of B tile
        // kt - 1 + NB (the B part of group kt - 1; its stage was freed at the last barrier).
        {
          const int tb = kt - 1 + NB;
          const bool do_b = kt >= 1 && tb < nk;
          constexpr int NQ = cmax(cmax(NL * FN, NR), B_ROUNDS);  // slots: every MFMA, read and load
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            if (q < NL * FN) {
              const int i = q / FN, j = q % FN;
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[0][j], af[0][i], acc[i][j], 0, 0, 0,
                                                                           sbe[j], 0, sae[i]);
            }
            read_unit(kt, 1, 1, q);
            if (q >= NQ - B_ROUNDS && do_b) b_load(tb, q - (NQ - B_ROUNDS));
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (kt + 1 < nk) {
          wait_lgkm0();  // this wave's reads of tile kt are complete
          wait_tile(kt + NM <= nk, std::integral_constant<int, GM - 2>{});  // tile kt + 1 landed
          lds_barrier();  // for every wave: tile kt + 1 readable, tile kt's stages free
          read_exps(kt + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        // Second sub-step: MFMA q, fragment read q of tile kt + 1, then load q of the A part of
        // group kt (A rounds, then the scale load), so the MFMA pipe restarts right after the
        // barrier.
        {
          const int ta = kt + NA;
          const bool do_a = kt + 1 < nk && ta < nk;
          const uint32_t abase = a_stage(ta);
          constexpr int NLD = A_ROUNDS + 1;  // load slots (the scale slot is empty on waves > SW)
          constexpr int NQ = cmax(cmax(NL * FN, NR), NLD);
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            if (q < NL * FN) {
              const int i = q / FN, j = q % FN;
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[1][j], af[1][i], acc[i][j], 0, 0, 0,
                                                                           sbe[j], 0, sae[i]);
            }
            read_unit(kt + 1, 0, 0, q);  // unconditional: a branch would make the compiler wait for it
            const int p = q - (NQ - NLD);  // the loads take the last NLD slots
            if (p >= 0 && p < A_ROUNDS) {
              if (do_a) lds_dma16(a_src[p] + static_cast<int64_t>(ta) * kF8BK, abase + (NWAVE * p + wave) * 1024);
            } else if (p == A_ROUNDS) {
              if (do_a && wave < SW) lds_dma4(as_src + ta, scale_base(ta) + wave * 256);
              if (do_a && wave == SW) lds_dma4(ws_src + static_cast<int64_t>(ta) * nbn, scale_base(ta) + BM * 4);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (kt + 1 < nk) take_exps();
      }
    } else {
      f32x16_t tmp[NLA][FN];
      const f32x16_t zero16 = {};
      auto mfmas = [&](int buf, bool first) {
#pragma unroll
        for (int i = 0; i < NL; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            tmp[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[buf][j], af[buf][i],
                                                                         first ? zero16 : tmp[i][j], 0, 0, 0, 127, 0,
                                                                         127);
      };
      // Scales of tile kt for the promotion at the end of its iteration, read before the next
      // sub-step's fragments so that the promotion does not wait for those: per block i the scale
      // of this lane's accumulator row, per block j the weight block's.
      float sa[NLA];
      float sb[FN];
      auto read_scales = [&](int kt) {
        const uint32_t sbase = scale_base(kt);
#pragma unroll
        for (int i = 0; i < NL; ++i)
          sa[i] = *reinterpret_cast<const __attribute__((address_space(3))) float*>(
              static_cast<uintptr_t>(sbase + (wm * WROWS + i * 32 + lane % 32) * 4));
#pragma unroll
        for (int j = 0; j < FN; ++j)
          sb[j] = *reinterpret_cast<const __attribute__((address_space(3))) float*>(
              static_cast<uintptr_t>(sbase + BM * 4 + wslot[j] * 4));
      };
      for (int kt = 0; kt < nk; ++kt) {
        mfmas(0, true);
        read_frags(kt, 1, 1);
        if (kt + 1 < nk) {
          wait_lgkm0();  // this wave's reads of tile kt are complete
          wait_tile(kt + NM <= nk, std::integral_constant<int, GM - 2>{});  // tile kt + 1 landed
          lds_barrier();  // for every wave: tile kt + 1 readable, tile kt's stages free
          issue_group(kt);
        }
        mfmas(1, false);
        read_scales(kt);
        read_frags(kt + 1, 0, 0);  // past the last tile this reads a stale stage (in bounds, unused)
        // promote the block: acc += tmp * s_a[row] * s_b[column block]
#pragma unroll
        for (int i = 0; i < NL; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(tmp[i][j][r], sa[i] * sb[j], acc[i][j][r]);
      }
    }
  };
  dispatch_live<FM>(nlive, run);

  // ---- epilogue.  The MFMAs take the weight fragment as their first operand, so each computes a
  //      transposed 32x32 block: slot r of lane l of acc[i][j] is the wave's row i * 32 + l % 32
  //      and column j * 32 + (r / 4) * 8 + (l / 32) * 4 + (r % 4) of block j -- 4 adjacent
  //      columns of one row per group of 4 slots, written to LDS or memory 16 (fp32) or 8 (bf16)
  //      bytes at a time.
  if (SWIGLU) {
    // h = SiLU(gate) * up, staged through LDS as fp32 rows of the tile's 128 h columns (one 1 x 128
    // quantisation block per row).  Read back by 8 consecutive lanes per row, 16 columns each:
    // the block amax is a register max and 3 shuffles, and each lane stores 16 E4M3 codes at once.
    constexpr int kHS = 132;  // row stride in floats: 16 consecutive rows start 4 banks apart
    static_assert(BM * kHS * 4 <= C::S_RING, "h staging fits in the operand rings");
    const int F = ldb / 2;
    wait_lgkm0();
    __syncthreads();  // every wave is done with the operand ring
    float* hl = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i * 32 >= nl_rows) continue;  // no row of this block is live (wave-uniform)
      const int row_t = wm * WROWS + i * 32 + lane % 32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4_t w;
#pragma unroll
        for (int t = 0; t < 4; ++t) w[t] = silu_fast(acc[i][0][4 * q + t]) * acc[i][1][4 * q + t];
        *reinterpret_cast<f32x4_t*>(hl + row_t * kHS + wn * 32 + q * 8 + khalf * 4) = w;
      }
    }
    __syncthreads();
    uint8_t* hq = static_cast<uint8_t*>(out);
    const int seg = tid % 8;
#pragma unroll
    for (int pass = 0; pass < BM / 64; ++pass) {
      const int row_t = pass * 64 + tid / 8;
      const f32x4_t* src = reinterpret_cast<const f32x4_t*>(hl + row_t * kHS + seg * 16);
      const int64_t grow = tm.row0 + row_t;
      // gate folded into the expert: h of the row scaled by its gate before the block is quantised
      const float g = row_scale != nullptr ? row_scale[grow < tm.row_end ? grow : tm.row_end - 1] : 1.0f;
      f32x4_t v[4];
      float m = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = src[q];
        if (row_scale != nullptr) v[q] *= g;
        m = fmaxf(fmaxf(m, fmaxf(fabsf(v[q][0]), fabsf(v[q][1]))), fmaxf(fabsf(v[q][2]), fabsf(v[q][3])));
      }
      m = fmaxf(m, __shfl_xor(m, 1, kWave));
      m = fmaxf(m, __shfl_xor(m, 2, kWave));
      m = fmaxf(m, __shfl_xor(m, 4, kWave));
      if (grow < tm.row_end) {
        const float sc = e4m3_block_scale(m);  // a power of two
        const float inv = pow2_inverse(sc);    // exact: x * inv == x / sc
        u32x4_t codes;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float r[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) r[c] = fminf(fmaxf(v[q][c] * inv, -448.0f), 448.0f);
          codes[q] = pack_e4m3x4(r[0], r[1], r[2], r[3]);
        }
        *reinterpret_cast<u32x4_t*>(hq + grow * F + static_cast<int64_t>(tm.nt) * 128 + seg * 16) = codes;
        if (seg == 0) out_scales[grow * (F / 128) + tm.nt] = sc;
      }
    }
  } else if (!OUT_F32) {
    // bf16 y staged through LDS as [BM][256] (+ padding), 4 adjacent columns (8 bytes) per lane and
    // LDS write, and stored 16 bytes (8 columns) per lane along whole tile rows
    constexpr int kYS = 264;  // row stride in bf16: rows 16-byte aligned
    static_assert(BM * kYS * 2 <= C::S_RING, "y staging fits in the operand rings");
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    wait_lgkm0();
    __syncthreads();  // every wave is done with the operand ring
    bf16_t* yl = reinterpret_cast<bf16_t*>(smem);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i * 32 >= nl_rows) continue;  // no row of this block is live (wave-uniform)
      const int row_t = wm * WROWS + i * 32 + lane % 32;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2_t w = {pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                             pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
          *reinterpret_cast<u32x2_t*>(yl + row_t * kYS + wn * 64 + j * 32 + q * 8 + khalf * 4) = w;
        }
    }
    __syncthreads();
    const int seg = tid % 32;  // 8 columns each, 32 lanes per row
    const int64_t col = static_cast<int64_t>(tm.nt) * kBN + seg * 8;
    if (col < ldb) {  // ldb % 128 == 0: an 8-column group is wholly in or out
#pragma unroll
      for (int pass = 0; pass < BM / 16; ++pass) {
        const int row_t = pass * 16 + tid / 32;
        const int64_t grow = tm.row0 + row_t;
        if (grow < tm.row_end)
          *reinterpret_cast<u32x4_t*>(static_cast<bf16_t*>(out) + grow * ldb + col) =
              *reinterpret_cast<const u32x4_t*>(yl + row_t * kYS + seg * 8);
      }
    }
  } else {
    // fp32 y straight from the registers, 16 bytes (4 adjacent columns) per lane
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t grow = tm.row0 + wm * WROWS + i * 32 + lane % 32;
      if (grow >= tm.row_end) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t col = static_cast<int64_t>(tm.nt) * kBN + wn * 64 + j * 32 + q * 8 + khalf * 4;
          if (col < ldb) {  // ldb % 128 == 0: a 4-column group is wholly in or out
            const f32x4_t w = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + grow * ldb + col) = w;
          }
        }
    }
  }
}

template <int BM, bool SWIGLU, bool OUT_F32>
hipError_t launch_fp8(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs, const int32_t* offsets,
                      int64_t rows, int E, int K, int ldb, int NT, void* out, float* out_scales,
                      hipStream_t stream, const int32_t* gather, const int* mx_flag, const float* row_scale) {
  constexpr int smem = F8Cfg<BM>::SMEM;
  auto kern = gemm_fp8_kernel<BM, SWIGLU, OUT_F32>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (attr != hipSuccess) return attr;
  const int64_t mt = max_tiles<BM>(rows, E, offsets == nullptr);
  const unsigned grid = SWIGLU ? grid_for_any(mt, NT, E, offsets == nullptr) : grid_for(mt, NT);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kGemmThreads), smem, stream, A, As, B, Bs, offsets, rows, E, K, ldb,
                     NT, out, out_scales, gather, row_scale, mx_flag);
  return hipGetLastError();
}

// Both variants of one GEMM; the device flag lets exactly one of them run.
template <bool SWIGLU, bool OUT_F32>
hipError_t launch_fp8_both(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs,
                           const int32_t* offsets, int64_t rows, int E, int K, int ldb, int NT_mx, int NT_gen,
                           void* out, float* out_scales, hipStream_t stream, const int32_t* gather,
                           const int* mx_flag, const float* row_scale = nullptr) {
  hipError_t err = launch_fp8<192, SWIGLU, OUT_F32>(A, As, B, Bs, offsets, rows, E, K, ldb, NT_mx, out, out_scales,
                                                    stream, gather, mx_flag, row_scale);
  if (err != hipSuccess) return err;
  return launch_fp8<128, SWIGLU, OUT_F32>(A, As, B, Bs, offsets, rows, E, K, ldb, NT_gen, out, out_scales, stream,
                                          gather, mx_flag, row_scale);
}

}  // namespace

size_t fp8_hidden_bytes(int64_t rows, int F) {
  return (static_cast<size_t>(rows) * F + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_grouped_swiglu_fp8(const void* x_perm, const float* x_scales, const int32_t* offsets,
                                     int64_t rows, int E, int H, int F, const void* w1, const float* w1_scales,
                                     const void* w2, const float* w2_scales, void* y_perm, int out_dt,
                                     void* scratch, hipStream_t stream, hipEvent_t between, const int32_t* gather,
                                     const float* row_scale) {
  uint8_t* hq = static_cast<uint8_t*>(scratch);
  float* hs = reinterpret_cast<float*>(static_cast<char*>(scratch) + fp8_hidden_bytes(rows, F));
  int* flag = reinterpret_cast<int*>(static_cast<char*>(scratch) + fp8_hidden_bytes(rows, F) +
                                     ((static_cast<size_t>(rows) * (F / 128) * 4 + 255) & ~static_cast<size_t>(255)));
  // Which variant: every block scale a power of two -> MX.  Rows gathered through `gather` come
  // from this library's own quantiser (power-of-two scales by construction); caller-supplied
  // activation scales are checked with the weights'.
  const int64_t n0 = gather ? 0 : rows * (H / 128);
  const int64_t n1 = static_cast<int64_t>(E) * (H / 128) * (2 * F / 128), n2 = static_cast<int64_t>(E) * (F / 128) * (H / 128);
  const int64_t nall = n0 + n1 + n2;
  hipLaunchKernelGGL(fp8_flag_clear_kernel, dim3(1), dim3(1), 0, stream, flag);
  const unsigned gc = static_cast<unsigned>(ceil_div(nall, 256) < 1024 ? ceil_div(nall, 256) : 1024);
  hipLaunchKernelGGL(fp8_scale_check_kernel, dim3(gc), dim3(256), 0, stream, x_scales, n0, w1_scales, n1,
                     w2_scales, n2, flag);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nt1 = F / 128, nt2 = static_cast<int>(ceil_div(H, kBN));
  err = launch_fp8_both<true, false>(static_cast<const uint8_t*>(x_perm), x_scales, static_cast<const uint8_t*>(w1),
                                     w1_scales, offsets, rows, E, H, 2 * F, nt1, nt1, hq, hs, stream, gather, flag,
                                     row_scale);
  if (err != hipSuccess) return err;
  if (between && (err = hipEventRecord(between, stream)) != hipSuccess) return err;
  if (out_dt == 0)
    return launch_fp8_both<false, true>(hq, hs, static_cast<const uint8_t*>(w2), w2_scales, offsets, rows, E, F, H,
                                        nt2, nt2, y_perm, nullptr, stream, nullptr, flag);
  return launch_fp8_both<false, false>(hq, hs, static_cast<const uint8_t*>(w2), w2_scales, offsets, rows, E, F, H,
                                       nt2, nt2, y_perm, nullptr, stream, nullptr, flag);
}

}  // namespace moe
