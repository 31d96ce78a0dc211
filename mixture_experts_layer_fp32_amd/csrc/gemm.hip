// gemm.hip -- Compute stage: every local SwiGLU expert in one grouped GEMM launch per matrix.
//
// "Scalable Training of Mixture-of-Experts Models with Megatron Core", summary page, "Method",
// first paragraph: the experts run as one grouped GEMM over the permuted rows, so all local
// experts execute in a single call.  Per expert e and row p of e:
//     u = x_perm[p] . W1[e]   (W1 [E, H, 2F], columns [0, F) gate, [F, 2F) up)
//     h = SiLU(gate) * up     (fused into the first GEMM's epilogue)
//     y_perm[p] = h . W2[e]   (W2 [E, F, H])
//
// Sync-free ragged scheduling: the per-expert row counts live only in device memory
// (expert_offsets).  The host launches a grid sized by the bound
//     sum_e ceil(M_e / BM) <= floor((rows + E * (BM - 1)) / BM)
// and every workgroup rebuilds the per-expert m-tile prefix from the offsets in LDS, maps its
// (XCD-remapped) linear id to (expert, m-tile, n-tile), and exits if it has none.  With skewed
// expert loads the SwiGLU GEMM instead gives every XCD an equal share of every expert's tiles
// (gemm_common.hpp: map_tile_auto).
//
// bf16 kernel (gfx950): 512 threads = 8 waves, tile BM x 256 x 64, v_mfma_f32_32x32x16_bf16,
// operands streamed global -> LDS by direct loads into a ring of LDS stages (details at the
// kernel).  In SwiGLU mode a tile's 256 columns are 128 gate columns and the matching 128 up
// columns, placed so a lane holds gate and up of the same (row, column) in the same
// accumulator slot.  fp32 kernel: 64 x 64 tiles on v_mfma_f32_32x32x2_f32.  The e4m3 kernels
// are in gemm_fp8.hip.
#include "gemm_common.hpp"

namespace moe {
namespace {

using namespace gemm;

constexpr int kThreads = 256;  // fp32 path


// ------------------------------------------------------------------------------ bf16 path
// A: [rows, K] bf16 row-major (x_perm or h).  B: per expert [K, N] bf16 (N-contiguous, the
// layout the weights arrive in), or with BNK per expert [N, K] (K-contiguous: the transposed
// weight products of the backward, dh' = dy W2^T and dx_perm = du W1^T, read W2 and W1 as stored).
// SWIGLU: out h [rows, F] (F = N / 2), tile n covers gate cols n*128.. and up cols F + n*128..
// else:   out [rows, N], tile n covers cols n*256..
//
// Tile BM x 256 x 64 per iteration, 512 threads = 8 waves (2 per SIMD) in a 2 (M) x 4 (N) grid,
// each wave (BM/2) x 64 = FM x 2 blocks of v_mfma_f32_32x32x16_bf16 with fp32 accumulators.
// Both operands stream global -> LDS directly (global_load_lds_dwordx4: lane l of a
// wave-instruction lands at base + 16 l), so there is no register staging and no VALU work in
// the loop.  A ring of NA LDS stages for A and one of NB stages for B:
//   A stage: BM rows x 128 B; 16-byte chunk c of row r is stored at c ^ ((r >> 1) & 7).
//   B stage: 64 k-rows x 512 B, untransposed; chunk c of k-row k at c ^ 4 (k & 3).
// The weights (B) stream from HBM and get the deeper ring; the activation rows (A) are shared
// by all N tiles of an expert and mostly hit in L2.
// A fragments (lane l: row l % 32, k 8 (l / 32) .. +8) are one ds_read_b128 each.  B fragments
// are two ds_read_b64_tr_b16 each: within a group of 16 lanes, lane 16g + 4a + b receives
// 16-bit column b of the 8-byte pieces addressed by lanes 16g + a + 4e (e = 0..3), so source
// lane s addresses k-row 8 (s / 32) + 4 r + (s % 16) / 4 at column 16 ((s / 16) % 2) +
// 4 (s % 4) of the fragment and destination lane d collects column d % 32 for 4 consecutive k.
// The swizzles spread every fragment read of a 16-lane group over distinct banks.
// MODE kModeNT: B is [N, K]; a B stage is BN rows (columns n) x 128 B laid out, loaded and read
// exactly like an A stage (chunk c of row n at c ^ ((n >> 1) & 7), one ds_read_b128 per fragment).
// MODE kModeBatchK: independent per-expert GEMMs out_e [M, N] = A_e [M, K_e] . B_e [K_e, N] (the
// weight gradients of the backward) with a contraction of its own per expert, padded to a multiple
// of 64; `offsets` points at 2 (E + 1) ints: the padded contraction prefix P (A_e is columns
// [P_e, P_{e+1}) of A, whose row stride is the K argument; its padding columns hold zeros) and
// then the first B row of every expert (B_e is rows offsets[E + 1 + e] .. + P_{e+1} - P_e of B;
// the rows past the expert's own meet A's zero columns).  `rows` is M; out_e starts at e M N.
//
// Iteration kt (four 16-deep k-steps): each MFMA of k-step s is followed by one LDS read of the
// fragments of k-step s + 1 (in the order the MFMAs consume them) and, in some slots, one direct
// load.  Before the last k-step the wave waits for its own reads of tile kt and its own loads of
// tile kt + 1 and meets the other waves at the single barrier of the iteration; the last k-step
// then reads tile kt + 1's first fragments, so the MFMA pipe restarts right after the barrier,
// and in its last slots loads A tile kt + NA into the stage tile kt used.  The loads of B tile
// kt + NB follow in k-steps 1 and 2 of iteration kt + 1 -- or, with two B stages (320-row tiles,
// whose two 40 KB A stages leave room for only two), right after the A loads.  Loads go out
// after the reads and away from the barrier: a direct load issued ahead of a wave's LDS reads
// delays them (measured: the GEMMs ran 6-9% slower with each load issued right after the
// barrier, before its read).  A loads have most of an iteration to land, B loads more than
// NB - 2 (with two stages, most of one).
// Loads are unconditional: rows past the expert's end re-read its last row and column groups
// past the matrix edge re-read column 0; those results are never stored.
constexpr int kBKT = 64;        // K per iteration / stage
constexpr int kBRow = kBN * 2;  // bytes per [K, N] B k-row

template <int BM>
struct Bf16Rings {
  // LDS: 2 x 40 + 2 x 32 KB (BM 320), 2 x 32 + 3 x 32 KB (BM 256), 3 x 16 + 3 x 32 KB (BM 128)
  static constexpr int NA = BM >= 256 ? 2 : 3;
  static constexpr int NB = BM == 320 ? 2 : 3;
  // Where the loads of B tile j + NB go out: 0 = k-steps 1 and 2 of iteration j + 1, 2 = the last
  // k-step of iteration j, after its A loads: the earliest slot a two-stage B ring allows (the
  // latest, k-steps 1 and 2, made the DeepSeek-V3-shaped GEMM1 6% slower; B loads ahead of the A
  // loads in that k-step 3% slower; the A loads moved to k-step 0 of the next iteration: equal).
  static constexpr int B_PLACE = NB == 2 ? 2 : 0;
  static constexpr int A_BYTES = BM * kBKT * 2;
  static constexpr int B_BYTES = kBN * kBKT * 2;
  static constexpr int SMEM = NA * A_BYTES + NB * B_BYTES;
};

template <int BM, int WM, bool SWIGLU, bool OUT_F32, int S, int MODE = kModeNN>
__global__ __launch_bounds__(256 * WM) void gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, const int32_t* __restrict__ offsets,
    int64_t rows, int E, int K, int ldb, int NT, void* __restrict__ out, int ncu,
    const int32_t* __restrict__ gather, int ksplit, const float* __restrict__ row_scale) {
  using R = Bf16Rings<BM>;
  constexpr int NA = R::NA, NB = R::NB;
  constexpr int NWAVE = 4 * WM;                // WM along M x 4 along N
  constexpr int WROWS = BM / WM;               // rows per wave
  constexpr int FM = WROWS / 32;               // 32x32 blocks per wave along M
  constexpr int FN = 2;                        // 32x32 blocks per wave along N (64 columns)
  constexpr int A_BYTES = R::A_BYTES;
  constexpr int B_BYTES = R::B_BYTES;
  constexpr int B_RING = NA * A_BYTES;              // byte offset of the B ring
  constexpr int A_ROUNDS = A_BYTES / 1024 / NWAVE;  // 1 KB wave-instructions per wave per stage
  constexpr int B_ROUNDS = B_BYTES / 1024 / NWAVE;
  constexpr int RPT = A_ROUNDS + B_ROUNDS;
  static_assert(NA >= 2 && NB >= NA, "ring depths");
  static_assert(R::B_PLACE == 0 || NA == NB, "B loads beside the A loads: equal ring depths");
  static_assert(kMaxExpertsLds * 4 <= B_BYTES, "tile-map prefix fits in the first B stage");
  static_assert(MODE != kModeBatchK || (OUT_F32 && !SWIGLU && S == 1), "batched mode: plain fp32 out");
  constexpr bool BNK = MODE == kModeNT;

  extern __shared__ __attribute__((aligned(1024))) char smem[];
  // The per-expert m-tile prefix of the tile map lives in the first B stage until the first loads.
  TileMap tm;
  // skewed loads: SwiGLU GEMMs spread every expert over the XCDs (measured: the second GEMM,
  // whose activation rows are as large as its weights, runs better on the contiguous map)
  int* s_pref = reinterpret_cast<int*>(smem + B_RING);
  if constexpr (MODE == kModeBatchK) {
    if (!map_tile_batched<BM>(rows, E, NT, tm)) return;
  } else {
    if (SWIGLU ? !map_tile_auto<BM>(offsets, rows, E, NT, s_pref, tm, ncu, S)
               : !map_tile<BM>(offsets, rows, E, NT, s_pref, tm, ncu, S))
      return;
  }
  __syncthreads();
  // Split K (one dense matrix, fp32 out): n-tile index ks * NT / ksplit + n covers n-tile n over
  // the ks-th 1/ksplit of K and writes its partial product to out + ks * rows * ldb.
  int nk = K / kBKT;
  int64_t k_first = 0;  // first K element of this tile
  if (ksplit > 1) {
    const int ntr = NT / ksplit;
    const int ks = tm.nt / ntr;
    tm.nt -= ks * ntr;
    nk /= ksplit;
    k_first = static_cast<int64_t>(ks) * nk * kBKT;
    out = static_cast<float*>(out) + static_cast<int64_t>(ks) * rows * ldb;
  }
  int64_t a_col0 = 0, b_row0 = static_cast<int64_t>(tm.expert) * K;  // batched: A column, B row of the expert
  if constexpr (MODE == kModeBatchK) {
    const int64_t p0 = offsets[tm.expert], p1 = offsets[tm.expert + 1];
    nk = static_cast<int>((p1 - p0) / kBKT);
    a_col0 = p0;
    b_row0 = offsets[E + 1 + tm.expert];
  }

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 4, wn = wave % 4;
  lds_void_t* lds = (lds_void_t*)smem;  // address-space cast: generic -> LDS
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));

  // ---- global sources of this lane's direct loads
  // A round p of wave w covers tile rows (8p + w) * 8 + lane / 8 (1 KB = 8 rows x 128 B);
  // stored chunk lane % 8 holds logical chunk (lane % 8) ^ ((row >> 1) & 7).
  const bf16_t* a_src[A_ROUNDS];
#pragma unroll
  for (int p = 0; p < A_ROUNDS; ++p) {
    const int r = (NWAVE * p + wave) * 8 + lane / 8;
    int64_t grow = tm.row0 + r;
    if (grow >= tm.row_end) grow = tm.row_end - 1;
    if constexpr (MODE == kModeBatchK) {
      grow -= static_cast<int64_t>(tm.expert) * rows;  // row of A_e
    } else {
      if (gather) grow = gather[grow];  // fused dispatch: row p of the tile is token gather[p]
    }
    a_src[p] = A + grow * K + a_col0 + k_first + (((lane % 8) ^ ((r >> 1) & 7)) * 8);
  }
  // A rounds wholly past the tile's last live 32-row block carry rows no fragment read uses (each
  // wave computes only its live blocks), so they are not loaded: the load path into LDS, busy most
  // of the time under these GEMMs, costs per instruction.  The waits below count the skipped loads.
  uint32_t a_dead = 0;
  {
    const int64_t live = tm.row_end - tm.row0 < BM ? tm.row_end - tm.row0 : BM;
    const int used = static_cast<int>((live + 31) / 32 * 32);
#pragma unroll
    for (int p = 0; p < A_ROUNDS; ++p)
      if ((NWAVE * p + wave) * 8 >= used) a_dead |= 1u << p;
  }
  a_dead = __builtin_amdgcn_readfirstlane(a_dead);
  const int n_dead = __builtin_popcount(a_dead);  // A loads this wave skips per A tile
  // B round p of wave w covers k-rows 2 (8p + w) + lane / 32 (1 KB = 2 k-rows x 512 B); stored
  // chunk lane % 32 holds logical chunk (lane % 32) ^ 4 ((2w + lane / 32) & 3).
  // BNK: round p of wave w covers B rows (columns) (8p + w) * 8 + lane / 8, as for A.
  const bf16_t* b_src = nullptr;
  const bf16_t* b_nk[BNK ? B_ROUNDS : 1];
  if constexpr (BNK) {
#pragma unroll
    for (int p = 0; p < B_ROUNDS; ++p) {
      const int r = (NWAVE * p + wave) * 8 + lane / 8;
      int64_t n = SWIGLU ? (r < 128 ? static_cast<int64_t>(tm.nt) * 128 + r
                                    : ldb / 2 + static_cast<int64_t>(tm.nt) * 128 + (r - 128))
                         : static_cast<int64_t>(tm.nt) * kBN + r;
      if (n >= ldb) n = 0;  // columns past the matrix edge re-read column 0 (never stored)
      b_nk[p] = B + (static_cast<int64_t>(tm.expert) * ldb + n) * K + k_first + (((lane % 8) ^ ((r >> 1) & 7)) * 8);
    }
  } else {
    const int b_lchunk = (lane % 32) ^ (4 * ((2 * wave + lane / 32) & 3));
    int64_t b_col;
    if (SWIGLU) {
      const int F = ldb / 2;
      b_col = (b_lchunk < 16) ? static_cast<int64_t>(tm.nt) * 128 + b_lchunk * 8
                              : F + static_cast<int64_t>(tm.nt) * 128 + (b_lchunk - 16) * 8;
    } else {
      b_col = static_cast<int64_t>(tm.nt) * kBN + b_lchunk * 8;
    }
    if (b_col >= ldb) b_col = 0;  // ldb % 8 == 0: an 8-column group is wholly in or out
    b_src = B + b_row0 * ldb + (k_first + 2 * wave + lane / 32) * ldb + b_col;
  }
  const int64_t b_round = static_cast<int64_t>(2 * NWAVE) * ldb;
  const int64_t b_kstep = static_cast<int64_t>(kBKT) * ldb;

  auto a_stage = [&](int kt) { return lds_base + static_cast<uint32_t>(kt % NA) * A_BYTES; };
  auto b_stage = [&](int kt) { return lds_base + B_RING + static_cast<uint32_t>(kt % NB) * B_BYTES; };
  // Load group j (j >= -NB): A tile j + NA and B tile j + NB, each if it exists.  The prologue
  // issues groups -NB .. -1 whole with this; in the loop the A part of group j goes out in
  // iteration j and its B part in iteration j + 1 (the k-step slots below).
  auto issue_group = [&](int j) {
    const int ta = j + NA, tb = j + NB;
    if (ta >= 0 && ta < nk) {
      const uint32_t abase = a_stage(ta);
#pragma unroll
      for (int p = 0; p < A_ROUNDS; ++p)
        if (!((a_dead >> p) & 1u))
          lds_dma16(a_src[p] + static_cast<int64_t>(ta) * kBKT, abase + (NWAVE * p + wave) * 1024);
    }
    if (tb < nk) {
      const uint32_t bbase = b_stage(tb);
      const bf16_t* bs = b_src + static_cast<int64_t>(tb) * b_kstep;
#pragma unroll
      for (int p = 0; p < B_ROUNDS; ++p) {
        if constexpr (BNK)
          lds_dma16(b_nk[p] + static_cast<int64_t>(tb) * kBKT, bbase + (NWAVE * p + wave) * 1024);
        else
          lds_dma16(bs + p * b_round, bbase + (NWAVE * p + wave) * 1024);
      }
    }
  };
  // Loads issued after both A and B tile t + 1 by the time iteration t waits (load group j: A
  // tile j + NA at the end of iteration j, B tile j + NB at the start of iteration j + 1), when
  // every tile they name exists (t + NB <= nk): B tile t + 2 when NB > NA (its A partner came
  // earlier), then NA - 2 whole groups, each n_dead A loads short.  Otherwise wait for all.
  constexpr int B_AFTER_A = NB > NA ? B_ROUNDS : 0;
  auto wait_tile_next = [&](int t) {
    if (t + NB <= nk) wait_vmcnt_less<B_AFTER_A + (NA - 2) * RPT, NA - 2, A_ROUNDS>(n_dead);
    else wait_vmcnt<0>();
  };

  // ---- fragment addresses (byte offsets inside a stage; k-step ks adds 32 B (A) or 16 k-rows (B))
  uint32_t a_row_off[FM], a_sw[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = wm * WROWS + i * 32 + lane % 32;
    a_row_off[i] = r * 128;
    a_sw[i] = (r >> 1) & 7;
  }
  uint32_t b_off[BNK ? 1 : FN][2];
  uint32_t b_row_off[BNK ? FN : 1], b_sw[BNK ? FN : 1];
  if constexpr (BNK) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = (SWIGLU ? j * 128 + wn * 32 : wn * 64 + j * 32) + lane % 32;
      b_row_off[j] = r * 128;
      b_sw[j] = (r >> 1) & 7;
    }
  } else {
    const int g = lane / 16, h = lane / 32, a4 = lane % 4, e = (lane % 16) / 4;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      // SwiGLU: block 0 = gate columns wn*32.., block 1 = the matching up columns 128 + wn*32..
      const int cb = SWIGLU ? j * 128 + wn * 32 : wn * 64 + j * 32;
      const int col = cb + 16 * (g % 2) + 4 * a4;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int krow = 8 * h + 4 * r + e;
        b_off[j][r] = krow * kBRow + (((col / 8) ^ (4 * e)) << 4) + (col % 8) * 2;
      }
    }
  }
  const int khalf = lane / 32;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Only the 32-row blocks of this wave that hold rows of the expert are computed: NL of the
  // wave's FM blocks (a wave-uniform count; the last m-tile of an expert is usually partial).
  int nl_rows = static_cast<int>((tm.row_end - tm.row0 < BM ? tm.row_end - tm.row0 : BM)) - wm * WROWS;
  nl_rows = nl_rows < 0 ? 0 : nl_rows;
  const int nlive = __builtin_amdgcn_readfirstlane(nl_rows >= WROWS ? FM : (nl_rows + 31) / 32);

  auto run = [&](auto nl_c) {
    constexpr int NL = decltype(nl_c)::value;
    constexpr int NLA = NL > 0 ? NL : 1;
    bf16x8_t af[2][NLA], bfr[2][FN];
    auto read_b = [&](uint32_t bbase, int ks, int buf, int j) {
      if constexpr (BNK) {
        const uint32_t chunk = ks * 2 + khalf;
        bfr[buf][j] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(
            static_cast<uintptr_t>(bbase + b_row_off[j] + ((chunk ^ b_sw[j]) << 4)));
      } else {
        v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<lds_v4i16_t*>(static_cast<uintptr_t>(bbase + b_off[j][0] + ks * 16 * kBRow)));
        v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<lds_v4i16_t*>(static_cast<uintptr_t>(bbase + b_off[j][1] + ks * 16 * kBRow)));
        typedef short v8i16_t __attribute__((ext_vector_type(8)));
        v8i16_t both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        bfr[buf][j] = __builtin_bit_cast(bf16x8_t, both);
      }
    };
    auto read_a = [&](uint32_t abase, int ks, int buf, int i) {
      const uint32_t chunk = ks * 2 + khalf;
      af[buf][i] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(
          static_cast<uintptr_t>(abase + a_row_off[i] + ((chunk ^ a_sw[i]) << 4)));
    };
    // read unit q (B0, A0, B1, A1, A2, ...: the order the i-major MFMAs consume them) of k-step ks
    // of tile kt into buffer buf
    auto read_unit = [&](int kt, int ks, int buf, int q) {
      if constexpr (NL > 0) {
        if (q == 0) read_b(b_stage(kt), ks, buf, 0);
        else if (q == 1) read_a(a_stage(kt), ks, buf, 0);
        else if (q < 2 + FN - 1) read_b(b_stage(kt), ks, buf, q - 1);
        else if (q < NL + FN) read_a(a_stage(kt), ks, buf, q - FN);
      }
    };
    constexpr int NR = NL > 0 ? NL + FN : 0;  // read units per k-step
    static_assert(B_ROUNDS % 2 == 0, "B loads split over two k-steps");
    // k-step ks (0..2) of tile kt: MFMA q, fragment read q of k-step ks + 1, then, in k-steps 1
    // and 2, half of the loads of B tile kt - 1 + NB (the B part of load group kt - 1, into the
    // stage freed at the previous iteration's barrier)
    auto kstep = [&](auto ks_c, int kt) {
      constexpr int ks = decltype(ks_c)::value;
      constexpr int BL = (ks == 0 || R::B_PLACE != 0) ? 0 : B_ROUNDS / 2, B0 = ks == 2 ? B_ROUNDS / 2 : 0;
      constexpr int NQ = cmax(cmax(NL * FN, NR), BL);
      const int tb = kt - 1 + NB;
      const bool do_b = kt >= 1 && tb < nk;
      const uint32_t bbase = b_stage(tb);
      const bf16_t* bs = b_src + static_cast<int64_t>(tb) * b_kstep;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (q < NL * FN) {
          const int i = q / FN, j = q % FN;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ks % 2][j], af[ks % 2][i], acc[i][j], 0, 0, 0);
        }
        if (q < NR) read_unit(kt, ks + 1, (ks + 1) % 2, q);
        if (q < BL && do_b) {
          if constexpr (BNK)
            lds_dma16(b_nk[B0 + q] + static_cast<int64_t>(tb) * kBKT, bbase + (NWAVE * (B0 + q) + wave) * 1024);
          else
            lds_dma16(bs + (B0 + q) * b_round, bbase + (NWAVE * (B0 + q) + wave) * 1024);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    for (int j = -NB; j < 0; ++j) issue_group(j);
    // tile 0: groups -NA + 1 .. -1 (and B(NB - NA) when NB > NA) may still be in flight
    if (NB <= nk) wait_vmcnt_less<B_AFTER_A + (NA - 1) * RPT, NA - 1, A_ROUNDS>(n_dead); else wait_vmcnt<0>();
    lds_barrier();
#pragma unroll
    for (int q = 0; q < NR; ++q) read_unit(0, 0, 0, q);
    for (int kt = 0; kt < nk; ++kt) {
      kstep(std::integral_constant<int, 0>{}, kt);
      kstep(std::integral_constant<int, 1>{}, kt);
      kstep(std::integral_constant<int, 2>{}, kt);
      if (kt + 1 < nk) {
        wait_lgkm0();        // this wave's reads of tile kt are complete
        wait_tile_next(kt);  // this wave's loads of A and B tile kt + 1 have landed
        lds_barrier();       // ... for every wave: tile kt + 1 readable, tile kt's stages free
      }
      __builtin_amdgcn_sched_barrier(0);
      // last k-step: MFMA q, fragment read q of tile kt + 1 (restarting the MFMA pipe right after
      // the barrier), and in its last slots the loads of A tile kt + NA (the A part of load group
      // kt, into the stage tile kt just left)
      {
        const int ta = kt + NA, tb = kt + NB;
        const bool do_a = kt + 1 < nk && ta < nk;
        const bool do_b = R::B_PLACE == 2 && kt + 1 < nk && tb < nk;
        const uint32_t abase = a_stage(ta), bbase = b_stage(tb);
        const bf16_t* bs = b_src + static_cast<int64_t>(tb) * b_kstep;
        constexpr int BLL = R::B_PLACE == 2 ? B_ROUNDS : 0;  // B loads in this k-step
        constexpr int NQ = cmax(cmax(NL * FN, NR), A_ROUNDS + BLL);
        constexpr int AQ = NQ - A_ROUNDS - BLL;              // first slot with an A load
        constexpr int BQ = NQ - BLL;                         // first slot with a B load
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          if (q < NL * FN) {
            const int i = q / FN, j = q % FN;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[1][j], af[1][i], acc[i][j], 0, 0, 0);
          }
          // unconditional: past the last tile this reads a stale stage (in bounds, never used); a
          // branch here would make the compiler wait for these reads before the next MFMAs
          if (q < NR) read_unit(kt + 1, 0, 0, q);
          if (q >= AQ && q < BQ && do_a && !((a_dead >> (q - AQ)) & 1u))
            lds_dma16(a_src[q - AQ] + static_cast<int64_t>(ta) * kBKT, abase + (NWAVE * (q - AQ) + wave) * 1024);
          if (q >= BQ && do_b) {
            if constexpr (BNK)
              lds_dma16(b_nk[q - BQ] + static_cast<int64_t>(tb) * kBKT, bbase + (NWAVE * (q - BQ) + wave) * 1024);
            else
              lds_dma16(bs + (q - BQ) * b_round, bbase + (NWAVE * (q - BQ) + wave) * 1024);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  dispatch_live<FM>(nlive, run);

  // ---- epilogue.  The MFMAs take the weight fragment as their first operand, so each computes a
  //      transposed 32x32 block: slot r of lane l of acc[i][j] is the wave's row i * 32 + l % 32
  //      and column j * 32 + (r / 4) * 8 + (l / 32) * 4 + (r % 4) of block j, so every lane holds
  //      4 adjacent columns of one row per group of 4 slots.
  if constexpr (!OUT_F32) {
    // bf16 results (SwiGLU: h = SiLU(gate) * up) staged through LDS -- the operand rings are free
    // once every wave is past its last reads -- 4 adjacent columns (8 bytes) per lane and LDS
    // write, then stored 16 bytes (8 columns) per lane, whole tile rows per wave instruction.  The
    // whole tile is staged at once, or one wave row group (WROWS rows) at a time where it does not
    // fit (BM 320 without SwiGLU).  (With one column per lane -- the other operand order -- the
    // staging took one 2-byte LDS write per value: 9% of the DeepSeek-V3-shaped GEMM2.  Storing
    // the 8-byte pieces straight to global memory instead, 32 rows per instruction, was slower.)
    constexpr int NTH = NWAVE * kWave;
    constexpr int COLS = SWIGLU ? 128 : kBN;  // output columns of the tile
    constexpr int LS = COLS + 8;              // row stride in bf16 (rows 16-byte aligned)
    constexpr int GROUPS = BM * LS * 2 <= R::SMEM ? 1 : WM;
    constexpr int GROWS = BM / GROUPS;        // rows staged at once
    static_assert(GROWS * LS * 2 <= R::SMEM, "output staging fits in the operand rings");
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    wait_lgkm0();
    __syncthreads();
    bf16_t* st = reinterpret_cast<bf16_t*>(smem);
    constexpr int SEGS = COLS / 8, RPP = NTH / SEGS;  // lanes per row, rows per pass
    static_assert(GROWS % RPP == 0, "whole passes per staged group");
    const int seg = tid % SEGS;
    const int64_t ldo = SWIGLU ? ldb / 2 : ldb;
    const int64_t col = static_cast<int64_t>(tm.nt) * COLS + seg * 8;
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) {
      if (GROUPS == 1 || wm == g) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          if (i * 32 >= nl_rows) continue;  // no row of this block is live (wave-uniform)
          const int row_t = wm * WROWS + i * 32 + lane % 32;
          const int row_s = row_t - g * GROWS;  // row in the staging buffer
          float gate = 1.0f;  // gate folded into the expert: h scaled by the row's gate before rounding
          if (SWIGLU && row_scale != nullptr) {
            const int64_t gr = tm.row0 + row_t;
            gate = row_scale[gr < tm.row_end ? gr : tm.row_end - 1];
          }
          constexpr int NJ = SWIGLU ? 1 : FN;  // output column blocks (SwiGLU: gate 0 with up 1)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c = (SWIGLU ? wn * 32 : wn * 64 + j * 32) + q * 8 + khalf * 4;
              float v[4];
#pragma unroll
              for (int t = 0; t < 4; ++t)
                v[t] = SWIGLU ? silu_fast(acc[i][0][4 * q + t]) * acc[i][1][4 * q + t] * gate : acc[i][j][4 * q + t];
              const u32x2_t w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
              *reinterpret_cast<u32x2_t*>(st + row_s * LS + c) = w;
            }
        }
      }
      __syncthreads();
      if (col < ldo) {  // ldo % 8 == 0: an 8-column group is wholly in or out
#pragma unroll
        for (int pass = 0; pass < GROWS / RPP; ++pass) {
          const int row_s = pass * RPP + tid / SEGS;
          const int64_t grow = tm.row0 + g * GROWS + row_s;
          if (grow < tm.row_end)
            *reinterpret_cast<u32x4_t*>(static_cast<bf16_t*>(out) + grow * ldo + col) =
                *reinterpret_cast<const u32x4_t*>(st + row_s * LS + seg * 8);
        }
      }
      if (GROUPS > 1) __syncthreads();
    }
  } else if constexpr (SWIGLU) {
    // fp32 h straight from the registers, 16 bytes (4 adjacent columns) per lane
    const int64_t ldo = ldb / 2;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t grow = tm.row0 + wm * WROWS + i * 32 + lane % 32;
      if (grow >= tm.row_end) continue;
      const float gate = row_scale != nullptr ? row_scale[grow] : 1.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t c = static_cast<int64_t>(tm.nt) * 128 + wn * 32 + q * 8 + khalf * 4;
        f32x4_t w;
#pragma unroll
        for (int t = 0; t < 4; ++t) w[t] = silu_fast(acc[i][0][4 * q + t]) * acc[i][1][4 * q + t] * gate;
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + grow * ldo + c) = w;
      }
    }
  } else {
    // fp32 results staged through LDS one wave row group (WROWS rows) at a time -- or one 32-row
    // block of it where the group does not fit (BM 320) -- then written a whole row per wave
    // instruction (16 bytes per lane, the tile row's 256 columns contiguous): with one 4-byte store
    // per accumulator slot every instruction wrote 128-byte pieces of two rows, and the weight
    // gradients of the backward write gigabytes of fp32 this way.
    constexpr int LSF = kBN + 4;  // fp32 row stride: 16 consecutive rows start 4 banks apart
    constexpr int FMC = FM * 32 * LSF * 4 <= R::SMEM ? FM : 1;  // 32-row blocks staged at once
    constexpr int CROWS = FMC * 32;
    static_assert(CROWS * LSF * 4 <= R::SMEM, "one staged chunk of fp32 results fits in the rings");
    float* st = reinterpret_cast<float*>(smem);
    wait_lgkm0();
    __syncthreads();
#pragma unroll
    for (int gc = 0; gc < WM * (FM / FMC); ++gc) {
      const int g = gc / (FM / FMC), c = gc % (FM / FMC);  // wave row group, chunk of its blocks
      if (wm == g) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          if (i / FMC != c) continue;
          const int row_l = (i % FMC) * 32 + lane % 32;
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4_t w = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
              *reinterpret_cast<f32x4_t*>(st + row_l * LSF + wn * 64 + j * 32 + q * 8 + khalf * 4) = w;
            }
        }
      }
      __syncthreads();
      const int64_t col = static_cast<int64_t>(tm.nt) * kBN + lane * 4;
      for (int row_l = wave; row_l < CROWS; row_l += NWAVE) {
        const int64_t grow = tm.row0 + g * WROWS + c * CROWS + row_l;
        if (grow < tm.row_end && col < ldb) {  // ldb % 4 == 0: a 4-column group is wholly in or out
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(st + row_l * LSF + lane * 4);
          f32x4_t* dst = reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + grow * ldb + col);
          // the backward's products (weights read as stored, per-expert weight gradients: up to tens
          // of GB of fp32) stream past the caches (DeepSeek-V3-shaped dW1 10.6 -> 9.7 ms); the
          // router's partial products are read back at once and keep the cached store (route
          // 147 -> 158 us when streamed)
          if constexpr (MODE != kModeNN) __builtin_nontemporal_store(v, dst);
          else *dst = v;
        }
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------------------ fp32 path
// v_mfma_f32_32x32x2_f32: lane l holds A[l % 32][k = l / 32] and B[k = l / 32][l % 32].
// Tile 64 x 64 (SwiGLU: 32 gate + 32 matching up columns), K step 16, 4 waves in 2 x 2.
constexpr int kF32BM = 64, kF32BN = 64, kF32BK = 16;

template <bool SWIGLU>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(const float* __restrict__ A,
                                                           const float* __restrict__ B,
                                                           const int32_t* __restrict__ offsets,
                                                           int64_t rows, int E, int K, int ldb, int NT,
                                                           float* __restrict__ out,
                                                           const int32_t* __restrict__ gather,
                                                           const float* __restrict__ row_scale) {
  __shared__ float sa[kF32BM][kF32BK + 1];
  __shared__ float sb[kF32BK][kF32BN + 4];
  __shared__ int s_pref[kMaxExpertsLds];
  TileMap tm;
  if (!map_tile<kF32BM>(offsets, rows, E, NT, s_pref, tm)) return;

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;
  const float* Bexp = B + static_cast<int64_t>(tm.expert) * K * ldb;
  const int F = ldb / 2;

  f32x16_t acc = {};
  for (int k0 = 0; k0 < K; k0 += kF32BK) {
    for (int i = tid; i < kF32BM * kF32BK; i += kThreads) {
      int r = i / kF32BK, kk = i % kF32BK;
      int64_t grow = tm.row0 + r;
      sa[r][kk] = grow < tm.row_end ? A[(gather ? gather[grow] : grow) * K + k0 + kk] : 0.0f;
    }
    for (int i = tid; i < kF32BK * kF32BN; i += kThreads) {
      int kk = i / kF32BN, c = i % kF32BN;
      int64_t col;
      if (SWIGLU)
        col = (c < 32) ? static_cast<int64_t>(tm.nt) * 32 + c : F + static_cast<int64_t>(tm.nt) * 32 + (c - 32);
      else
        col = static_cast<int64_t>(tm.nt) * kF32BN + c;
      sb[kk][c] = col < ldb ? Bexp[static_cast<int64_t>(k0 + kk) * ldb + col] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kF32BK; ks += 2) {
      float a = sa[wm * 32 + lane % 32][ks + lane / 32];
      float b = sb[ks + lane / 32][wn * 32 + lane % 32];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  // SwiGLU: waves wn = 0 (gate) and wn = 1 (up) hold matching columns; exchange through LDS.
  if (SWIGLU) {
    __shared__ float s_up[2][16][kWave];
    if (wn == 1)
      for (int r = 0; r < 16; ++r) s_up[wm][r][lane] = acc[r];
    __syncthreads();
    if (wn == 0) {
      for (int r = 0; r < 16; ++r) {
        const int64_t grow = tm.row0 + wm * 32 + (r / 4) * 8 + (lane / 32) * 4 + (r % 4);
        if (grow >= tm.row_end) continue;
        float h = silu(acc[r]) * s_up[wm][r][lane];
        if (row_scale != nullptr) h *= row_scale[grow];
        out[grow * F + static_cast<int64_t>(tm.nt) * 32 + lane % 32] = h;
      }
    }
  } else {
    for (int r = 0; r < 16; ++r) {
      const int64_t grow = tm.row0 + wm * 32 + (r / 4) * 8 + (lane / 32) * 4 + (r % 4);
      const int64_t col = static_cast<int64_t>(tm.nt) * kF32BN + wn * 32 + lane % 32;
      if (grow >= tm.row_end || col >= ldb) continue;
      out[grow * ldb + col] = acc[r];
    }
  }
}

// Tail of the second GEMM.  Its tiles are K = F deep (16 times the first GEMM's for Mixtral-like
// shapes), and when their count leaves the last wave of workgroups mostly empty, each tile of
// that wave is cut into kBands row bands computed by separate workgroups (the band's dead
// 32-row blocks skip their MFMAs), so the last wave ends about kBands times sooner.
constexpr int kBands = 4;

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int BM, bool SWIGLU, bool OUT_F32, int WM = 2, int S = 1, int MODE = kModeNN>
hipError_t launch_bf16(const bf16_t* A, const bf16_t* B, const int32_t* offsets, int64_t rows, int E,
                       int K, int ldb, int NT, void* out, hipStream_t stream, int ncu = 0,
                       const int32_t* gather = nullptr, int ksplit = 1, const float* row_scale = nullptr) {
  constexpr int smem = Bf16Rings<BM>::SMEM;
  auto kern = gemm_bf16_kernel<BM, WM, SWIGLU, OUT_F32, S, MODE>;
  // once per instantiation (and never inside a stream capture after the first eager call)
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (attr != hipSuccess) return attr;
  const int64_t mt = MODE == kModeBatchK ? ceil_div(rows, BM) * E : max_tiles<BM>(rows, E, offsets == nullptr);
  const unsigned grid = MODE == kModeBatchK ? static_cast<unsigned>(8 * ceil_div(mt * NT, 8))
                        : SWIGLU            ? grid_for_any(mt, NT, E, offsets == nullptr, ncu, S)
                                            : grid_for(mt, NT, ncu, S);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256 * WM), smem, stream, A, B, offsets, rows, E, K, ldb, NT, out, ncu,
                     gather, ksplit, row_scale);
  return hipGetLastError();
}

// Second GEMM, with the banded tail when the device's CU count is known.
template <int BM, bool OUT_F32>
hipError_t launch_bf16_down(const bf16_t* h, const bf16_t* w2, const int32_t* offsets, int64_t rows, int E, int F,
                            int H, int nt2, void* y_perm, hipStream_t stream) {
  const int ncu = device_cus();
  if (ncu < 2) return launch_bf16<BM, false, OUT_F32>(h, w2, offsets, rows, E, F, H, nt2, y_perm, stream);
  return launch_bf16<BM, false, OUT_F32, 2, kBands>(h, w2, offsets, rows, E, F, H, nt2, y_perm, stream, ncu);
}

// GEMM1 (+SwiGLU) then GEMM2 with BM-row tiles; `between` (optional) is recorded after GEMM1.
template <int BM>
hipError_t launch_bf16_pair(const void* x_perm, const void* w1, const void* w2, const int32_t* offsets,
                            int64_t rows, int E, int H, int F, void* y_perm, int out_dt, void* scratch,
                            hipStream_t stream, hipEvent_t between, const int32_t* gather, const float* row_scale) {
  bf16_t* h = static_cast<bf16_t*>(scratch);
  hipError_t err = launch_bf16<BM, true, false>(static_cast<const bf16_t*>(x_perm), static_cast<const bf16_t*>(w1),
                                                offsets, rows, E, H, 2 * F, F / 128, h, stream, 0, gather, 1,
                                                row_scale);
  if (err != hipSuccess) return err;
  if (between && (err = hipEventRecord(between, stream)) != hipSuccess) return err;
  const int nt2 = static_cast<int>(ceil_div(H, kBN));
  if (out_dt == 0)
    return launch_bf16_down<BM, true>(h, static_cast<const bf16_t*>(w2), offsets, rows, E, F, H, nt2, y_perm, stream);
  return launch_bf16_down<BM, false>(h, static_cast<const bf16_t*>(w2), offsets, rows, E, F, H, nt2, y_perm, stream);
}

}  // namespace

size_t grouped_swiglu_scratch_bytes(int64_t rows, int F, int dt) {
  if (dt == 0) return static_cast<size_t>(rows) * F * 4;
  if (dt == 1) return static_cast<size_t>(rows) * F * 2;
  if (dt == 3) return fp4_hidden_bytes(rows, F);
  // fp8: h codes + their 1x128 scales + the kernel-variant flag
  return fp8_hidden_bytes(rows, F) + ((static_cast<size_t>(rows) * (F / 128) * 4 + 255) & ~static_cast<size_t>(255)) +
         256;
}

hipError_t launch_dense_gemm_f32out(const void* A, const void* B, int64_t rows, int K, int N, float* out,
                                    hipStream_t stream, int ksplit, int bm) {
  if (rows <= 0) return hipSuccess;
  if (ksplit < 1 || (K / kBKT) % ksplit != 0 || (bm != 128 && bm != 256)) return hipErrorInvalidValue;
  const int nt = static_cast<int>(ceil_div(N, kBN)) * ksplit;
  const bf16_t* a = static_cast<const bf16_t*>(A);
  const bf16_t* b = static_cast<const bf16_t*>(B);
  return bm == 256 ? launch_bf16<256, false, true>(a, b, nullptr, rows, 1, K, N, nt, out, stream, 0, nullptr, ksplit)
                   : launch_bf16<128, false, true>(a, b, nullptr, rows, 1, K, N, nt, out, stream, 0, nullptr, ksplit);
}

// Tile height of the grouped bf16 GEMMs for `rows` rows over E experts (dense: one expert, no
// offsets): 128-row tiles when experts average fewer than 192 rows; 320-row tiles when they average
// 232 to 304 rows, so that an expert of up to 320 rows (most of them, with the spread of a balanced
// router) streams each weight tile through LDS once instead of twice; else 256-row tiles (the last,
// partial m-tile of an expert only computes its live 32-row blocks).  DeepSeek-V3-shaped routing
// (211-304 rows per expert): forward GEMM1 4.31 -> 3.87 ms, GEMM2 2.42 -> 2.34 ms; with exactly 224
// rows per expert (one tile either way) the 256-row tiles and their three B stages are 5% faster,
// with exactly 288 rows the 320-row tiles 12%.
int grouped_tile_rows(int64_t rows, int E, bool dense) {
  const int64_t e = dense ? 1 : E;
  if (rows < 192 * e) return 128;
  return !dense && rows >= 232 * e && rows <= 304 * e ? 320 : 256;
}

template <bool OUT_F32, int MODE>
hipError_t launch_grouped_plain(const void* A, const void* B, const int32_t* offsets, int64_t rows, int E, int K,
                                int N, void* out, hipStream_t stream, const int32_t* gather) {
  if (rows <= 0) return hipSuccess;
  const int nt = static_cast<int>(ceil_div(N, kBN));
  const bf16_t* a = static_cast<const bf16_t*>(A);
  const bf16_t* b = static_cast<const bf16_t*>(B);
  switch (grouped_tile_rows(rows, E, offsets == nullptr)) {
    case 320: return launch_bf16<320, false, OUT_F32, 2, 1, MODE>(a, b, offsets, rows, E, K, N, nt, out, stream, 0, gather);
    case 256: return launch_bf16<256, false, OUT_F32, 2, 1, MODE>(a, b, offsets, rows, E, K, N, nt, out, stream, 0, gather);
    default: return launch_bf16<128, false, OUT_F32, 2, 1, MODE>(a, b, offsets, rows, E, K, N, nt, out, stream, 0, gather);
  }
}

hipError_t launch_grouped_gemm_f32out(const void* A, const void* B, const int32_t* offsets, int64_t rows, int E,
                                      int K, int N, float* out, hipStream_t stream, const int32_t* gather) {
  return launch_grouped_plain<true, kModeNN>(A, B, offsets, rows, E, K, N, out, stream, gather);
}

hipError_t launch_grouped_gemm_nt_f32out(const void* A, const void* B, const int32_t* offsets, int64_t rows, int E,
                                         int K, int N, float* out, hipStream_t stream, const int32_t* gather) {
  return launch_grouped_plain<true, kModeNT>(A, B, offsets, rows, E, K, N, out, stream, gather);
}

hipError_t launch_grouped_gemm_nt_bf16out(const void* A, const void* B, const int32_t* offsets, int64_t rows, int E,
                                          int K, int N, void* out, hipStream_t stream, const int32_t* gather) {
  return launch_grouped_plain<false, kModeNT>(A, B, offsets, rows, E, K, N, out, stream, gather);
}

hipError_t launch_batched_gemm_f32out(const void* A, int64_t lda, const void* B, const int32_t* kinfo, int E, int M,
                                      int N, float* out, hipStream_t stream) {
  if (E <= 0 || M <= 0 || N <= 0) return hipSuccess;
  if (lda % 8 != 0 || N % 8 != 0 || lda > INT32_MAX) return hipErrorInvalidValue;
  const int nt = static_cast<int>(ceil_div(N, kBN));
  const bf16_t* a = static_cast<const bf16_t*>(A);
  const bf16_t* b = static_cast<const bf16_t*>(B);
  const int K = static_cast<int>(lda);
  return M >= 256 ? launch_bf16<256, false, true, 2, 1, kModeBatchK>(a, b, kinfo, M, E, K, N, nt, out, stream)
                  : launch_bf16<128, false, true, 2, 1, kModeBatchK>(a, b, kinfo, M, E, K, N, nt, out, stream);
}

hipError_t launch_grouped_swiglu(const void* x_perm, const void* x_scales, int dt,
                                 const int32_t* offsets, int64_t rows, int E, int H, int F,
                                 const void* w1, const void* w1_scales, const void* w2,
                                 const void* w2_scales, void* y_perm, int out_dt, void* scratch,
                                 hipStream_t stream, hipEvent_t between, const int32_t* gather,
                                 const float* row_scale) {
  if (dt == 2)
    return launch_grouped_swiglu_fp8(x_perm, static_cast<const float*>(x_scales), offsets, rows, E, H, F, w1,
                                     static_cast<const float*>(w1_scales), w2, static_cast<const float*>(w2_scales),
                                     y_perm, out_dt, scratch, stream, between, gather, row_scale);
  if (dt == 3)
    return launch_grouped_swiglu_fp4(x_perm, x_scales, offsets, rows, E, H, F, w1, w1_scales, w2, w2_scales, y_perm,
                                     out_dt, scratch, stream, between, gather, row_scale);
  if (dt == 0) {
    float* h = static_cast<float*>(scratch);
    const int nt1 = F / 32, nt2 = static_cast<int>(ceil_div(H, kF32BN));
    const unsigned g1 = grid_for(max_tiles<kF32BM>(rows, E, offsets == nullptr), nt1);
    hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(g1), dim3(kThreads), 0, stream,
                       static_cast<const float*>(x_perm), static_cast<const float*>(w1), offsets, rows, E,
                       H, 2 * F, nt1, h, gather, row_scale);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (between && (err = hipEventRecord(between, stream)) != hipSuccess) return err;
    const unsigned g2 = grid_for(max_tiles<kF32BM>(rows, E, offsets == nullptr), nt2);
    hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(g2), dim3(kThreads), 0, stream, h,
                       static_cast<const float*>(w2), offsets, rows, E, F, H, nt2,
                       static_cast<float*>(y_perm), static_cast<const int32_t*>(nullptr),
                       static_cast<const float*>(nullptr));
    return hipGetLastError();
  }
  if (dt == 1) {
    switch (grouped_tile_rows(rows, E, offsets == nullptr)) {
      case 320:
        return launch_bf16_pair<320>(x_perm, w1, w2, offsets, rows, E, H, F, y_perm, out_dt, scratch, stream,
                                     between, gather, row_scale);
      case 256:
        return launch_bf16_pair<256>(x_perm, w1, w2, offsets, rows, E, H, F, y_perm, out_dt, scratch, stream,
                                     between, gather, row_scale);
      default:
        return launch_bf16_pair<128>(x_perm, w1, w2, offsets, rows, E, H, F, y_perm, out_dt, scratch, stream,
                                     between, gather, row_scale);
    }
  }
  return hipErrorNotSupported;
}

}  // namespace moe
