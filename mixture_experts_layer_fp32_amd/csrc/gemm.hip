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
// (XCD-remapped) linear id to (expert, m-tile, n-tile), and exits if it has none.
//
// bf16 kernel (gfx950): 256 threads = 4 waves in a 2 x 2 grid, tile BM x 256 x 64, MFMA
// v_mfma_f32_32x32x16_bf16.  Both LDS tiles are stored K-contiguous (row-major A as loaded;
// the N-contiguous weight tile transposed in registers, 8 x 8 bf16 per thread, before the LDS
// store), with a 16-byte-chunk XOR swizzle so the 16-byte fragment reads and the transposed
// stores avoid bank conflicts.  Double-buffered LDS, one barrier per K step, next K tile
// prefetched into registers during the MFMAs.  In SwiGLU mode a tile's 256 columns are 128
// gate columns and the matching 128 up columns, placed so a lane holds gate and up of the
// same (row, column) in the same accumulator slot.
#include "gemm_common.hpp"

namespace moe {
namespace {

using namespace gemm;

constexpr int kThreads = 256;  // fp32 path


// ------------------------------------------------------------------------------ bf16 path
// A: [rows, K] bf16 row-major (x_perm or h).  B: per expert [K, N] bf16 (N-contiguous, the
// layout the weights arrive in) or, with B_NK, [N, K] (K-contiguous).
// SWIGLU: out h [rows, F] (F = N / 2), tile n covers gate cols n*128.. and up cols F + n*128..
// else:   out [rows, N], tile n covers cols n*256..
//
// Tile BM x 256 x 64 per iteration, 512 threads = 8 waves (2 per SIMD) in a 2 (M) x 4 (N) grid,
// each wave (BM/2) x 64 = FM x 2 blocks of v_mfma_f32_32x32x16_bf16 with fp32 accumulators.
// Both operands stream global -> LDS directly (global_load_lds_dwordx4: lane l of a
// wave-instruction lands at base + 16 l), so there is no register staging and no VALU work in
// the loop.  Two LDS stages per operand (128 KB):
//   A stage: BM rows x 128 B; 16-byte chunk c of row r is stored at c ^ ((r >> 1) & 7).
//   B stage, [K, N] weights: 64 k-rows x 512 B, untransposed; chunk c of k-row k at c ^ 4 (k & 3).
//   B stage, [N, K] weights: like A (256 n-rows x 128 B).
// A fragments (lane l: row l % 32, k 8 (l / 32) .. +8) are one ds_read_b128 each.  B fragments
// from [K, N] are two ds_read_b64_tr_b16 each: within a group of 16 lanes, lane 16g + 4a + b
// receives 16-bit column b of the 8-byte pieces addressed by lanes 16g + a + 4e (e = 0..3), so
// source lane s addresses k-row 8 (s / 32) + 4 r + (s % 16) / 4 at column 16 ((s / 16) % 2) +
// 4 (s % 4) of the fragment and destination lane d collects column d % 32 for 4 consecutive k.
// The swizzles spread every fragment read of a 16-lane group over distinct banks.
//
// Iteration kt (four 16-deep k-steps): MFMAs of k-step s interleave with the LDS reads of the
// fragments of k-step s + 1.  Before the last k-step the wave waits for its own reads of tile
// kt and its own loads of tile kt + 1, meets the other waves at the single barrier of the
// iteration, issues the loads of tile kt + 2 into tile kt's stages, and then runs the last
// k-step while reading tile kt + 1's first fragments.
// Loads are unconditional: rows past the expert's end re-read its last row and column groups
// past the matrix edge re-read column 0; those results are never stored.
constexpr int kBKT = 64;        // K per iteration / stage
constexpr int kBRow = kBN * 2;  // bytes per [K, N] B k-row

template <int BM, bool SWIGLU, bool OUT_F32, bool B_NK>
__global__ __launch_bounds__(kGemmThreads) void gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, const int32_t* __restrict__ offsets,
    int64_t rows, int E, int K, int ldb, int NT, void* __restrict__ out) {
  constexpr int NWAVE = kGemmThreads / kWave;  // 8: 2 along M x 4 along N
  constexpr int FM = BM / 64;                  // 32x32 blocks per wave along M
  constexpr int FN = 2;                        // 32x32 blocks per wave along N (64 columns)
  constexpr int A_BYTES = BM * kBKT * 2;
  constexpr int B_BYTES = kBN * kBKT * 2;
  constexpr int B_BASE = 2 * A_BYTES;               // byte offset of the two B stages
  constexpr int A_ROUNDS = A_BYTES / 1024 / NWAVE;  // 1 KB wave-instructions per wave per stage
  constexpr int B_ROUNDS = B_BYTES / 1024 / NWAVE;

  extern __shared__ __attribute__((aligned(1024))) char smem[];
  __shared__ int s_pref[kMaxExpertsLds];

  TileMap tm;
  if (!map_tile<BM>(offsets, rows, E, NT, s_pref, tm)) return;

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
    a_src[p] = A + grow * K + (((lane % 8) ^ ((r >> 1) & 7)) * 8);
  }
  // B sources.  [K, N]: round p of wave w covers k-rows 2 (8p + w) + lane / 32 (1 KB = 2 k-rows
  // x 512 B); stored chunk lane % 32 holds logical chunk (lane % 32) ^ 4 ((2w + lane / 32) & 3).
  // [N, K]: round p covers n-rows (8p + w) * 8 + lane / 8, swizzled like A.
  const bf16_t* b_src[B_ROUNDS];
  int64_t b_kstep;
  if (!B_NK) {
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
    const bf16_t* b0 = B + static_cast<int64_t>(tm.expert) * K * ldb +
                       static_cast<int64_t>(2 * wave + lane / 32) * ldb + b_col;
#pragma unroll
    for (int p = 0; p < B_ROUNDS; ++p) b_src[p] = b0 + static_cast<int64_t>(2 * NWAVE * p) * ldb;
    b_kstep = static_cast<int64_t>(kBKT) * ldb;
  } else {
#pragma unroll
    for (int p = 0; p < B_ROUNDS; ++p) {
      const int r = (NWAVE * p + wave) * 8 + lane / 8;
      int64_t n;
      if (SWIGLU) {
        const int F = ldb / 2;
        n = (r < 128) ? static_cast<int64_t>(tm.nt) * 128 + r : F + static_cast<int64_t>(tm.nt) * 128 + (r - 128);
      } else {
        n = static_cast<int64_t>(tm.nt) * kBN + r;
      }
      if (n >= ldb) n = 0;
      b_src[p] = B + (static_cast<int64_t>(tm.expert) * ldb + n) * K + (((lane % 8) ^ ((r >> 1) & 7)) * 8);
    }
    b_kstep = kBKT;
  }

  auto issue_loads = [&](int kt) {
    const uint32_t abase = lds_base + (kt & 1) * A_BYTES;
    const uint32_t bbase = lds_base + B_BASE + (kt & 1) * B_BYTES;
#pragma unroll
    for (int p = 0; p < A_ROUNDS; ++p)
      lds_dma16(a_src[p] + static_cast<int64_t>(kt) * kBKT, abase + (NWAVE * p + wave) * 1024);
#pragma unroll
    for (int p = 0; p < B_ROUNDS; ++p)
      lds_dma16(b_src[p] + static_cast<int64_t>(kt) * b_kstep, bbase + (NWAVE * p + wave) * 1024);
  };

  // ---- fragment addresses (byte offsets inside a stage; k-step ks adds 32 B (A, [N,K] B) or
  // 16 k-rows ([K,N] B))
  uint32_t a_row_off[FM], a_sw[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = wm * (BM / 2) + i * 32 + lane % 32;
    a_row_off[i] = r * 128;
    a_sw[i] = (r >> 1) & 7;
  }
  uint32_t b_off[FN][2], b_sw[FN];
  if (B_NK) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int cb = SWIGLU ? j * 128 + wn * 32 : wn * 64 + j * 32;
      const int r = cb + lane % 32;
      b_off[j][0] = r * 128;
      b_off[j][1] = 0;
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
      b_sw[j] = 0;
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

  bf16x8_t af[2][FM], bfr[2][FN];
  auto read_frags = [&](int kt, int ks, int buf) {
    const uint32_t abase = lds_base + (kt & 1) * A_BYTES;
    const uint32_t bbase = lds_base + B_BASE + (kt & 1) * B_BYTES;
    const uint32_t chunk = ks * 2 + khalf;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      af[buf][i] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(
          static_cast<uintptr_t>(abase + a_row_off[i] + ((chunk ^ a_sw[i]) << 4)));
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if (B_NK) {
        bfr[buf][j] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(
            static_cast<uintptr_t>(bbase + b_off[j][0] + ((chunk ^ b_sw[j]) << 4)));
      } else {
        v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_v4i16_t*>(
            static_cast<uintptr_t>(bbase + b_off[j][0] + ks * 16 * kBRow)));
        v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_v4i16_t*>(
            static_cast<uintptr_t>(bbase + b_off[j][1] + ks * 16 * kBRow)));
        typedef short v8i16_t __attribute__((ext_vector_type(8)));
        v8i16_t both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        bfr[buf][j] = __builtin_bit_cast(bf16x8_t, both);
      }
    }
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bfr[buf][j], acc[i][j], 0, 0, 0);
  };
  // MFMAs of one k-step interleaved with the LDS reads of the next k-step's fragments
  constexpr int NREADS = FM + (B_NK ? FN : 2 * FN);
  constexpr int NMFMA = FM * FN;
  constexpr int RPM = (NREADS + NMFMA - 1) / NMFMA;  // LDS reads per MFMA slot
  auto interleave = [&]() { sched_mfma_reads<0, NMFMA, NREADS, RPM>(); };

  const int nk = K / kBKT;
  issue_loads(0);
  if (nk > 1) {
    issue_loads(1);
    wait_vmcnt<A_ROUNDS + B_ROUNDS>();  // tile 0 landed (tile 1 may be in flight)
  } else {
    wait_vmcnt<0>();
  }
  lds_barrier();
  read_frags(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    mfmas(0);
    read_frags(kt, 1, 1);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    mfmas(1);
    read_frags(kt, 2, 0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    mfmas(0);
    read_frags(kt, 3, 1);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) {
      wait_lgkm0();       // this wave's reads of tile kt are complete
      wait_vmcnt<0>();    // this wave's loads of tile kt + 1 have landed
      lds_barrier();      // ... for every wave: tile kt + 1 readable, tile kt's stages free
      if (kt + 2 < nk) issue_loads(kt + 2);
    }
    __builtin_amdgcn_sched_barrier(0);
    mfmas(1);
    read_frags(kt + 1, 0, 0);  // past the last tile this reads a stale stage (in bounds, unused)
    interleave();
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- epilogue.  32x32 accumulator layout: slot r of lane l is
  //      row (r / 4) * 8 + (l / 32) * 4 + (r % 4), column l % 32.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row_t = wm * (BM / 2) + i * 32 + (r / 4) * 8 + khalf * 4 + (r % 4);
      const int64_t grow = tm.row0 + row_t;
      if (grow >= tm.row_end) continue;
      if (SWIGLU) {
        const int F = ldb / 2;
        const float g = acc[i][0][r], u = acc[i][1][r];
        const float h = silu_fast(g) * u;
        const int64_t col = static_cast<int64_t>(tm.nt) * 128 + wn * 32 + lane % 32;
        if (OUT_F32)
          static_cast<float*>(out)[grow * F + col] = h;
        else
          static_cast<bf16_t*>(out)[grow * F + col] = f32_to_bf16(h);
      } else {
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
                                                           float* __restrict__ out) {
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
      sa[r][kk] = grow < tm.row_end ? A[grow * K + k0 + kk] : 0.0f;
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
        const float h = silu(acc[r]) * s_up[wm][r][lane];
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

template <int BM, bool SWIGLU, bool OUT_F32, bool B_NK = false>
hipError_t launch_bf16(const bf16_t* A, const bf16_t* B, const int32_t* offsets, int64_t rows, int E,
                       int K, int ldb, int NT, void* out, hipStream_t stream) {
  constexpr int smem = 2 * BM * kBKT * 2 + 2 * kBN * kBKT * 2;
  auto kern = gemm_bf16_kernel<BM, SWIGLU, OUT_F32, B_NK>;
  // once per instantiation (and never inside a stream capture after the first eager call)
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (attr != hipSuccess) return attr;
  const unsigned grid = grid_for(max_tiles<BM>(rows, E, offsets == nullptr), NT);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kGemmThreads), smem, stream, A, B, offsets, rows, E, K, ldb, NT,
                     out);
  return hipGetLastError();
}

// GEMM1 (+SwiGLU) then GEMM2 with BM-row tiles; `between` (optional) is recorded after GEMM1.
template <int BM>
hipError_t launch_bf16_pair(const void* x_perm, const void* w1, const void* w2, const int32_t* offsets,
                            int64_t rows, int E, int H, int F, void* y_perm, int out_dt, void* scratch,
                            hipStream_t stream, hipEvent_t between) {
  bf16_t* h = static_cast<bf16_t*>(scratch);
  hipError_t err = launch_bf16<BM, true, false>(static_cast<const bf16_t*>(x_perm), static_cast<const bf16_t*>(w1),
                                                offsets, rows, E, H, 2 * F, F / 128, h, stream);
  if (err != hipSuccess) return err;
  if (between && (err = hipEventRecord(between, stream)) != hipSuccess) return err;
  const int nt2 = static_cast<int>(ceil_div(H, kBN));
  if (out_dt == 0)
    return launch_bf16<BM, false, true>(h, static_cast<const bf16_t*>(w2), offsets, rows, E, F, H, nt2, y_perm, stream);
  return launch_bf16<BM, false, false>(h, static_cast<const bf16_t*>(w2), offsets, rows, E, F, H, nt2, y_perm, stream);
}

}  // namespace

size_t grouped_swiglu_scratch_bytes(int64_t rows, int F, int dt) {
  if (dt == 0) return static_cast<size_t>(rows) * F * 4;
  if (dt == 1) return static_cast<size_t>(rows) * F * 2;
  // fp8: h codes + their 1x128 scales
  return fp8_hidden_bytes(rows, F) + static_cast<size_t>(rows) * (F / 128) * 4;
}

hipError_t launch_grouped_swiglu(const void* x_perm, const float* x_scales, int dt,
                                 const int32_t* offsets, int64_t rows, int E, int H, int F,
                                 const void* w1, const float* w1_scales, const void* w2,
                                 const float* w2_scales, void* y_perm, int out_dt, void* scratch,
                                 hipStream_t stream, hipEvent_t between) {
  if (dt == 2)
    return launch_grouped_swiglu_fp8(x_perm, x_scales, offsets, rows, E, H, F, w1, w1_scales, w2, w2_scales,
                                     y_perm, out_dt, scratch, stream, between);
  if (dt == 0) {
    float* h = static_cast<float*>(scratch);
    const int nt1 = F / 32, nt2 = static_cast<int>(ceil_div(H, kF32BN));
    const unsigned g1 = grid_for(max_tiles<kF32BM>(rows, E, offsets == nullptr), nt1);
    hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(g1), dim3(kThreads), 0, stream,
                       static_cast<const float*>(x_perm), static_cast<const float*>(w1), offsets, rows, E,
                       H, 2 * F, nt1, h);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (between && (err = hipEventRecord(between, stream)) != hipSuccess) return err;
    const unsigned g2 = grid_for(max_tiles<kF32BM>(rows, E, offsets == nullptr), nt2);
    hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(g2), dim3(kThreads), 0, stream, h,
                       static_cast<const float*>(w2), offsets, rows, E, F, H, nt2,
                       static_cast<float*>(y_perm));
    return hipGetLastError();
  }
  if (dt == 1) {
    // 256-row tiles when experts average >= 768 rows, else 128-row tiles (less padding)
    const bool big = offsets == nullptr ? rows >= 768 : rows >= 768 * static_cast<int64_t>(E);
    return big ? launch_bf16_pair<256>(x_perm, w1, w2, offsets, rows, E, H, F, y_perm, out_dt, scratch, stream, between)
               : launch_bf16_pair<128>(x_perm, w1, w2, offsets, rows, E, H, F, y_perm, out_dt, scratch, stream, between);
  }
  return hipErrorNotSupported;
}

}  // namespace moe
