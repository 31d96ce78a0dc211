// gemm_fp4.hip -- Compute stage with MXFP4 expert GEMMs (both operands 4-bit).
//
// The pages name low-precision training in FP8 and NVFP4 ("Scalable Training of Mixture-of-Experts
// Models with Megatron Core", index page, abstract; summary page, "Key claims" [§5]).  The 4-bit
// format CDNA4's matrix cores take natively is MXFP4: FP4 E2M1 elements, one E8M0 (power-of-two)
// scale per 32 consecutive elements along the contraction, which v_mfma_scale_f32_32x32x64_f8f6f4
// applies per lane in hardware.  Per expert e and row p of e:
//     u = x_perm[p] . W1[e];  h = SiLU(gate) * up  (fused epilogue, h re-quantised to MXFP4)
//     y_perm[p] = h . W2[e]
// Layouts: every operand is stored contraction-contiguous, two elements per byte (element 2i in
// the low nibble) with one E8M0 byte per 32 elements:
//     activations / h   [rows, K / 2] + [rows, K / 32]
//     W1[e] (logical [H, 2F])   stored [2F, H / 2] + [2F, H / 32]
//     W2[e] (logical [F, H])    stored [H, F / 2] + [H, F / 32]
// so both MFMA operands are read the same way: lane l takes 32 consecutive elements (16 bytes) of
// row (or weight column) l % 32, half l / 32 of the 64-deep step, plus that block's scale byte.
//
// Tile BM x 256 (SwiGLU: 128 gate + the matching 128 up columns), 8 waves in a 2 (M) x 4 (N)
// grid, each wave (BM / 2) x 64 in 32 x 32 blocks.  K advances 256 elements (128 bytes per row)
// per stage; a ring of NS LDS stages holds the A rows, the 256 B rows and both operands' scale
// bytes of a stage, all loaded global -> LDS by direct loads (16-byte rows, 4-byte scale words).
// Chunk c (16 bytes) of row r of a stage is stored at chunk c ^ ((r >> 1) & 7).  One barrier per
// stage; the loads of stage kt + NS - 1 go out right after it, into the slot stage kt - 1 left.
#include "gemm_common.hpp"

namespace moe {
namespace {

using namespace gemm;

constexpr int kF4KS = 256;          // K elements per stage
constexpr int kF4Row = kF4KS / 2;   // bytes per row per stage
constexpr int kF4Blocks = kF4KS / 32;  // E8M0 scales per row per stage (8 bytes)

template <int BM>
struct F4Cfg {
  static constexpr int NS = 3;                      // ring stages
  static constexpr int A_BYTES = BM * kF4Row;
  static constexpr int B_BYTES = kBN * kF4Row;
  static constexpr int AS_BYTES = BM * kF4Blocks;
  static constexpr int BS_BYTES = kBN * kF4Blocks;
  static constexpr int B_OFF = A_BYTES, AS_OFF = A_BYTES + B_BYTES, BS_OFF = AS_OFF + AS_BYTES;
  static constexpr int STAGE = BS_OFF + BS_BYTES;
  static constexpr int SMEM = NS * STAGE;
};

typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t_f4;
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2_t;

// 4 bytes per lane from global memory straight into LDS at lds_addr + 4 * lane.
__device__ __forceinline__ void lds_dma4_f4(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gptr),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// Global weight row (stored [N, K / 2]) of row r of a 256-row B tile: SwiGLU tiles hold gate
// rows nt * 128 .. and the matching up rows F + nt * 128 ..; others rows nt * 256 + r (rows past
// N re-read row 0: never stored).
template <bool SWIGLU>
__device__ __forceinline__ int64_t b_tile_row(int nt, int r, int N) {
  int64_t n;
  if (SWIGLU) {
    const int F = N / 2;
    n = r < 128 ? static_cast<int64_t>(nt) * 128 + r : F + static_cast<int64_t>(nt) * 128 + (r - 128);
  } else {
    n = static_cast<int64_t>(nt) * kBN + r;
  }
  return n < N ? n : 0;
}

template <int BM, bool SWIGLU, bool OUT_F32>
__global__ __launch_bounds__(kGemmThreads) void gemm_fp4_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ A_scales, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ B_scales, const int32_t* __restrict__ offsets, int64_t rows, int E, int K, int N,
    int NT, void* __restrict__ out, uint8_t* __restrict__ out_scales, const int32_t* __restrict__ gather,
    const float* __restrict__ row_scale) {
  using C = F4Cfg<BM>;
  constexpr int NS = C::NS;
  constexpr int NWAVE = kGemmThreads / kWave;      // 8: 2 along M x 4 along N
  constexpr int WROWS = BM / 2;
  constexpr int FM = WROWS / 32, FN = 2;
  constexpr int A_ROUNDS = C::A_BYTES / 1024 / NWAVE;  // 16-byte direct loads per wave per stage
  constexpr int B_ROUNDS = C::B_BYTES / 1024 / NWAVE;
  constexpr int AS_WAVES = C::AS_BYTES / 256;          // waves with one 4-byte scale load of A
  constexpr int BS_ROUNDS = C::BS_BYTES / 256 / NWAVE; // 4-byte scale loads of B per wave
  static_assert(C::A_BYTES % (1024 * NWAVE) == 0 && C::BS_BYTES % (256 * NWAVE) == 0, "tile shape");
  static_assert(AS_WAVES <= NWAVE, "A scale loads");

  extern __shared__ __attribute__((aligned(1024))) char smem[];
  __shared__ int s_pref[kMaxExpertsLds];
  TileMap tm;
  if (SWIGLU ? !map_tile_auto<BM>(offsets, rows, E, NT, s_pref, tm) : !map_tile<BM>(offsets, rows, E, NT, s_pref, tm))
    return;

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 4, wn = wave % 4;
  const int khalf = lane / 32;
  lds_void_t* lds = (lds_void_t*)smem;
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
  const int nk = K / kF4KS;
  const int kb_row = K / 32;     // scale bytes per row
  const int64_t kbytes = K / 2;  // code bytes per row

  // ---- global sources of the direct loads.  A (or B) round p of wave w covers tile rows
  // (8 p + w) * 8 + lane / 8 (1 KB = 8 rows x 128 B); stored chunk lane % 8 holds logical chunk
  // (lane % 8) ^ ((row >> 1) & 7).
  const uint8_t* a_src[A_ROUNDS];
#pragma unroll
  for (int p = 0; p < A_ROUNDS; ++p) {
    const int r = (NWAVE * p + wave) * 8 + lane / 8;
    int64_t grow = tm.row0 + r;
    if (grow >= tm.row_end) grow = tm.row_end - 1;
    if (gather) grow = gather[grow];  // fused dispatch: row p of the tile is token gather[p]
    a_src[p] = A + grow * kbytes + (((lane % 8) ^ ((r >> 1) & 7)) * 16);
  }
  const uint8_t* Bexp = B + static_cast<int64_t>(tm.expert) * N * kbytes;
  const uint8_t* b_src[B_ROUNDS];
#pragma unroll
  for (int p = 0; p < B_ROUNDS; ++p) {
    const int r = (NWAVE * p + wave) * 8 + lane / 8;
    b_src[p] = Bexp + b_tile_row<SWIGLU>(tm.nt, r, N) * kbytes + (((lane % 8) ^ ((r >> 1) & 7)) * 16);
  }
  // scale words: A word d = 64 w + lane (waves w < AS_WAVES) is half d % 2 of row d / 2's 8 bytes;
  // B word d = 64 (8 q + w) + lane likewise for the B tile's rows
  const uint8_t* as_src = nullptr;
  if (wave < AS_WAVES) {
    const int d = 64 * wave + lane;
    int64_t grow = tm.row0 + d / 2;
    if (grow >= tm.row_end) grow = tm.row_end - 1;
    if (gather) grow = gather[grow];
    as_src = A_scales + grow * kb_row + (d % 2) * 4;
  }
  const uint8_t* bs_src[BS_ROUNDS];
#pragma unroll
  for (int q = 0; q < BS_ROUNDS; ++q) {
    const int d = 64 * (NWAVE * q + wave) + lane;
    bs_src[q] = B_scales + (static_cast<int64_t>(tm.expert) * N + b_tile_row<SWIGLU>(tm.nt, d / 2, N)) * kb_row +
                (d % 2) * 4;
  }
  auto stage_base = [&](int kt) { return lds_base + static_cast<uint32_t>(kt % NS) * C::STAGE; };
  auto issue_stage = [&](int kt) {
    if (kt >= nk) return;
    const uint32_t base = stage_base(kt);
    const int64_t kofs = static_cast<int64_t>(kt) * kF4Row;
#pragma unroll
    for (int p = 0; p < A_ROUNDS; ++p) lds_dma16(a_src[p] + kofs, base + (NWAVE * p + wave) * 1024);
#pragma unroll
    for (int p = 0; p < B_ROUNDS; ++p) lds_dma16(b_src[p] + kofs, base + C::B_OFF + (NWAVE * p + wave) * 1024);
    if (wave < AS_WAVES) lds_dma4_f4(as_src + kt * kF4Blocks, base + C::AS_OFF + wave * 256);
#pragma unroll
    for (int q = 0; q < BS_ROUNDS; ++q)
      lds_dma4_f4(bs_src[q] + kt * kF4Blocks, base + C::BS_OFF + (NWAVE * q + wave) * 256);
  };
  // loads per wave per stage (the A-scale word only on waves < AS_WAVES)
  constexpr int RPT = A_ROUNDS + B_ROUNDS + BS_ROUNDS;
  // stage kt has landed once at most `later` stages issued after it are still in flight
  auto wait_stage = [&](int later) {
    if (later <= 0) { wait_vmcnt<0>(); return; }
    if (wave < AS_WAVES) wait_vmcnt<RPT + 1>();
    else wait_vmcnt<RPT>();
  };
  static_assert(NS == 3, "wait_stage assumes at most one later stage in flight");

  // ---- fragment and scale addresses inside a stage
  uint32_t a_row[FM], a_sw[FM], b_row[FN], b_sw[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = wm * WROWS + i * 32 + lane % 32;
    a_row[i] = r;
    a_sw[i] = (r >> 1) & 7;
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int r = SWIGLU ? j * 128 + wn * 32 + lane % 32 : wn * 64 + j * 32 + lane % 32;
    b_row[j] = r;
    b_sw[j] = (r >> 1) & 7;
  }

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  int nl_rows = static_cast<int>((tm.row_end - tm.row0 < BM ? tm.row_end - tm.row0 : BM)) - wm * WROWS;
  nl_rows = nl_rows < 0 ? 0 : nl_rows;
  const int nlive = __builtin_amdgcn_readfirstlane(nl_rows >= WROWS ? FM : (nl_rows + 31) / 32);

  auto run = [&](auto nl_c) {
    constexpr int NL = decltype(nl_c)::value;
    constexpr int NLA = NL > 0 ? NL : 1;
    i32x8_t af[2][NLA], bf[2][FN];
    u32x2_t sa[NLA], sb[FN];
    auto read_frags = [&](uint32_t base, int s, int buf) {
      const uint32_t c = 2 * s + khalf;  // 16-byte chunk: elements 64 s + 32 khalf .. +32
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const u32x4_t v = *reinterpret_cast<const lds_u32x4_t_f4*>(
            static_cast<uintptr_t>(base + C::B_OFF + b_row[j] * kF4Row + ((c ^ b_sw[j]) << 4)));
        bf[buf][j] = i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const u32x4_t v = *reinterpret_cast<const lds_u32x4_t_f4*>(
            static_cast<uintptr_t>(base + a_row[i] * kF4Row + ((c ^ a_sw[i]) << 4)));
        af[buf][i] = i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
      }
    };
    auto read_scales = [&](uint32_t base) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
        sa[i] = *reinterpret_cast<const lds_u32x2_t*>(static_cast<uintptr_t>(base + C::AS_OFF + a_row[i] * 8));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        sb[j] = *reinterpret_cast<const lds_u32x2_t*>(static_cast<uintptr_t>(base + C::BS_OFF + b_row[j] * 8));
    };
    // sub-step s: block 2 s + khalf of the stage's 8 per row: word s / 2, byte 2 (s % 2) + khalf
    auto mfmas = [&](int s, int buf) {
      const int sh = 8 * (2 * (s % 2) + khalf);
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int ea = static_cast<int>((s < 2 ? sa[i][0] : sa[i][1]) >> sh);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int eb = static_cast<int>((s < 2 ? sb[j][0] : sb[j][1]) >> sh);
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[buf][j], af[buf][i], acc[i][j], 4, 4, 0, eb,
                                                                       0, ea);
        }
      }
    };

#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue_stage(st);
    for (int kt = 0; kt < nk; ++kt) {
      wait_stage(kt + 1 < nk ? 1 : 0);  // this wave's loads of stage kt have landed
      lds_barrier();                    // every wave's: stage kt readable, stage kt - 1 free
      issue_stage(kt + NS - 1);         // into the slot stage kt - 1 used
      if constexpr (NL > 0) {
        const uint32_t base = stage_base(kt);
        read_scales(base);
        read_frags(base, 0, 0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (s < 3) read_frags(base, s + 1, (s + 1) % 2);
          mfmas(s, s % 2);
        }
      }
      wait_lgkm0();  // this wave's reads of stage kt are done before the next barrier frees it
    }
  };
  dispatch_live<FM>(nlive, run);

  // ---- epilogue.  The MFMAs take the weight fragment as their first operand, so each computes a
  //      transposed 32x32 block: slot r of lane l of acc[i][j] is the wave's row i * 32 + l % 32
  //      and column j * 32 + (r / 4) * 8 + (l / 32) * 4 + (r % 4) of block j -- 4 adjacent
  //      columns of one row per group of 4 slots, written 16 (fp32) or 8 (bf16) bytes at a time.
  __syncthreads();  // every wave is done with the ring
  if constexpr (SWIGLU) {
    // h = SiLU(gate) * up (x the row's gate when folded), staged as fp32 [BM][128 + 8]; then 8 lanes
    // per row, 16 columns each: a 32-column block is 2 lanes (amax: 1 shuffle), each lane packs
    // its 16 codes into 8 bytes and even lanes write the block's E8M0 byte.
    constexpr int kHS = 132;  // row stride in floats: 16 consecutive rows start 4 banks apart
    static_assert(BM * kHS * 4 <= C::SMEM, "h staging fits in the ring");
    const int F = N / 2;
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
      const int64_t grow = tm.row0 + row_t;
      const float g = row_scale != nullptr ? row_scale[grow < tm.row_end ? grow : tm.row_end - 1] : 1.0f;
      const f32x4_t* src = reinterpret_cast<const f32x4_t*>(hl + row_t * kHS + seg * 16);
      float v[16];
      float m = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t w = src[q];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          v[4 * q + c] = row_scale != nullptr ? w[c] * g : w[c];
          m = fmaxf(m, fabsf(v[4 * q + c]));
        }
      }
      m = fmaxf(m, __shfl_xor(m, 1, kWave));
      const int e = fp4_block_e8m0(m);
      const float inv = e8m0_inverse(e);
      uint32_t packed[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float* p = v + 8 * h;
        packed[h] = pack_fp4x8(p[0] * inv, p[1] * inv, p[2] * inv, p[3] * inv, p[4] * inv, p[5] * inv, p[6] * inv,
                               p[7] * inv);
      }
      if (grow < tm.row_end) {
        *reinterpret_cast<u32x2_t*>(hq + grow * (F / 2) + static_cast<int64_t>(tm.nt) * 64 + seg * 8) =
            u32x2_t{packed[0], packed[1]};
        if ((seg & 1) == 0) out_scales[grow * (F / 32) + tm.nt * 4 + seg / 2] = static_cast<uint8_t>(e);
      }
    }
  } else if constexpr (!OUT_F32) {
    constexpr int kYS = 264;  // bf16 row stride: rows 16-byte aligned
    static_assert(BM * kYS * 2 <= C::SMEM, "y staging fits in the ring");
    bf16_t* yl = reinterpret_cast<bf16_t*>(smem);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i * 32 >= nl_rows) continue;  // no row of this block is live (wave-uniform)
      const int row_t = wm * WROWS + i * 32 + lane % 32;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<u32x2_t*>(yl + row_t * kYS + wn * 64 + j * 32 + q * 8 + khalf * 4) =
              u32x2_t{pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                      pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
    }
    __syncthreads();
    const int seg = tid % 32;
    const int64_t col = static_cast<int64_t>(tm.nt) * kBN + seg * 8;
    if (col < N) {  // N % 256 == 0
#pragma unroll
      for (int pass = 0; pass < BM / 16; ++pass) {
        const int row_t = pass * 16 + tid / 32;
        const int64_t grow = tm.row0 + row_t;
        if (grow < tm.row_end)
          *reinterpret_cast<u32x4_t*>(static_cast<bf16_t*>(out) + grow * N + col) =
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
          if (col < N) {  // N % 256 == 0
            const f32x4_t w = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + grow * N + col) = w;
          }
        }
    }
  }
}

constexpr int kF4BM = 128;

template <bool SWIGLU, bool OUT_F32>
hipError_t launch_fp4(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs,
                      const int32_t* offsets, int64_t rows, int E, int K, int N, int NT, void* out,
                      uint8_t* out_scales, hipStream_t stream, const int32_t* gather, const float* row_scale) {
  constexpr int smem = F4Cfg<kF4BM>::SMEM;
  auto kern = gemm_fp4_kernel<kF4BM, SWIGLU, OUT_F32>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (attr != hipSuccess) return attr;
  const int64_t mt = max_tiles<kF4BM>(rows, E, offsets == nullptr);
  const unsigned grid = SWIGLU ? grid_for_any(mt, NT, E, offsets == nullptr) : grid_for(mt, NT);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kGemmThreads), smem, stream, A, As, B, Bs, offsets, rows, E, K, N, NT,
                     out, out_scales, gather, row_scale);
  return hipGetLastError();
}

}  // namespace

size_t fp4_hidden_bytes(int64_t rows, int F) {
  const size_t codes = (static_cast<size_t>(rows) * (F / 2) + 255) & ~static_cast<size_t>(255);
  const size_t scales = (static_cast<size_t>(rows) * (F / 32) + 255) & ~static_cast<size_t>(255);
  return codes + scales;
}

hipError_t launch_grouped_swiglu_fp4(const void* x_perm, const void* x_scales, const int32_t* offsets,
                                     int64_t rows, int E, int H, int F, const void* w1, const void* w1_scales,
                                     const void* w2, const void* w2_scales, void* y_perm, int out_dt,
                                     void* scratch, hipStream_t stream, hipEvent_t between, const int32_t* gather,
                                     const float* row_scale) {
  uint8_t* hq = static_cast<uint8_t*>(scratch);
  uint8_t* hs = hq + ((static_cast<size_t>(rows) * (F / 2) + 255) & ~static_cast<size_t>(255));
  const int nt1 = F / 128, nt2 = static_cast<int>(ceil_div(H, kBN));
  hipError_t err = launch_fp4<true, false>(static_cast<const uint8_t*>(x_perm), static_cast<const uint8_t*>(x_scales),
                                           static_cast<const uint8_t*>(w1), static_cast<const uint8_t*>(w1_scales),
                                           offsets, rows, E, H, 2 * F, nt1, hq, hs, stream, gather, row_scale);
  if (err != hipSuccess) return err;
  if (between && (err = hipEventRecord(between, stream)) != hipSuccess) return err;
  if (out_dt == 0)
    return launch_fp4<false, true>(hq, hs, static_cast<const uint8_t*>(w2), static_cast<const uint8_t*>(w2_scales),
                                   offsets, rows, E, F, H, nt2, y_perm, nullptr, stream, nullptr, nullptr);
  return launch_fp4<false, false>(hq, hs, static_cast<const uint8_t*>(w2), static_cast<const uint8_t*>(w2_scales),
                                  offsets, rows, E, F, H, nt2, y_perm, nullptr, stream, nullptr, nullptr);
}

}  // namespace moe
