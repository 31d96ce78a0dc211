// common.hpp -- shared device helpers and the internal launcher interface of the MoE library.
// gfx950 (CDNA4) only: 64-lane wavefronts, MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32 (two values per instruction,
// the shader's default rounding mode, round to nearest even).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return static_cast<bf16_t>(pack_bf16x2(f, 0.0f)); }

// SiLU(z) = z / (1 + e^-z)
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Four fp32 values already clamped to [-448, 448] -> four OCP E4M3 ("e4m3fn") codes, byte i for
// value i, rounded to nearest with ties to even (the format: 1-4-3 bits, bias 7, subnormals m 2^-9,
// largest finite 448): gfx950's v_cvt_pk_fp8_f32, two values per instruction, in the shader's
// default rounding mode.  A negative value that rounds to zero is written as +0 (code 0x00), so a
// zero is always the one code.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  const uint32_t u = static_cast<uint32_t>(w);
  const uint32_t mag = u & 0x7F7F7F7Fu;
  const uint32_t nz = (mag + 0x7F7F7F7Fu) & 0x80808080u;  // bit 7 of a byte: its magnitude is not 0
  return mag | (u & nz);
}

// Scale of an e4m3 block with max magnitude amax: the smallest power of two 2^q with
// 448 * 2^q >= amax, q clamped to [-127, 127] (an E8M0 value), or 1 for an all-zero block.
// For a normal amax = 1.m * 2^(e - 127): 448 = 1.75 * 2^8, so q = e - 135, plus one when
// 1.m > 1.75 (mantissa bits above 0x600000); a subnormal amax gives q < -127.
__device__ __forceinline__ float e4m3_block_scale(float amax) {
  if (!(amax > 0.0f)) return 1.0f;
  const uint32_t u = __float_as_uint(amax);
  const int e = static_cast<int>((u >> 23) & 0xFFu);
  int q = e == 0 ? -127 : e - 135 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  q = q < -127 ? -127 : (q > 127 ? 127 : q);
  return q == -127 ? __uint_as_float(0x00400000u) : __uint_as_float(static_cast<uint32_t>(q + 127) << 23);
}

// 1 / s for a scale from e4m3_block_scale (s = 2^q, q in [-127, 127], or 1): 2^-q, built from the
// exponent bits, so x * pow2_inverse(s) is x / s rounded once, exactly like the division.
__device__ __forceinline__ float pow2_inverse(float s) {
  const uint32_t u = __float_as_uint(s);
  if (u == 0x00400000u) return __uint_as_float(0x7F000000u);  // 1 / 2^-127 = 2^127
  const uint32_t e = u >> 23;                                   // 1 .. 254 (s is positive, normal)
  return e == 254u ? __uint_as_float(0x00400000u) : __uint_as_float((254u - e) << 23);
}

// E8M0 byte of a power-of-two fp32 scale (its biased exponent; 2^-127 -> 0).
__device__ __forceinline__ int e8m0_of(float s) { return static_cast<int>((__float_as_uint(s) >> 23) & 0xFFu); }

// ---- MXFP4: FP4 E2M1 elements (1 sign, 2 exponent bits with bias 1, 1 mantissa bit; magnitudes
// 0, 0.5, 1, 1.5, 2, 3, 4, 6) with one E8M0 scale byte (2^(e - 127)) per 32 elements.
// Codes of eight scaled values (|v| <= 6), nibble i for value i (low nibble first): the nearest
// magnitude, ties to the even-mantissa code, on gfx950's v_cvt_scalef32_pk_fp4_f32 (two values per
// instruction, scale 1, the shader's default rounding mode); a negative value that rounds to zero
// is written as +0 (code 0), so a zero is always the one code.
__device__ __forceinline__ uint32_t pack_fp4x8(float v0, float v1, float v2, float v3, float v4, float v5,
                                               float v6, float v7) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v0, v1, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v2, v3, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v4, v5, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v6, v7, 1.0f, 3);
  const uint32_t mag = w & 0x77777777u;
  const uint32_t nz = (mag + 0x77777777u) & 0x88888888u;  // bit 3 of a nibble: its magnitude is not 0
  return mag | (w & nz);
}

// E8M0 byte of the smallest power of two 2^q with 6 * 2^q >= amax, q in [-127, 127]; 127 (2^0) for
// an all-zero block.  For a normal amax = 1.m * 2^(E - 127): 6 = 1.5 * 2^2, so q = E - 129, plus
// one when 1.m > 1.5 (mantissa bits above 0x400000); a subnormal amax needs q = -127.
__device__ __forceinline__ int fp4_block_e8m0(float amax) {
  if (!(amax > 0.0f)) return 127;
  const uint32_t u = __float_as_uint(amax);
  const int E = static_cast<int>((u >> 23) & 0xFFu);
  int q = E == 0 ? -127 : E - 129 + ((u & 0x7FFFFFu) > 0x400000u ? 1 : 0);
  q = q < -127 ? -127 : (q > 127 ? 127 : q);
  return q + 127;
}

// 2^(127 - e), the inverse of the E8M0 scale e in [0, 254] (2^-127 is the fp32 subnormal 0x00400000):
// x * e8m0_inverse(e) is x / 2^(e - 127) rounded once.
__device__ __forceinline__ float e8m0_inverse(int e) {
  return e < 254 ? __uint_as_float(static_cast<uint32_t>(254 - e) << 23) : __uint_as_float(0x00400000u);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 0xFu;
  uint32_t m = c & 7u;
  float mag;
  if (e == 0) {
    mag = static_cast<float>(m) * (1.0f / 512.0f);
  } else {
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  }
  return __uint_as_float(__float_as_uint(mag) | s);
}

// Wave-wide reductions (64 lanes) with cross-lane shuffles.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------ launcher interface
// Every launcher enqueues on `stream` and returns hipGetLastError() of its launches.
// dtype codes follow moe.h: 0 = fp32, 1 = bf16, 2 = fp8 e4m3, 3 = MXFP4.  Scale pointers are
// fp32 arrays for e4m3 and E8M0 byte arrays for MXFP4.

// scratch: logits (when `logits` is null) followed by the split router weight
hipError_t launch_route(const void* x, int x_dt, const float* w_router, const float* bias, int64_t T,
                        int H, int E, int k, int score, int norm, float* logits, int32_t* ids,
                        float* gates, void* scratch, hipStream_t stream);
size_t route_scratch_bytes(int64_t T, int H, int E, bool logits_given);

size_t permute_scratch_bytes(int64_t T, int E, int k);
// With gates [T, k] and gate_perm [T k] (both or neither), also writes each permuted row's gate:
// gate_perm[row_map[t, j]] = gates[t, j].
hipError_t launch_permute(const void* x, int x_dt, const int32_t* ids, int64_t T, int H, int E, int k,
                          void* x_perm, int perm_dt, void* x_perm_scales, int32_t* row_map,
                          int32_t* src_token, int32_t* counts, int32_t* offsets, void* scratch,
                          hipStream_t stream, const float* gates = nullptr, float* gate_perm = nullptr);

size_t grouped_swiglu_scratch_bytes(int64_t rows, int F, int dt);
// offsets == nullptr means one expert owning rows [0, rows) (the shared expert).  With
// `gather`, row p of the first GEMM's A operand is row gather[p] of x_perm (and of x_scales):
// the dispatch permutation fused into the GEMM's loads, so x_perm can be the unpermuted input.
// With `row_scale` [rows], the SwiGLU epilogue multiplies row p of h by row_scale[p] before it is
// rounded (the routing gate folded into the expert), so y_perm row p comes out scaled by it.
hipError_t launch_grouped_swiglu(const void* x_perm, const void* x_scales, int dt,
                                 const int32_t* offsets, int64_t rows, int E, int H, int F,
                                 const void* w1, const void* w1_scales, const void* w2,
                                 const void* w2_scales, void* y_perm, int out_dt, void* scratch,
                                 hipStream_t stream, hipEvent_t between = nullptr,
                                 const int32_t* gather = nullptr, const float* row_scale = nullptr);

// Dense out[rows, N] (fp32) = A[rows, K] . B[K, N] with bf16 A and B (B N-contiguous),
// K % 64 == 0, N % 8 == 0: the grouped-GEMM kernel with one expert, on bm-row tiles (128 or 256).
// With ksplit > 1 (K / 64 a multiple of ksplit) K is cut into ksplit equal slices and out[s] (at
// out + s * rows * N) gets slice s's partial product; the caller sums them.
hipError_t launch_dense_gemm_f32out(const void* A, const void* B, int64_t rows, int K, int N, float* out,
                                    hipStream_t stream, int ksplit = 1, int bm = 128);

// Grouped out[p, :] (fp32) = A[gather ? gather[p] : p] . B_e over the rows of each expert, bf16
// operands (B [E, K, N] N-contiguous, K % 64 == 0, N % 256 == 0): the grouped-GEMM kernel without
// the SwiGLU epilogue.  gather entries must lie inside A.
hipError_t launch_grouped_gemm_f32out(const void* A, const void* B, const int32_t* offsets, int64_t rows, int E,
                                      int K, int N, float* out, hipStream_t stream, const int32_t* gather);

// The same with the weight read transposed: out[p, n] = sum_k A[gather ? gather[p] : p, k] B_e[n, k],
// B [E, N, K] K-contiguous (the stored W2 [F, H] and W1 [H, 2F] of an expert read as W2^T, W1^T),
// bf16 operands, K % 64 == 0, N % 8 == 0, fp32 out.
hipError_t launch_grouped_gemm_nt_f32out(const void* A, const void* B, const int32_t* offsets, int64_t rows, int E,
                                         int K, int N, float* out, hipStream_t stream, const int32_t* gather);

// The same with bf16 output (fp32 accumulation, one rounding per element), N % 8 == 0.
hipError_t launch_grouped_gemm_nt_bf16out(const void* A, const void* B, const int32_t* offsets, int64_t rows, int E,
                                          int K, int N, void* out, hipStream_t stream, const int32_t* gather);

// E independent products out_e [M, N] (fp32, out_e at out + e M N) = A_e . B_e, bf16 operands:
// A_e is columns [P_e, P_{e+1}) of A [M, lda] (P = kinfo[0 .. E], multiples of 64; A's columns
// past an expert's own rows hold zeros) and B_e is P_{e+1} - P_e rows of B [*, N] from row
// kinfo[E + 1 + e] on (rows that B must hold, finite).  lda % 8 == 0, N % 8 == 0.
hipError_t launch_batched_gemm_f32out(const void* A, int64_t lda, const void* B, const int32_t* kinfo, int E, int M,
                                      int N, float* out, hipStream_t stream);

// FP8 (E4M3) path: x_perm codes + [rows, H/128] scales, weights as codes + 128x128-block scales;
// the SwiGLU output h is re-quantised to E4M3 in 1x128 blocks in the scratch buffer
// (fp8_hidden_bytes(rows, F) bytes of codes, then [rows, F/128] fp32 scales).
size_t fp8_hidden_bytes(int64_t rows, int F);
hipError_t launch_grouped_swiglu_fp8(const void* x_perm, const float* x_scales, const int32_t* offsets,
                                     int64_t rows, int E, int H, int F, const void* w1, const float* w1_scales,
                                     const void* w2, const float* w2_scales, void* y_perm, int out_dt,
                                     void* scratch, hipStream_t stream, hipEvent_t between,
                                     const int32_t* gather, const float* row_scale = nullptr);
// Per-row 1x128 E4M3 quantisation of a dense [T, H] bf16 / fp32 matrix (shared-expert input).
hipError_t launch_quant_rows_fp8(const void* x, int x_dt, int64_t T, int H, uint8_t* codes, float* scales,
                                 hipStream_t stream);

// MXFP4 path: activations [rows, H / 2] codes + [rows, H / 32] E8M0; weights stored contraction-
// contiguous, W1 [E, 2F, H / 2] + [E, 2F, H / 32] and W2 [E, H, F / 2] + [E, H, F / 32]; h re-quantised
// to MXFP4 in 1 x 32 blocks in the scratch buffer (fp4_hidden_bytes(rows, F) bytes: codes, then
// scales, each 256-byte aligned).  H and F multiples of 256.
size_t fp4_hidden_bytes(int64_t rows, int F);
hipError_t launch_grouped_swiglu_fp4(const void* x_perm, const void* x_scales, const int32_t* offsets,
                                     int64_t rows, int E, int H, int F, const void* w1, const void* w1_scales,
                                     const void* w2, const void* w2_scales, void* y_perm, int out_dt,
                                     void* scratch, hipStream_t stream, hipEvent_t between,
                                     const int32_t* gather, const float* row_scale = nullptr);
// Per-row 1x32 MXFP4 quantisation of a dense [T, H] bf16 matrix (H % 32 == 0).
hipError_t launch_quant_rows_fp4(const void* x, int64_t T, int H, uint8_t* codes, uint8_t* scales,
                                 hipStream_t stream);

// gates == nullptr: every weight is 1 (rows already scaled by their gates).
hipError_t launch_combine(const void* y_perm, int y_dt, const int32_t* row_map, const float* gates,
                          const void* shared_out, int64_t T, int H, int k, void* y, int out_dt,
                          hipStream_t stream);

// ------------------------------------------------------------------------ backward
constexpr int kMaxTopk = 16;

struct BackwardShape {
  int64_t T;
  int H, E, k, F, Fs, score, norm;
};
// Inputs and outputs of the layer backward (device pointers; shapes as in moe.h).
struct BackwardIO {
  const void *x, *dy;  // [T, H] in the layer's dtype
  const float* w_router;
  const void *w1, *w2, *ws1, *ws2;
  const float* logits;  // forward routing state
  const int32_t* ids;
  const float* gates;
  const int32_t *offsets, *row_map, *src_token;
  void* dx;  // [T, H] in the layer's dtype
  float *dw_router, *dw1, *dw2, *dws1, *dws2;
};
// Workspace pieces: u = x W1 [R, 2F] and dh' = dy W2^T [R, F] in fp32; du [R, 2F] and g h [R, F]
// in the GEMM operand type; dg [R]; dxp [R, H]; dlogits [T, E]; dlogits W_r^T [T, H]; the shared
// expert's u, dh', du, h and dx.
struct BackwardScratch {
  float* dwr_part;  // [router_slices, H, E] partial router-weight gradients (null for one slice)
  float *u, *dhp;
  void *du, *gh;
  float *dg;
  void* dxp;  // [T*k, H] row gradients in the layer's dtype (bf16 rows are summed in fp32)
  float *dl, *dxr;
  float *us, *dhs;
  void *dus, *ghs;
  void* dxs;  // the shared expert's [T, H] input gradient, in the layer's dtype
  // bf16 weight gradients as per-expert products (launch_batched_gemm_f32out): the padded
  // contraction table (2 (E + 1) ints, routed and shared), the transposed zero-padded activations
  // ([H or F][ld_t]) and dy gathered into expert-row order with 64 zero rows after the end
  int32_t *kinfo, *kinfo_s;
  void *xt, *dyp;
  int64_t ld_t;
  // the router's products of a bf16 layer as bf16 products (router_split): dlogits split into
  // three bf16 parts ([T, 6E] for dx, [T + 64, 3E] for dW_r), W_r split ([H, 6E]), the row slices of
  // dW_r's contraction (offsets, S + 1 ints) and their partial products [S, H, 3E]
  void *ra6, *rb6, *rd3;
  int32_t* roff;
  float* rpart;
  int rS;
};
// Row slices of the router-weight gradient x^T dlogits (its [H, E] output has few tiles).
int router_slices(int64_t T, int H, int E);
// Whether a layer's router products run as split bf16 products (bf16 layers, E % 32 == 0,
// H % 64 == 0), and the row slices of dW_r's contraction then.
bool router_split(const BackwardShape& sh, int dt);
int router_split_slices(int64_t T);
// Carves the workspace from `base` (null: sizes only); *bytes receives the total.
BackwardScratch carve_backward(const BackwardShape& sh, int dt, void* base, size_t* bytes);
// dt: 0 = fp32, 1 = bf16 (activations, weights and dy alike).  events: null or 9 hipEvent_t
// (null entries skipped) recorded before the backward, after the routed experts' u, dh', SwiGLU
// backward, dW2, dxp and dW1 steps, after the shared expert, and at the end.
hipError_t launch_layer_backward(const BackwardShape& sh, int dt, const BackwardIO& io, const BackwardScratch& ws,
                                 hipStream_t stream, hipEvent_t const* events);

}  // namespace moe
