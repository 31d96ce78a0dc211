// api.hip -- the extern "C" boundary declared in include/moe.h: host-side validation,
// workspace carving and stage launches.  No device memory is allocated, nothing is copied to
// the host and nothing synchronises, so every entry point is HIP-graph capturable.
#include <mutex>

#include "../../include/moe.h"
#include "common.hpp"

// Scratch of moe_forward_static, for callers that cannot allocate: one copy of this array on every
// GPU the library runs on, held until the process ends.  Host code never uses its name as an
// address (on the host the name is a stand-in, not device memory): static_scratch() resolves the
// device address with hipGetSymbolAddress once per device and every use goes through that.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

using moe::ceil_div;

constexpr size_t kAlign = 256;
size_t align_up(size_t n) { return (n + kAlign - 1) & ~(kAlign - 1); }

moe_status from_hip(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  if (e == hipErrorNotSupported) return MOE_ERR_UNSUPPORTED;
  return MOE_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_common(int64_t T, int32_t H, int32_t E, int32_t k) {
  if (T < 0 || H < 1 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E)
    return MOE_ERR_INVALID_ARG;
  if (T * static_cast<int64_t>(k) >= (int64_t{1} << 31)) return MOE_ERR_INVALID_ARG;
  if (H % 8 != 0) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

bool act_dtype_ok(moe_dtype d) { return d == MOE_F32 || d == MOE_BF16; }

size_t elt_bytes(moe_dtype d) { return d == MOE_F32 ? 4 : (d == MOE_BF16 ? 2 : 1); }

bool low_precision(moe_dtype d) { return d == MOE_FP8_E4M3 || d == MOE_MXFP4; }

// grouped-GEMM shape rules per dtype
moe_status check_gemm_shape(moe_dtype dt, int32_t H, int32_t F) {
  if (H < 1 || F < 1) return MOE_ERR_INVALID_ARG;
  if (dt == MOE_F32) return (H % 32 == 0 && F % 32 == 0) ? MOE_OK : MOE_ERR_INVALID_ARG;
  if (dt == MOE_BF16) return (H % 64 == 0 && F % 128 == 0) ? MOE_OK : MOE_ERR_INVALID_ARG;
  if (dt == MOE_FP8_E4M3) return (H % 128 == 0 && F % 128 == 0) ? MOE_OK : MOE_ERR_INVALID_ARG;
  if (dt == MOE_MXFP4) return (H % 256 == 0 && F % 256 == 0) ? MOE_OK : MOE_ERR_INVALID_ARG;
  return MOE_ERR_INVALID_ARG;
}

// Bump allocator over the caller's workspace.
struct Carve {
  char* base;
  size_t used = 0;
  explicit Carve(void* p) : base(static_cast<char*>(p)) {}
  void* take(size_t n) {
    void* p = base ? base + used : nullptr;
    used += align_up(n);
    return p;
  }
};

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: not supported by this build";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
    case MOE_ERR_TOO_LARGE:
      return "MOE_ERR_TOO_LARGE: the call needs more scratch than the static MOE_STATIC_SCRATCH_BYTES";
  }
  return "unknown moe_status";
}

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

size_t moe_route_workspace_size(int64_t T, int32_t H, int32_t E, int32_t logits_given) {
  if (T < 0 || E < 1 || H < 1) return 0;
  return align_up(moe::route_scratch_bytes(T, H, E, logits_given != 0));
}

moe_status moe_route(const void* x, moe_dtype x_dt, const float* w_router, const float* bias, int64_t T,
                     int32_t H, int32_t E, int32_t k, moe_score score, int32_t norm_topk, float* logits,
                     int32_t* topk_ids, float* topk_gates, void* workspace, size_t workspace_bytes,
                     moe_stream_t stream) {
  moe_status st = check_common(T, H, E, k);
  if (st != MOE_OK) return st;
  if (!act_dtype_ok(x_dt) || (score != MOE_SOFTMAX && score != MOE_SIGMOID)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;  // nothing to do; empty tensors may carry null pointers
  if (!x || !w_router || !topk_ids || !topk_gates) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_route_workspace_size(T, H, E, logits != nullptr);
  if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
  return from_hip(moe::launch_route(x, x_dt, w_router, bias, T, H, E, k, score, norm_topk ? 1 : 0,
                                    logits, topk_ids, topk_gates, workspace,
                                    static_cast<hipStream_t>(stream)));
}

size_t moe_permute_workspace_size(int64_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || k < 1) return 0;
  return align_up(moe::permute_scratch_bytes(T, E, k));
}

moe_status moe_permute(const void* x, moe_dtype x_dt, const int32_t* topk_ids, int64_t T, int32_t H,
                       int32_t E, int32_t k, void* x_perm, moe_dtype perm_dt, void* x_perm_scales,
                       int32_t* row_map, int32_t* src_token, int32_t* expert_counts,
                       int32_t* expert_offsets, void* workspace, size_t workspace_bytes,
                       moe_stream_t stream) {
  moe_status st = check_common(T, H, E, k);
  if (st != MOE_OK) return st;
  if (!act_dtype_ok(x_dt)) return MOE_ERR_INVALID_ARG;
  if (!topk_ids || !row_map || !src_token || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (x_perm) {
    if (!x) return MOE_ERR_INVALID_ARG;
    if (perm_dt == MOE_FP8_E4M3) {
      if (x_dt != MOE_BF16 || H % 128 != 0 || !x_perm_scales) return MOE_ERR_INVALID_ARG;
    } else if (perm_dt == MOE_MXFP4) {
      if (x_dt != MOE_BF16 || H % 32 != 0 || !x_perm_scales) return MOE_ERR_INVALID_ARG;
    } else if (perm_dt != x_dt) {
      return MOE_ERR_INVALID_ARG;
    }
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_INVALID_ARG;
  }
  if (workspace_bytes < moe_permute_workspace_size(T, E, k) || !workspace) return MOE_ERR_WORKSPACE;
  if (T == 0) return MOE_ERR_UNSUPPORTED;  // no token: expert_offsets would stay unwritten
  return from_hip(moe::launch_permute(x, x_dt, topk_ids, T, H, E, k, x_perm, perm_dt, x_perm_scales,
                                      row_map, src_token, expert_counts, expert_offsets, workspace,
                                      static_cast<hipStream_t>(stream)));
}

size_t moe_grouped_swiglu_workspace_size(int64_t rows, int32_t F, moe_dtype dt) {
  if (rows < 0 || F < 1) return 0;
  return align_up(moe::grouped_swiglu_scratch_bytes(rows, F, dt));
}

moe_status moe_grouped_swiglu(const void* x_perm, const void* x_perm_scales, moe_dtype dt,
                              const int32_t* expert_offsets, int64_t rows, int32_t E, int32_t H, int32_t F,
                              const void* w1, const void* w1_scales, const void* w2,
                              const void* w2_scales, void* y_perm, moe_dtype out_dt, void* workspace,
                              size_t workspace_bytes, moe_stream_t stream) {
  if (rows < 0 || rows >= (int64_t{1} << 31) || E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARG;
  moe_status st = check_gemm_shape(dt, H, F);
  if (st != MOE_OK) return st;
  if (dt == MOE_F32 && out_dt != MOE_F32) return MOE_ERR_INVALID_ARG;
  if (!act_dtype_ok(out_dt)) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;  // nothing to do; empty tensors may carry null pointers
  if (!x_perm || !expert_offsets || !w1 || !w2 || !y_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_perm) || !aligned16(y_perm)) return MOE_ERR_INVALID_ARG;  // 16-byte row pieces
  if (low_precision(dt) && (!x_perm_scales || !w1_scales || !w2_scales)) return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < moe_grouped_swiglu_workspace_size(rows, F, dt) || !workspace)
    return MOE_ERR_WORKSPACE;
  return from_hip(moe::launch_grouped_swiglu(x_perm, x_perm_scales, dt, expert_offsets, rows, E, H, F,
                                             w1, w1_scales, w2, w2_scales, y_perm, out_dt, workspace,
                                             static_cast<hipStream_t>(stream)));
}

moe_status moe_unpermute_combine(const void* y_perm, moe_dtype y_dt, const int32_t* row_map,
                                 const float* topk_gates, const void* shared_out, int64_t T, int32_t H,
                                 int32_t k, void* y, moe_dtype out_dt, moe_stream_t stream) {
  if (T < 0 || H < 8 || H % 8 != 0 || k < 1 || k > MOE_MAX_TOPK) return MOE_ERR_INVALID_ARG;
  if (!act_dtype_ok(y_dt) || !act_dtype_ok(out_dt)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;  // nothing to do; empty tensors may carry null pointers
  if (!y_perm || !row_map || !topk_gates || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y_perm) || !aligned16(y) || (shared_out && !aligned16(shared_out)))
    return MOE_ERR_INVALID_ARG;
  return from_hip(moe::launch_combine(y_perm, y_dt, row_map, topk_gates, shared_out, T, H, k, y, out_dt,
                                      static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------------------ fused forward
namespace {

struct ForwardPlan {
  void *logits, *route_ws, *ids, *gates, *counts, *offsets, *row_map, *src, *perm_ws, *x_perm, *x_scales, *xq,
      *xq_scales, *gemm_ws, *y_perm, *sh_ws, *sh_out, *gate_perm;
  size_t bytes;
};

moe_status validate_layer(const moe_layer* L) {
  if (!L) return MOE_ERR_INVALID_ARG;
  moe_status st = check_common(0, L->H, L->E, L->k);
  if (st != MOE_OK) return st;
  if (!act_dtype_ok(L->x_dt) || !act_dtype_ok(L->out_dt)) return MOE_ERR_INVALID_ARG;
  if (L->score != MOE_SOFTMAX && L->score != MOE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (L->gate_in_expert != 0 && L->gate_in_expert != 1) return MOE_ERR_INVALID_ARG;
  if (L->w_dt == MOE_F32 && (L->x_dt != MOE_F32)) return MOE_ERR_INVALID_ARG;
  if (L->w_dt == MOE_BF16 && L->x_dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (low_precision(L->w_dt) && L->x_dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  st = check_gemm_shape(L->w_dt, L->H, L->F);
  if (st != MOE_OK) return st;
  if (L->Fs < 0) return MOE_ERR_INVALID_ARG;
  if (L->Fs > 0) {
    st = check_gemm_shape(L->w_dt, L->H, L->Fs);
    if (st != MOE_OK) return st;
    if (!L->ws1 || !L->ws2) return MOE_ERR_INVALID_ARG;
  }
  if (!L->w_router || !L->w1 || !L->w2) return MOE_ERR_INVALID_ARG;
  if (low_precision(L->w_dt) &&
      (!L->w1_scales || !L->w2_scales || (L->Fs > 0 && (!L->ws1_scales || !L->ws2_scales))))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// The first grouped GEMM gathers its rows straight from x (or from x quantised once per token
// in the e4m3 / MXFP4 paths) through src_token, so the permuted copy x_perm exists only when the
// caller asks for it through moe_debug.
ForwardPlan plan(const moe_layer* L, int64_t T, void* ws, const moe_debug* dbg) {
  const int64_t R = T * L->k;
  const size_t xe = elt_bytes(L->x_dt);
  const bool fp8 = L->w_dt == MOE_FP8_E4M3, fp4 = L->w_dt == MOE_MXFP4;
  Carve c(ws);
  ForwardPlan p{};
  auto pick = [&](void* user, size_t n) { void* w = c.take(n); return user ? user : w; };
  p.logits = pick(dbg ? dbg->logits : nullptr, T * L->E * 4);
  p.route_ws = c.take(moe::route_scratch_bytes(T, L->H, L->E, true));
  p.ids = pick(dbg ? dbg->topk_ids : nullptr, R * 4);
  p.gates = pick(dbg ? dbg->topk_gates : nullptr, R * 4);
  p.counts = pick(dbg ? dbg->expert_counts : nullptr, L->E * 4);
  p.offsets = pick(dbg ? dbg->expert_offsets : nullptr, (L->E + 1) * 4);
  p.row_map = pick(dbg ? dbg->row_map : nullptr, R * 4);
  p.src = pick(dbg ? dbg->src_token : nullptr, R * 4);
  p.perm_ws = c.take(moe::permute_scratch_bytes(T, L->E, L->k));
  // debug-only outputs with no workspace share (the layout must not depend on dbg)
  p.x_perm = dbg ? dbg->x_perm : nullptr;
  p.x_scales = (low_precision(L->w_dt) && p.x_perm) ? dbg->x_perm_scales : nullptr;
  p.xq = fp8 ? c.take(T * L->H) : (fp4 ? c.take(T * (L->H / 2)) : nullptr);
  p.xq_scales = fp8 ? c.take(T * (L->H / 128) * 4) : (fp4 ? c.take(T * (L->H / 32)) : nullptr);
  p.gemm_ws = c.take(moe::grouped_swiglu_scratch_bytes(R, L->F, L->w_dt));
  p.y_perm = pick(dbg ? dbg->y_perm : nullptr, R * L->H * xe);
  if (L->Fs > 0) {
    p.sh_ws = c.take(moe::grouped_swiglu_scratch_bytes(T, L->Fs, L->w_dt));
    p.sh_out = c.take(T * L->H * xe);
  }
  p.gate_perm = L->gate_in_expert ? c.take(R * 4) : nullptr;  // each permuted row's gate
  p.bytes = c.used;
  return p;
}

}  // namespace

size_t moe_workspace_size(const moe_layer* L, int64_t T) {
  if (validate_layer(L) != MOE_OK || T < 0) return 0;
  return plan(L, T, nullptr, nullptr).bytes;
}

moe_status moe_forward(const moe_layer* L, const void* x, int64_t T, void* y, const moe_debug* dbg,
                       void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  moe_status st = validate_layer(L);
  if (st != MOE_OK) return st;
  st = check_common(T, L->H, L->E, L->k);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;  // nothing to do; empty tensors may carry null pointers
  if (!x || !y || !aligned16(x) || !aligned16(y)) return MOE_ERR_INVALID_ARG;
  if (dbg && dbg->x_perm && (!aligned16(dbg->x_perm) || (low_precision(L->w_dt) && !dbg->x_perm_scales)))
    return MOE_ERR_INVALID_ARG;  // e4m3 / MXFP4 rows come with their scales
  const size_t need = plan(L, T, nullptr, nullptr).bytes;
  if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
  ForwardPlan p = plan(L, T, workspace, dbg);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t R = T * L->k;
  const bool fp8 = L->w_dt == MOE_FP8_E4M3, fp4 = L->w_dt == MOE_MXFP4;
  auto ev = [&](int i) -> hipEvent_t { return dbg ? static_cast<hipEvent_t>(dbg->stage_events[i]) : nullptr; };
  auto mark = [&](int i) -> hipError_t { return ev(i) ? hipEventRecord(ev(i), s) : hipSuccess; };

  hipError_t e = mark(0);
  if (e != hipSuccess) return from_hip(e);
  e = moe::launch_route(x, L->x_dt, L->w_router, L->bias, T, L->H, L->E, L->k, L->score,
                                   L->norm_topk ? 1 : 0, static_cast<float*>(p.logits),
                                   static_cast<int32_t*>(p.ids), static_cast<float*>(p.gates), p.route_ws, s);
  if (e == hipSuccess) e = mark(1);
  if (e != hipSuccess) return from_hip(e);
  // gate folded into the experts: dispatch also writes each permuted row's gate, the first GEMM's
  // SwiGLU epilogue scales h by it, and combine sums the k rows unweighted
  float* gate_perm = static_cast<float*>(p.gate_perm);
  e = moe::launch_permute(x, L->x_dt, static_cast<int32_t*>(p.ids), T, L->H, L->E, L->k, p.x_perm,
                          L->w_dt, p.x_scales, static_cast<int32_t*>(p.row_map),
                          static_cast<int32_t*>(p.src), static_cast<int32_t*>(p.counts),
                          static_cast<int32_t*>(p.offsets), p.perm_ws, s,
                          gate_perm ? static_cast<float*>(p.gates) : nullptr, gate_perm);
  // the e4m3 and MXFP4 paths quantise each token once (1x128 / 1x32 blocks); the GEMM gathers its rows
  const void* a = x;
  if (e == hipSuccess && fp8) {
    e = moe::launch_quant_rows_fp8(x, L->x_dt, T, L->H, static_cast<uint8_t*>(p.xq),
                                   static_cast<float*>(p.xq_scales), s);
    a = p.xq;
  } else if (e == hipSuccess && fp4) {
    e = moe::launch_quant_rows_fp4(x, T, L->H, static_cast<uint8_t*>(p.xq), static_cast<uint8_t*>(p.xq_scales), s);
    a = p.xq;
  }
  if (e == hipSuccess) e = mark(2);
  if (e != hipSuccess) return from_hip(e);
  e = moe::launch_grouped_swiglu(a, p.xq_scales, L->w_dt, static_cast<int32_t*>(p.offsets),
                                 R, L->E, L->H, L->F, L->w1, L->w1_scales, L->w2, L->w2_scales, p.y_perm, L->x_dt,
                                 p.gemm_ws, s, ev(3), static_cast<int32_t*>(p.src), gate_perm);
  if (e == hipSuccess) e = mark(4);
  if (e != hipSuccess) return from_hip(e);
  if (L->Fs > 0) {  // every token, unpermuted (quantised like the routed rows in the e4m3 path)
    e = moe::launch_grouped_swiglu(a, p.xq_scales, L->w_dt, nullptr, T, 1, L->H, L->Fs,
                                   L->ws1, L->ws1_scales, L->ws2, L->ws2_scales, p.sh_out, L->x_dt, p.sh_ws, s);
    if (e != hipSuccess) return from_hip(e);
  }
  e = mark(5);
  if (e != hipSuccess) return from_hip(e);
  e = moe::launch_combine(p.y_perm, L->x_dt, static_cast<int32_t*>(p.row_map),
                          gate_perm ? nullptr : static_cast<float*>(p.gates), L->Fs > 0 ? p.sh_out : nullptr, T,
                          L->H, L->k, y, L->out_dt, s);
  if (e == hipSuccess) e = mark(6);
  return from_hip(e);
}

// ------------------------------------------------------------------------------ backward
namespace {

moe::BackwardShape backward_shape(const moe_layer* L, int64_t T) {
  return moe::BackwardShape{T, L->H, L->E, L->k, L->F, L->Fs, L->score == MOE_SIGMOID ? 1 : 0, L->norm_topk ? 1 : 0};
}

size_t backward_bytes(const moe_layer* L, int64_t T) {
  size_t n = 0;
  moe::carve_backward(backward_shape(L, T), L->x_dt == MOE_F32 ? 0 : 1, nullptr, &n);
  return n;
}

}  // namespace

size_t moe_backward_workspace_size(const moe_layer* L, int64_t T) {
  if (validate_layer(L) != MOE_OK || low_precision(L->w_dt) || T < 0) return 0;
  return backward_bytes(L, T);
}

moe_status moe_backward(const moe_layer* L, const void* x, const void* dy, int64_t T, const moe_routing* r,
                        const moe_grads* g, void* const* stage_events, void* workspace, size_t workspace_bytes,
                        moe_stream_t stream) {
  moe_status st = validate_layer(L);
  if (st != MOE_OK) return st;
  if (low_precision(L->w_dt)) return MOE_ERR_UNSUPPORTED;
  st = check_common(T, L->H, L->E, L->k);
  if (st != MOE_OK) return st;
  if (!r || !g) return MOE_ERR_INVALID_ARG;
  auto ok = [](const void* p) { return p != nullptr && aligned16(p); };
  // weight gradients always exist (zero for T = 0); token-sized tensors only when T > 0
  if (!ok(g->dw_router) || !ok(g->dw1) || !ok(g->dw2)) return MOE_ERR_INVALID_ARG;
  if (L->Fs > 0 && (!ok(g->dws1) || !ok(g->dws2))) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!ok(x) || !ok(dy) || !ok(g->dx) || !ok(r->logits) || !ok(r->topk_ids) || !ok(r->topk_gates) ||
                !ok(r->expert_offsets) || !ok(r->row_map) || !ok(r->src_token)))
    return MOE_ERR_INVALID_ARG;
  const size_t need = backward_bytes(L, T);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
  const int dt = L->x_dt == MOE_F32 ? 0 : 1;
  const moe::BackwardShape sh = backward_shape(L, T);
  const moe::BackwardScratch ws = moe::carve_backward(sh, dt, workspace, nullptr);
  moe::BackwardIO io{x,          dy,          L->w_router,   L->w1,          L->w2,      L->ws1,       L->ws2,
                     r->logits,  r->topk_ids, r->topk_gates, r->expert_offsets, r->row_map, r->src_token, g->dx,
                     g->dw_router, g->dw1,    g->dw2,        g->dws1,        g->dws2};
  return from_hip(moe::launch_layer_backward(sh, dt, io, ws, static_cast<hipStream_t>(stream),
                                             reinterpret_cast<hipEvent_t const*>(stage_events)));
}

// ------------------------------------------------------------------------------ no allocation
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, resolved once per device (with that device
// current) and kept.
moe_status static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

moe_status moe_forward_static(const moe_layer* L, const void* x, int64_t T, void* y, const moe_debug* dbg,
                              moe_stream_t stream) {
  moe_status st = validate_layer(L);
  if (st != MOE_OK) return st;
  st = check_common(T, L->H, L->E, L->k);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (plan(L, T, nullptr, nullptr).bytes > MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_TOO_LARGE;
  void* ws = nullptr;
  st = static_scratch(&ws);
  if (st != MOE_OK) return st;
  return moe_forward(L, x, T, y, dbg, ws, MOE_STATIC_SCRATCH_BYTES, stream);
}

}  // extern "C"
