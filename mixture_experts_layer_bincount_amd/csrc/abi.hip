// C ABI entry points: argument validation, workspace carving and the launch
// sequences of the MoE layer forward pass.  Host statistics (capacity,
// imbalance, LPT packing) are plain host code.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <numeric>
#include <vector>

#include "moe_internal.h"

namespace moe {
namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

moe_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Shape checks common to every entry point.  `need_ffn` adds the constraints
// of the grouped GEMM tiles.
moe_status check_shape(const moe_shape* s, bool need_ffn) {
  if (!s) return fail(MOE_ERR_INVALID, "shape is NULL");
  if (s->T < 0 || s->T > (int64_t)1 << 30) return fail(MOE_ERR_INVALID, "T=%lld out of range", (long long)s->T);
  if (s->d <= 0) return fail(MOE_ERR_INVALID, "d=%d must be positive", s->d);
  if (s->E < 1 || s->E > 1024) return fail(MOE_ERR_INVALID, "E=%d must be in [1, 1024]", s->E);
  if (s->top_k < 1 || s->top_k > s->E || s->top_k > 32)
    return fail(MOE_ERR_INVALID, "top_k=%d must be in [1, min(E, 32)]", s->top_k);
  if (s->capacity < -1) return fail(MOE_ERR_INVALID, "capacity=%d must be >= -1", s->capacity);
  if (s->overflow < MOE_OVERFLOW_DROP || s->overflow > MOE_OVERFLOW_SHARED)
    return fail(MOE_ERR_INVALID, "overflow=%d is not a moe_overflow", s->overflow);
  if (s->reroute_rounds < 0 || s->reroute_rounds > 1024)
    return fail(MOE_ERR_INVALID, "reroute_rounds=%d must be in [0, 1024]", s->reroute_rounds);
  if (s->overflow == MOE_OVERFLOW_SHARED && !s->has_shared)
    return fail(MOE_ERR_INVALID, "overflow to the shared expert needs has_shared");
  if (s->router_packed < 0 || s->router_packed > 1)
    return fail(MOE_ERR_INVALID, "router_packed=%d must be 0 or 1", s->router_packed);
  if (s->router_packed && !router_mfma_epad(*s))
    return fail(MOE_ERR_UNSUPPORTED, "packed router weights need bf16 x and d %% 32 == 0");
  if (s->hidden_split < 0 || s->hidden_split > 1)
    return fail(MOE_ERR_INVALID, "hidden_split=%d must be 0 or 1", s->hidden_split);
  if (s->combine < MOE_COMBINE_AUTO || s->combine > MOE_COMBINE_FUSED)
    return fail(MOE_ERR_INVALID, "combine=%d is not a moe_combine_form", s->combine);
  if (s->n_groups < 0 || s->n_groups > 64)
    return fail(MOE_ERR_INVALID, "n_groups=%d must be in [0, 64]", s->n_groups);
  if (s->n_groups > 1) {
    if (s->E % s->n_groups != 0)
      return fail(MOE_ERR_INVALID, "n_groups=%d must divide E=%d", s->n_groups, s->E);
    if (s->topk_groups < 1 || s->topk_groups > s->n_groups)
      return fail(MOE_ERR_INVALID, "topk_groups=%d must be in [1, n_groups]", s->topk_groups);
    if ((int64_t)s->top_k > (int64_t)s->topk_groups * (s->E / s->n_groups))
      return fail(MOE_ERR_INVALID, "top_k=%d exceeds the experts of topk_groups groups",
                  s->top_k);
    if (s->overflow == MOE_OVERFLOW_REROUTE)
      return fail(MOE_ERR_UNSUPPORTED, "re-routing is not combined with group-limited routing");
  }
  if (s->T * (int64_t)s->top_k > ((int64_t)1 << 31) - 1)
    return fail(MOE_ERR_INVALID, "T*top_k exceeds int32");
  if (s->kind == MOE_EXPERT_SWIGLU) {
    if (s->act_dtype != MOE_DT_BF16) return fail(MOE_ERR_UNSUPPORTED, "SwiGLU experts need bf16 x");
    if (s->w_dtype != MOE_DT_BF16 && s->w_dtype != MOE_DT_FP8_E4M3 && s->w_dtype != MOE_DT_INT8 &&
        s->w_dtype != MOE_DT_INT4)
      return fail(MOE_ERR_UNSUPPORTED, "SwiGLU experts need bf16, fp8-e4m3, int8 or int4 weights");
    if (need_ffn) {
      if (s->d % 64 != 0) return fail(MOE_ERR_INVALID, "d=%d must be a multiple of 64", s->d);
      if (s->d_ff <= 0 || s->d_ff % 128 != 0)
        return fail(MOE_ERR_INVALID, "d_ff=%d must be a positive multiple of 128", s->d_ff);
      // the grouped GEMM addresses each operand with 32-bit byte offsets
      const int64_t lim = ((int64_t)1 << 31) - 1;
      const int64_t A = s->T * (int64_t)s->top_k;
      const int64_t P_max = s->capacity < 0 ? A : std::min<int64_t>(A, (int64_t)s->E * s->capacity);
      const int64_t H_rows = P_max + (s->has_shared ? s->T : 0);
      if (s->T * (int64_t)s->d * 2 > lim ||
          H_rows * (int64_t)s->d_ff * 2 * (s->hidden_split ? 2 : 1) > lim ||
          (int64_t)s->d * s->d_ff * 2 > lim)
        return fail(MOE_ERR_UNSUPPORTED, "an operand exceeds 2 GiB (x, hidden rows or one expert matrix)");
    }
    if (s->d % 8 != 0) return fail(MOE_ERR_INVALID, "d=%d must be a multiple of 8", s->d);
  } else if (s->kind == MOE_EXPERT_LINEAR_BIAS) {
    if (s->act_dtype != MOE_DT_F32 || s->w_dtype != MOE_DT_F32)
      return fail(MOE_ERR_UNSUPPORTED, "Linear+bias experts need fp32 x and weights");
    if (s->has_shared) return fail(MOE_ERR_UNSUPPORTED, "shared expert needs SwiGLU experts");
  } else {
    return fail(MOE_ERR_INVALID, "unknown expert kind %d", s->kind);
  }
  return MOE_OK;
}

moe_status check_ptr(const void* p, const char* name, size_t align = 4) {
  if (!p) return fail(MOE_ERR_INVALID, "%s is NULL", name);
  if (!aligned(p, align)) return fail(MOE_ERR_INVALID, "%s is not %zu-byte aligned", name, align);
  return MOE_OK;
}

#define MOE_TRY(expr)               \
  do {                              \
    moe_status _st = (expr);        \
    if (_st != MOE_OK) return _st;  \
  } while (0)

moe_status check_weights(const moe_shape* s, const moe_weights* w) {
  if (!w) return fail(MOE_ERR_INVALID, "weights is NULL");
  if (s->kind == MOE_EXPERT_LINEAR_BIAS) {
    MOE_TRY(check_ptr(w->W, "W"));
    MOE_TRY(check_ptr(w->b, "b"));
    return MOE_OK;
  }
  const bool fp8 = s->w_dtype != MOE_DT_BF16;  // quantised codes (8 or 4 bits) + scales
  const size_t al = fp8 ? 8 : 16;
  MOE_TRY(check_ptr(w->W1, "W1", al));
  MOE_TRY(check_ptr(w->W3, "W3", al));
  MOE_TRY(check_ptr(w->W2, "W2", al));
  if (fp8) {
    MOE_TRY(check_ptr(w->s1, "s1"));
    MOE_TRY(check_ptr(w->s3, "s3"));
    MOE_TRY(check_ptr(w->s2, "s2"));
  }
  if (s->has_shared) {
    MOE_TRY(check_ptr(w->W1s, "W1s", al));
    MOE_TRY(check_ptr(w->W3s, "W3s", al));
    MOE_TRY(check_ptr(w->W2s, "W2s", al));
    if (fp8) {
      MOE_TRY(check_ptr(w->s1s, "s1s"));
      MOE_TRY(check_ptr(w->s3s, "s3s"));
      MOE_TRY(check_ptr(w->s2s, "s2s"));
    }
  }
  return MOE_OK;
}

struct Ws {
  RerouteWs rr;
  int32_t* fin;
  int32_t* cnt2;
  float* shw;
  float* partial;
  void* wsplit;
  int32_t* chunk_hist;
  int32_t* chunk_base;
  int32_t* perm_token;
  float* perm_w;
  int32_t* slot_pos;
  void* H;
  float* Yp;
};

Ws carve(const WsLayout& L, void* ws) {
  char* b = (char*)ws;
  return Ws{RerouteWs{(int32_t*)(b + L.off_cand), (int32_t*)(b + L.off_req),
                      (int32_t*)(b + L.off_nxt), (int32_t*)(b + L.off_used),
                      (int32_t*)(b + L.off_room)},
            (int32_t*)(b + L.off_fin), (int32_t*)(b + L.off_cnt2),
            L.off_shw ? (float*)(b + L.off_shw) : nullptr,
            (float*)(b + L.off_partial),     (void*)(b + L.off_wsplit), (int32_t*)(b + L.off_chunk_hist),
            (int32_t*)(b + L.off_chunk_base), (int32_t*)(b + L.off_perm_token),
            (float*)(b + L.off_perm_w),       (int32_t*)(b + L.off_slot_pos),
            (void*)(b + L.off_H),             L.grouped_combine ? (float*)(b + L.off_Yp) : nullptr};
}

// ---- stage timing
constexpr int kStages = 6;
const char* kStageNames[kStages] = {"router_gemm", "topk", "dispatch", "clear_y",
                                    "gate_up_swiglu", "down_combine"};
struct TimedCall {
  hipEvent_t ev[kStages + 1];
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<TimedCall> g_calls;

// Events of one call, or nullptrs when timing is off.
struct CallEvents {
  hipEvent_t ev[kStages + 1] = {};
  bool on = false;
  void begin(hipStream_t st) {
    {
      std::lock_guard<std::mutex> g(g_tmu);
      on = g_timing;
    }
    if (!on) return;
    for (auto& e : ev) hipEventCreate(&e);
    hipEventRecord(ev[0], st);
  }
  void mark(int stage_end, hipStream_t st) {
    if (on) hipEventRecord(ev[stage_end], st);
  }
  void finish() {
    if (!on) return;
    TimedCall c;
    for (int i = 0; i <= kStages; ++i) c.ev[i] = ev[i];
    std::lock_guard<std::mutex> g(g_tmu);
    g_calls.push_back(c);
  }
  hipEvent_t at(int i) const { return on ? ev[i] : nullptr; }
};

}  // namespace

WsLayout ws_layout(const moe_shape& s) {
  WsLayout L{};
  const int64_t A = s.T * (int64_t)s.top_k;
  L.router_splits = router_splits_for(s);
  const int chunk = dispatch_chunk(s.top_k);
  L.nchunks = (int)std::max<int64_t>(1, (A + chunk - 1) / chunk);
  L.P_max = (s.capacity < 0) ? A : std::min<int64_t>(A, (int64_t)s.E * s.capacity);
  L.H_rows = L.P_max + (s.has_shared ? s.T : 0);
  size_t off = 0;
  L.off_partial = off;
  off = align256(off + (size_t)L.router_splits * s.T * s.E * sizeof(float));
  L.off_wsplit = off;
  if (!s.router_packed) off = align256(off + router_split_bytes(s));
  L.off_chunk_hist = off;
  off = align256(off + (size_t)L.nchunks * s.E * sizeof(int32_t));
  L.off_chunk_base = off;
  off = align256(off + (size_t)L.nchunks * s.E * sizeof(int32_t));
  L.off_perm_token = off;
  off = align256(off + (size_t)std::max<int64_t>(L.P_max, 1) * sizeof(int32_t));
  L.off_perm_w = off;
  off = align256(off + (size_t)std::max<int64_t>(L.P_max, 1) * sizeof(float));
  L.off_slot_pos = off;
  off = align256(off + (size_t)std::max<int64_t>(A, 1) * sizeof(int32_t));
  L.off_H = off;
  if (s.kind == MOE_EXPERT_SWIGLU)
    off = align256(off + (size_t)L.H_rows * s.d_ff * 2 * (s.hidden_split ? 2 : 1));
  // partial tiles of split tail tiles (gate/up with a long K, the grouped-
  // output down projection with a long K)
  L.slab_floats = gemm_slab_floats(s, L.P_max);
  L.off_slab = off;
  off = align256(off + L.slab_floats * sizeof(float));
  L.grouped_combine = use_grouped_combine(s);
  L.off_Yp = off;
  if (L.grouped_combine) off = align256(off + (size_t)L.H_rows * s.d * sizeof(float));
  const int64_t KR = reroute_candidates(s);
  L.off_cand = off;
  off = align256(off + (size_t)std::max<int64_t>(s.T * KR, 1) * sizeof(int32_t));
  L.off_fin = off;
  off = align256(off + (size_t)std::max<int64_t>(A, 1) * sizeof(int32_t));
  L.off_req = off;
  off = align256(off + (size_t)std::max<int64_t>(A, 1) * sizeof(int32_t));
  L.off_nxt = off;
  off = align256(off + (size_t)std::max<int64_t>(s.T, 1) * sizeof(int32_t));
  L.off_used = off;
  off = align256(off + (size_t)s.E * sizeof(int32_t));
  L.off_room = off;
  off = align256(off + (size_t)s.E * sizeof(int32_t));
  L.off_cnt2 = off;
  off = align256(off + (size_t)s.E * sizeof(int32_t));
  L.off_shw = 0;  // 0: not carved (offset 0 is the router partials)
  if (s.overflow == MOE_OVERFLOW_SHARED) {
    L.off_shw = off;
    off = align256(off + (size_t)std::max<int64_t>(s.T, 1) * sizeof(float));
  }
  L.total = off;
  return L;
}

bool use_grouped_combine(const moe_shape& s) {
  if (s.combine == MOE_COMBINE_GROUPED) return true;
  if (s.combine == MOE_COMBINE_FUSED || s.kind != MOE_EXPERT_SWIGLU) return false;
  // Few rows per expert (decode): the atomic form, whose down projection may
  // split K over workgroups; otherwise the grouped output (measured faster
  // with many experts per token or a large y, and deterministic).
  const int64_t A = s.T * (int64_t)s.top_k;
  const int64_t P_max = (s.capacity < 0) ? A : std::min<int64_t>(A, (int64_t)s.E * s.capacity);
  return P_max / s.E > 32;
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_capacity(int64_t T, int32_t E, int32_t k, double cf) {
  if (T < 0 || E <= 0 || k <= 0) return -2;
  if (!(cf > 0.0)) return -1;
  const double c = ceil((cf * (double)(T * (int64_t)k)) / (double)E);
  if (c > 2147483647.0) return 2147483647;
  return (int)c;
}

size_t moe_router_packed_bytes(const moe_shape* shape) {
  if (check_shape(shape, false) != MOE_OK) return 0;
  return router_split_bytes(*shape);
}

moe_status moe_pack_router(const moe_shape* shape, const float* W_g, void* packed, void* stream) {
  MOE_TRY(check_shape(shape, false));
  if (!router_mfma_epad(*shape))
    return fail(MOE_ERR_UNSUPPORTED, "this router takes no packed weights (fp32 x or d %% 32 != 0)");
  MOE_TRY(check_ptr(W_g, "W_g"));
  MOE_TRY(check_ptr(packed, "packed", 16));
  return hip_status(launch_router_pack(*shape, W_g, packed, (hipStream_t)stream), "router pack");
}

size_t moe_workspace_bytes(const moe_shape* shape) {
  if (check_shape(shape, false) != MOE_OK) return 0;
  return ws_layout(*shape).total;
}

moe_status moe_route(const moe_shape* shape, const void* x, const float* W_g, const float* b_g,
                     float* logits, int32_t* topk_idx, float* topk_w, void* ws, void* stream) {
  MOE_TRY(check_shape(shape, false));
  const moe_shape& s = *shape;
  if (s.E > 256 && !router_mfma_epad(s))
    return fail(MOE_ERR_UNSUPPORTED, "more than 256 experts need bf16 x with d %% 32 == 0 (E=%d)", s.E);
  if (s.T == 0) return MOE_OK;
  MOE_TRY(check_ptr(x, "x"));
  MOE_TRY(check_ptr(W_g, "W_g"));
  MOE_TRY(check_ptr(topk_idx, "topk_idx"));
  MOE_TRY(check_ptr(topk_w, "topk_w"));
  MOE_TRY(check_ptr(ws, "ws", 256));
  const WsLayout L = ws_layout(s);
  const Ws W = carve(L, ws);
  hipStream_t st = (hipStream_t)stream;
  MOE_TRY(hip_status(launch_router_gemm(s, x, W_g, W.partial, L.router_splits, W.wsplit, st), "router gemm"));
  return hip_status(launch_topk(s, W.partial, L.router_splits, b_g, logits, topk_idx, topk_w, st),
                    "top-k");
}

moe_status moe_route_from_logits(const moe_shape* shape, const float* logits, int32_t* topk_idx,
                                 float* topk_w, void* stream) {
  MOE_TRY(check_shape(shape, false));
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  MOE_TRY(check_ptr(logits, "logits"));
  MOE_TRY(check_ptr(topk_idx, "topk_idx"));
  MOE_TRY(check_ptr(topk_w, "topk_w"));
  return hip_status(launch_topk(s, logits, 1, nullptr, nullptr, topk_idx, topk_w,
                                (hipStream_t)stream),
                    "top-k");
}

moe_status moe_reroute(const moe_shape* shape, const float* logits, const int32_t* topk_idx,
                       int32_t* final_idx, void* ws, void* stream) {
  MOE_TRY(check_shape(shape, false));
  const moe_shape& s = *shape;
  if (s.n_groups > 1)
    return fail(MOE_ERR_UNSUPPORTED, "re-routing is not combined with group-limited routing");
  if (s.T == 0) return MOE_OK;
  MOE_TRY(check_ptr(logits, "logits"));
  MOE_TRY(check_ptr(topk_idx, "topk_idx"));
  MOE_TRY(check_ptr(final_idx, "final_idx"));
  MOE_TRY(check_ptr(ws, "ws", 256));
  const WsLayout L = ws_layout(s);
  const Ws W = carve(L, ws);
  hipStream_t st = (hipStream_t)stream;
  // the ranking past the top-k: the top-k selection continued on the same logits
  if (reroute_rounds_eff(s) > 0 && s.capacity >= 0)
    MOE_TRY(hip_status(launch_topk(s, logits, 1, nullptr, nullptr, nullptr, nullptr, st,
                                   W.rr.cand, reroute_candidates(s)),
                       "candidates"));
  return hip_status(launch_reroute(s, L, topk_idx, final_idx, nullptr, W.rr, W.chunk_hist,
                                   W.chunk_base, st),
                    "reroute");
}

moe_status moe_dispatch(const moe_shape* shape, const int32_t* topk_idx, const float* topk_w,
                        const void* x, int32_t* counts, int32_t* offsets, uint8_t* keep,
                        int32_t* perm_token, float* perm_w, int32_t* slot_pos, void* x_perm,
                        void* ws, void* stream) {
  MOE_TRY(check_shape(shape, false));
  const moe_shape& s = *shape;
  MOE_TRY(check_ptr(counts, "counts"));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(ws, "ws", 256));
  if (s.T > 0) {
    MOE_TRY(check_ptr(topk_idx, "topk_idx"));
    MOE_TRY(check_ptr(topk_w, "topk_w"));
    MOE_TRY(check_ptr(perm_token, "perm_token"));
    MOE_TRY(check_ptr(perm_w, "perm_w"));
    MOE_TRY(check_ptr(slot_pos, "slot_pos"));
    if (x_perm) {
      MOE_TRY(check_ptr(x, "x"));
      const size_t al = ((size_t)s.d * (s.act_dtype == MOE_DT_F32 ? 4 : 2)) % 16 == 0 ? 16 : 4;
      MOE_TRY(check_ptr(x_perm, "x_perm", al));
      MOE_TRY(check_ptr(x, "x", al));
    }
  }
  const WsLayout L = ws_layout(s);
  const Ws W = carve(L, ws);
  hipStream_t st = (hipStream_t)stream;
  MOE_TRY(hip_status(launch_dispatch(s, L, topk_idx, topk_w, counts, offsets, keep, perm_token,
                                     perm_w, slot_pos, W.chunk_hist, W.chunk_base, st),
                     "dispatch"));
  if (x_perm && s.T > 0)
    MOE_TRY(hip_status(launch_gather(s, L.P_max, offsets, perm_token, x, x_perm, st), "gather"));
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_shape* shape, const moe_weights* w, const void* x,
                          const int32_t* offsets, const int32_t* perm_token, const float* perm_w,
                          float* y_perm, float* y, void* ws, void* stream) {
  MOE_TRY(check_shape(shape, true));
  const moe_shape& s = *shape;
  if ((y_perm == nullptr) == (y == nullptr))
    return fail(MOE_ERR_INVALID, "exactly one of y_perm and y must be non-NULL");
  if (s.T == 0) return MOE_OK;
  MOE_TRY(check_weights(&s, w));
  MOE_TRY(check_ptr(x, "x", 16));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(perm_token, "perm_token"));
  MOE_TRY(check_ptr(ws, "ws", 256));
  if (y) {
    if (s.overflow == MOE_OVERFLOW_SHARED)
      return fail(MOE_ERR_UNSUPPORTED,
                  "overflow to the shared expert: use y_perm and moe_combine");
    MOE_TRY(check_ptr(y, "y", 16));
    MOE_TRY(check_ptr(perm_w, "perm_w"));
  } else {
    MOE_TRY(check_ptr(y_perm, "y_perm", 16));
  }
  const WsLayout L = ws_layout(s);
  const Ws W = carve(L, ws);
  return hip_status(launch_expert_ffn(s, L, *w, x, offsets, perm_token, perm_w, y_perm, y, W.H,
                                      (hipStream_t)stream),
                    "expert ffn");
}

moe_status moe_combine(const moe_shape* shape, const float* y_perm, const int32_t* slot_pos,
                       const float* topk_w, float* y, void* stream) {
  MOE_TRY(check_shape(shape, false));
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  MOE_TRY(check_ptr(y_perm, "y_perm"));
  MOE_TRY(check_ptr(slot_pos, "slot_pos"));
  MOE_TRY(check_ptr(topk_w, "topk_w"));
  MOE_TRY(check_ptr(y, "y"));
  return hip_status(launch_combine(s, ws_layout(s).P_max, y_perm, slot_pos, topk_w, y,
                                   (hipStream_t)stream),
                    "combine");
}

}  // extern "C"

namespace moe {
namespace {

// The layer's launch sequence over a workspace `ws` of ws_layout(*shape)
// bytes.  `timed`: record the stage events when stage timing is enabled.
moe_status forward_impl(const moe_shape* shape, const void* x, const float* W_g, const float* b_g,
                        const moe_weights* w, float* y, int32_t* topk_idx, float* topk_w,
                        int32_t* counts, int32_t* offsets, void* ws, void* stream, bool timed) {
  MOE_TRY(check_shape(shape, true));
  const moe_shape& s = *shape;
  if (s.E > 256 && !router_mfma_epad(s))
    return fail(MOE_ERR_UNSUPPORTED, "more than 256 experts need bf16 x with d %% 32 == 0 (E=%d)", s.E);
  MOE_TRY(check_ptr(counts, "counts"));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(ws, "ws", 256));
  hipStream_t st = (hipStream_t)stream;
  const WsLayout L = ws_layout(s);
  const Ws W = carve(L, ws);
  if (s.T == 0) {
    // Nothing routed: counts are zero and offsets all zero.
    return hip_status(launch_dispatch(s, L, topk_idx, topk_w, counts, offsets, nullptr, W.perm_token,
                                      W.perm_w, W.slot_pos, W.chunk_hist, W.chunk_base, st),
                      "dispatch");
  }
  MOE_TRY(check_ptr(x, "x", 16));
  MOE_TRY(check_ptr(W_g, "W_g"));
  MOE_TRY(check_ptr(y, "y", 16));
  MOE_TRY(check_ptr(topk_idx, "topk_idx"));
  MOE_TRY(check_ptr(topk_w, "topk_w"));
  MOE_TRY(check_weights(&s, w));
  CallEvents ce;
  if (timed) ce.begin(st);
  MOE_TRY(hip_status(launch_router_gemm(s, x, W_g, W.partial, L.router_splits, W.wsplit, st), "router gemm"));
  ce.mark(1, st);
  // re-routing: the top-k kernel also lists each token's further candidates
  const bool reroute = s.overflow == MOE_OVERFLOW_REROUTE && s.capacity >= 0 &&
                       reroute_rounds_eff(s) > 0;
  MOE_TRY(hip_status(launch_topk(s, W.partial, L.router_splits, b_g, nullptr, topk_idx, topk_w,
                                 st, reroute ? W.rr.cand : nullptr,
                                 reroute ? reroute_candidates(s) : 0),
                     "top-k"));
  ce.mark(2, st);
  if (reroute) {
    // final experts, then the grouping of those (capacity already respected)
    MOE_TRY(hip_status(launch_reroute(s, L, topk_idx, W.fin, counts, W.rr, W.chunk_hist,
                                      W.chunk_base, st),
                       "reroute"));
    moe_shape s2 = s;
    s2.capacity = -1;
    MOE_TRY(hip_status(launch_dispatch(s2, L, W.fin, topk_w, W.cnt2, offsets, nullptr,
                                       W.perm_token, W.perm_w, W.slot_pos, W.chunk_hist,
                                       W.chunk_base, st, /*hist_ready=*/true),
                       "dispatch"));
  } else {
    MOE_TRY(hip_status(launch_dispatch(s, L, topk_idx, topk_w, counts, offsets, nullptr,
                                       W.perm_token, W.perm_w, W.slot_pos, W.chunk_hist,
                                       W.chunk_base, st),
                       "dispatch"));
  }
  const float* shared_w = nullptr;
  if (s.overflow == MOE_OVERFLOW_SHARED && !L.grouped_combine) {
    MOE_TRY(hip_status(launch_shared_weights(s, W.slot_pos, topk_w, W.shw, st), "shared weights"));
    shared_w = W.shw;
  }
  ce.mark(3, st);
  if (L.grouped_combine) {
    // grouped fp32 output, then the combine kernel writes every element of y
    ce.mark(4, st);
    MOE_TRY(hip_status(launch_expert_ffn(s, L, *w, x, offsets, W.perm_token, W.perm_w, W.Yp,
                                         nullptr, W.H, st, ce.at(5)),
                       "expert ffn"));
    const moe_status r = hip_status(
        launch_combine(s, L.P_max, W.Yp, W.slot_pos, topk_w, y, st), "combine");
    ce.mark(6, st);
    ce.finish();
    return r;
  }
  // y starts at zero for the atomic combine: SwiGLU experts clear it inside
  // the gate/up launch, the Linear+bias ones with a fill kernel
  const bool swiglu = s.kind == MOE_EXPERT_SWIGLU;
  if (!swiglu) MOE_TRY(hip_status(launch_fill_zero(y, s.T * (int64_t)s.d, st), "clear y"));
  ce.mark(4, st);
  const moe_status r = hip_status(launch_expert_ffn(s, L, *w, x, offsets, W.perm_token, W.perm_w,
                                                    nullptr, y, W.H, st, ce.at(5), shared_w,
                                                    /*zero_y=*/swiglu),
                                  "expert ffn");
  ce.mark(6, st);
  ce.finish();
  return r;
}

// ---- the allocation-free variant of moe_forward: a fixed scratch array in
// device memory (one copy per device, held until the process ends) in place
// of the caller's workspace.  Host code never passes the array's name to a
// kernel: it uses the device address hipGetSymbolAddress gives, per device.
constexpr size_t kNoallocScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) char scratch[kNoallocScratchBytes];

struct ScratchAddress {
  std::once_flag once[kMaxDevices];
  hipError_t err[kMaxDevices] = {};
  void* ptr[kMaxDevices] = {};
};
ScratchAddress g_scratch;

// The current device's copy of `scratch`, looked up once per device.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch.once[dev], [&] {
    g_scratch.err[dev] = hipGetSymbolAddress(&g_scratch.ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch.err[dev] != hipSuccess) return g_scratch.err[dev];
  *out = g_scratch.ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace moe

extern "C" {

moe_status moe_forward(const moe_shape* shape, const void* x, const float* W_g, const float* b_g,
                       const moe_weights* w, float* y, int32_t* topk_idx, float* topk_w,
                       int32_t* counts, int32_t* offsets, void* ws, void* stream) {
  return forward_impl(shape, x, W_g, b_g, w, y, topk_idx, topk_w, counts, offsets, ws, stream,
                      /*timed=*/true);
}

moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const float* W_g,
                               const float* b_g, const moe_weights* w, float* y,
                               int32_t* topk_idx, float* topk_w, int32_t* counts,
                               int32_t* offsets, void* stream) {
  MOE_TRY(check_shape(shape, true));
  const size_t need = ws_layout(*shape).total;
  if (need > kNoallocScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_forward_noalloc: this shape needs %zu bytes of scratch, more than the "
                "library's fixed %zu (use moe_forward with a workspace)",
                need, kNoallocScratchBytes);
  void* ws = nullptr;
  MOE_TRY(hip_status(scratch_address(&ws), "scratch address"));
  return forward_impl(shape, x, W_g, b_g, w, y, topk_idx, topk_w, counts, offsets, ws, stream,
                      /*timed=*/false);
}

double moe_load_imbalance(const int64_t* load, int32_t E) {
  if (!load || E <= 0) return -1.0;
  int64_t mx = load[0], mn = load[0];
  for (int i = 1; i < E; ++i) {
    mx = std::max(mx, load[i]);
    mn = std::min(mn, load[i]);
  }
  return (double)mx / ((double)mn + 1e-6);
}

moe_status moe_lpt_pack(const int64_t* load, int32_t E, int32_t D, int32_t* assignment,
                        int64_t* bin_load) {
  if (!load || !assignment || !bin_load || E <= 0 || D <= 0)
    return fail(MOE_ERR_INVALID, "moe_lpt_pack: bad arguments");
  std::vector<int> order(E);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return load[a] > load[b]; });
  for (int i = 0; i < D; ++i) bin_load[i] = 0;
  for (int e : order) {
    int best = 0;
    for (int i = 1; i < D; ++i)
      if (bin_load[i] < bin_load[best]) best = i;
    assignment[e] = best;
    bin_load[best] += load[e];
  }
  return MOE_OK;
}

moe_status moe_eplb_plan(const int32_t* counts, int32_t E, int32_t D, int32_t extra,
                         int32_t* replicas, int32_t* slot_device, int32_t* slot_load,
                         int64_t* device_load, void* stream) {
  if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID, "E=%d must be in [1, 1024]", E);
  if (D < 1 || D > 64) return fail(MOE_ERR_INVALID, "D=%d must be in [1, 64]", D);
  if (extra < 0 || extra > 1024 || E + extra > 2048)
    return fail(MOE_ERR_INVALID, "extra=%d must be in [0, 1024] with E + extra <= 2048", extra);
  MOE_TRY(check_ptr(counts, "counts"));
  MOE_TRY(check_ptr(replicas, "replicas"));
  MOE_TRY(check_ptr(slot_device, "slot_device"));
  MOE_TRY(check_ptr(slot_load, "slot_load"));
  MOE_TRY(check_ptr(device_load, "device_load", 8));
  return hip_status(launch_eplb_plan(counts, E, D, extra, replicas, slot_device, slot_load,
                                     device_load, (hipStream_t)stream),
                    "eplb plan");
}

moe_status moe_timing_enable(int on) {
  std::lock_guard<std::mutex> g(g_tmu);
  g_timing = on != 0;
  return MOE_OK;
}

int moe_timing_collect(double* ms, int n, int* calls) {
  std::vector<TimedCall> cs;
  {
    std::lock_guard<std::mutex> g(g_tmu);
    cs.swap(g_calls);
  }
  std::vector<double> acc(kStages, 0.0);
  for (auto& c : cs) {
    hipEventSynchronize(c.ev[kStages]);
    for (int i = 0; i < kStages; ++i) {
      float t = 0.f;
      if (hipEventElapsedTime(&t, c.ev[i], c.ev[i + 1]) == hipSuccess) acc[i] += t;
    }
    for (auto e : c.ev) hipEventDestroy(e);
  }
  if (ms)
    for (int i = 0; i < std::min(n, kStages); ++i) ms[i] = acc[i];
  if (calls) *calls = (int)cs.size();
  return kStages;
}

const char* moe_timing_stage_name(int stage) {
  return (stage >= 0 && stage < kStages) ? kStageNames[stage] : "";
}

const char* moe_last_error(void) { return g_err; }

}  // extern "C"
