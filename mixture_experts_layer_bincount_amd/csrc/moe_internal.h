// Internal declarations shared by the HIP translation units of the library.
// Not part of the public ABI (that is include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDispatchChunk = 1024;  // assignments per histogram / rank chunk
constexpr int kFp8Group = 128;        // output features per fp8 scale

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

constexpr int kMaxDevices = 64;  // devices whose launch facts are cached

// Compute units of device `dev` (of the current device), queried once per device.
int device_cus(int dev);
int current_device_cus();

// ---------------------------------------------------------------- workspace
struct WsLayout {
  int router_splits;     // split-K factor of the router GEMM
  int nchunks;           // dispatch chunks of dispatch_chunk(k) assignments
  int64_t P_max;         // upper bound of kept assignments
  int64_t H_rows;        // rows of the hidden buffer (P_max + T for a shared expert)
  size_t off_partial;    // fp32 [router_splits, T, E]
  size_t off_wsplit;     // bf16 [3, E_pad, d] split router weights (MFMA router)
  size_t off_chunk_hist; // int32 [nchunks, E]
  size_t off_chunk_base; // int32 [nchunks, E]
  size_t off_perm_token; // int32 [P_max]
  size_t off_perm_w;     // fp32  [P_max]
  size_t off_slot_pos;   // int32 [T*k]
  size_t off_H;          // bf16  [H_rows, d_ff]
  size_t slab_floats;    // floats of the tail slab (0: no tail tile is split)
  size_t off_slab;       // fp32  [slab_floats] partial tiles of split tail tiles (SwiGLU)
  bool grouped_combine;  // moe_forward: grouped output + combine instead of atomics
  size_t off_Yp;         // fp32  [H_rows, d] (grouped_combine only)
  // overflow re-routing (always carved; small unless many rounds)
  size_t off_cand;       // int32 [T, KR] experts by decreasing logit
  size_t off_fin;        // int32 [T*k] expert each assignment holds
  size_t off_req;        // int32 [T*k] the round's requests
  size_t off_nxt;        // int32 [T] next candidate position per token
  size_t off_used;       // int32 [E] fill per expert
  size_t off_room;       // int32 [E] room per expert before the round
  size_t off_cnt2;       // int32 [E] counts of the final grouping (not returned)
  size_t off_shw;        // fp32  [T] shared-expert weights (overflow to shared only)
  size_t total;
};

// Re-routing state carved from the workspace.
struct RerouteWs {
  int32_t* cand;
  int32_t* req;
  int32_t* nxt;
  int32_t* used;
  int32_t* room;
};

// Rounds that can change anything (each asks at least one new expert per
// waiting slot): min(reroute_rounds, E - k); candidates per token needed:
// KR = min(E, k * (1 + rounds)).
int reroute_rounds_eff(const moe_shape& s);
int reroute_candidates(const moe_shape& s);

WsLayout ws_layout(const moe_shape& s);

// Floats of the partial-tile slab the grouped GEMMs may split tail tiles
// through for this shape (0 when neither launch splits): one partial tile
// per workgroup slot of the device, sized to the activation tile.
size_t gemm_slab_floats(const moe_shape& s, int64_t P_max);

// Whether moe_forward combines through a grouped fp32 output and a combine
// kernel (deterministic, no read-modify-write of y) rather than atomics in
// the down projection: yes unless experts average 32 rows or fewer.
bool use_grouped_combine(const moe_shape& s);

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  All are asynchronous.
int router_splits_for(const moe_shape& s);
// Experts padded to the MFMA router's 16-multiple (power of two), or 0 when
// the fp32-activation router runs instead (it handles up to 256 experts).
int router_mfma_epad(const moe_shape& s);
size_t router_split_bytes(const moe_shape& s);
// The MFMA router's split gate planes [3][E_pad][d] bf16 from W_g [d, E] fp32.
hipError_t launch_router_pack(const moe_shape& s, const float* W_g, void* packed, hipStream_t st);
// W_g: the fp32 gate, or (s.router_packed) the packed planes.
hipError_t launch_router_gemm(const moe_shape& s, const void* x, const float* W_g,
                              float* partial, int splits, void* split_ws, hipStream_t st);
// cand (optional): the selection continued to KR experts per token, cand[t,
// 0..KR) by decreasing logit (the ranking overflow re-routing follows).
// topk_idx / topk_w may be NULL when only cand is wanted.
hipError_t launch_topk(const moe_shape& s, const float* partial, int splits,
                       const float* b_g, float* logits, int32_t* topk_idx,
                       float* topk_w, hipStream_t st, int32_t* cand = nullptr, int KR = 0);

hipError_t launch_dispatch(const moe_shape& s, const WsLayout& L,
                           const int32_t* topk_idx, const float* topk_w,
                           int32_t* counts, int32_t* offsets, uint8_t* keep,
                           int32_t* perm_token, float* perm_w, int32_t* slot_pos,
                           int32_t* chunk_hist, int32_t* chunk_base, hipStream_t st,
                           bool hist_ready = false);
// Assignments per dispatch chunk: a multiple of k, so a token's slots share
// one chunk.
int dispatch_chunk(int k);
// Overflow re-routing: fin[T*k] receives each assignment's final expert or
// -1; counts (if given) the router's loads per expert.  R.cand must hold the
// ranked candidates (launch_topk with KR = reroute_candidates(s)).  On
// return chunk_hist holds the per-chunk histogram of fin, ready for
// launch_dispatch(..., hist_ready = true) over fin.
hipError_t launch_reroute(const moe_shape& s, const WsLayout& L, const int32_t* topk_idx,
                          int32_t* fin, int32_t* counts, const RerouteWs& R,
                          int32_t* chunk_hist, int32_t* chunk_base, hipStream_t st);
// shared_w[t] = 1 + sum of the token's dropped topk_w (slot_pos == -1).
hipError_t launch_shared_weights(const moe_shape& s, const int32_t* slot_pos,
                                 const float* topk_w, float* shared_w, hipStream_t st);
// One workgroup: replication, slot loads, LPT placement (see moe_eplb_plan).
hipError_t launch_eplb_plan(const int32_t* counts, int E, int D, int extra, int32_t* replicas,
                            int32_t* slot_device, int32_t* slot_load, int64_t* device_load,
                            hipStream_t st);
hipError_t launch_gather(const moe_shape& s, int64_t P_max, const int32_t* offsets,
                         const int32_t* perm_token, const void* x, void* x_perm,
                         hipStream_t st);

hipError_t launch_fill_zero(float* y, int64_t n, hipStream_t st);

hipError_t launch_expert_ffn(const moe_shape& s, const WsLayout& L,
                             const moe_weights& w, const void* x,
                             const int32_t* offsets, const int32_t* perm_token,
                             const float* perm_w, float* y_perm, float* y,
                             void* H, hipStream_t st, hipEvent_t ev_mid = nullptr,
                             const float* shared_w = nullptr, bool zero_y = false);

// y_perm holds P_max grouped rows, then (with a shared expert) T rows of
// the shared expert's output.
hipError_t launch_combine(const moe_shape& s, int64_t P_max, const float* y_perm,
                          const int32_t* slot_pos, const float* topk_w, float* y,
                          hipStream_t st);

}  // namespace moe
