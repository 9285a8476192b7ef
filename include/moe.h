/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE FFN layer forward pass.
 *
 * One Mixture-of-Experts FFN layer over one GPU's share of tokens, in five
 * stages (fde-learning "MoE 并行", 核心概念: Router -> dispatch -> expert
 * compute -> gather -> weighted combine; adv12 MoE + EPLB tutorial §3.1):
 *
 *   moe_route       router Linear, softmax, top-k, renormalised weights
 *   moe_reroute     (optional) overflow re-routing of over-capacity assignments
 *   moe_dispatch    per-expert bincount, exclusive-scan offsets, capacity drop,
 *                   grouping permutation (and optionally the gathered rows)
 *   moe_expert_ffn  grouped expert FFN over the grouped rows, with the combine
 *                   fused into its last GEMM (or a grouped output)
 *   moe_combine     weighted sum of each token's k grouped outputs
 *   moe_forward     all of the above on one stream, no host synchronisation
 *
 * Conventions shared by every entry point
 *   - Pointers marked [device] are device pointers (HIP global memory) on the
 *     current device; [host] are host pointers.  All arrays are row-major and
 *     densely packed.  The library never allocates device memory: every buffer,
 *     including the scratch workspace, belongs to the caller.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Device entry points only enqueue work; they return after validating the
 *     arguments and launching.  Results are valid once the stream reaches the
 *     end of the call.  Buffers are borrowed until then.
 *   - Validation is synchronous: MOE_ERR_INVALID for bad shapes or NULL
 *     pointers, MOE_ERR_UNSUPPORTED for a dtype/kind combination that is not
 *     built, MOE_ERR_HIP when a launch fails.  moe_last_error() gives the text.
 *     Faults inside kernels surface at the caller's next stream synchronisation.
 *   - T == 0 is valid: MOE_OK is returned; moe_dispatch and moe_forward then
 *     only write zero counts and offsets, the other entry points launch
 *     nothing.
 *   - NaN/Inf inputs are not checked; results are then unspecified.
 *   - Calls on different streams are independent when they use different
 *     output and workspace buffers.
 *
 * Layouts
 *   x        [T, d]        bf16 (SwiGLU experts) or fp32 (Linear+bias experts)
 *   W_g      [d, E]        fp32, the router Linear stored [in, out]
 *   b_g      [E]           fp32 router bias, optional
 *   W1, W3   [E, d_ff, d]  expert gate / up projections, [out, in] per expert
 *   W2       [E, d, d_ff]  expert down projection, [out, in] per expert
 *   s1, s3   [E, d_ff/128] fp32 scales of fp8, int8 or int4 W1 / W3 (one per 128 output rows)
 *   s2       [E, d/128]    fp32 scales of fp8, int8 or int4 W2
 *            (int4 matrices hold in/2 bytes per row: W1, W3 [E, d_ff, d/2], W2 [E, d, d_ff/2])
 *   W1s, W3s [d_ff, d], W2s [d, d_ff] (+ s1s, s3s [d_ff/128], s2s [d/128])
 *                          the shared expert (one always-on expert, weight 1)
 *   W        [E, d, d]     Linear+bias experts, [out, in];  b [E, d]
 *   topk_idx [T, k] int32  chosen experts, slot 0 the largest logit
 *   topk_w   [T, k] fp32   renormalised routing weights (sum 1 per token)
 *   y        [T, d] fp32   MoE branch output (the residual is the caller's)
 *
 * The [out, in] expert layout is nn.Linear's and the merged
 * [num_experts*ffn_dim, hidden_dim] layout of the MergedExpertLayer on the
 * iopenshare page (§5.2 专家融合与并行): the reduction dimension is contiguous.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_HIP = 3
} moe_status;

typedef enum moe_dtype {
  MOE_DT_F32 = 0,
  MOE_DT_BF16 = 1,
  MOE_DT_FP8_E4M3 = 2, /* OCP FP8 E4M3 (bias 7, max 448, no infinities) */
  MOE_DT_INT8 = 3,     /* symmetric int8 codes -127..127 (iopenshare §5.3: INT8 expert
                          weights); weight = code * scale */
  MOE_DT_INT4 = 4      /* symmetric int4 codes n in -7..7 (iopenshare §5.3: INT4 expert
                          weights; -8 is also accepted), each stored as the nibble
                          c = n + 8; along a weight row every group of 8 inputs takes 4
                          bytes, byte b holding input b in its low nibble and input b + 4
                          in its high nibble; weight = n * scale */
} moe_dtype;

typedef enum moe_expert_kind {
  MOE_EXPERT_LINEAR_BIAS = 0, /* expert(x) = x W^T + b, d -> d (adv12 tutorial §4.1) */
  MOE_EXPERT_SWIGLU = 1       /* expert(x) = (silu(x W1^T) * (x W3^T)) W2^T (iopenshare §5.2) */
} moe_expert_kind;

/* What happens to an assignment past its expert's capacity. */
typedef enum moe_overflow {
  MOE_OVERFLOW_DROP = 0,    /* dropped, adds nothing (tutorial Q2, Mixtral's choice;
                               fde-learning "MoE 并行": overflow takes the residual path) */
  MOE_OVERFLOW_REROUTE = 1, /* re-routed to the token's next-ranked expert with room,
                               in rounds (fde-learning "MoE 并行", 推理时的负载均衡); see
                               moe_reroute */
  MOE_OVERFLOW_SHARED = 2   /* its weight goes to the shared expert, whose weight for the
                               token becomes 1 + the sum of its dropped weights (tutorial
                               Q2, DeepSeek-V3's choice; "MoE 并行" Q4); needs has_shared */
} moe_overflow;

/* Form of the combine inside moe_forward. */
typedef enum moe_combine_form {
  MOE_COMBINE_AUTO = 0,    /* chosen from the shape: FUSED when experts average 32 rows or
                              fewer (decode-sized batches), else GROUPED */
  MOE_COMBINE_GROUPED = 1, /* the down projection writes a grouped fp32 output in the
                              workspace; a combine pass sums each token's rows in slot order
                              (no read-modify-write of y; bit-deterministic) */
  MOE_COMBINE_FUSED = 2    /* the combine is fused into the down projection's epilogue as
                              fp32 atomic adds into a cleared y (the weighted scatter-add;
                              summation order not fixed) */
} moe_combine_form;

/* The problem's parameters (fde-learning "MoE 并行" 关键参数: num_experts, top_k,
 * expert_capacity; tutorial §4.1 MoELayer(d_model, num_experts, top_k)). */
typedef struct moe_shape {
  int64_t T;          /* tokens, >= 0 */
  int32_t d;          /* model width */
  int32_t E;          /* routed experts, 1..1024 (moe_route / moe_forward: up to 256
                         with fp32 x, 1024 with bf16 x) */
  int32_t top_k;      /* experts per token, 1..min(E, 32) */
  int32_t d_ff;       /* expert hidden width (ignored for LINEAR_BIAS) */
  int32_t capacity;   /* tokens per expert, -1 = unlimited (see moe_capacity) */
  int32_t act_dtype;  /* moe_dtype of x: BF16 for SWIGLU, F32 for LINEAR_BIAS */
  int32_t w_dtype;    /* moe_dtype of expert weights: BF16, FP8_E4M3, INT8 or INT4 (SWIGLU),
                         F32 (LINEAR_BIAS) */
  int32_t kind;       /* moe_expert_kind */
  int32_t has_shared; /* 1: add one always-on SWIGLU shared expert (weight 1) */
  int32_t overflow;   /* moe_overflow; 0 (drop) when zero-initialised */
  int32_t reroute_rounds; /* MOE_OVERFLOW_REROUTE: re-routing rounds, 0..1024 */
  int32_t n_groups;    /* group-limited routing: G equal groups of consecutive experts
                          (2..64, dividing E); 0 or 1 = off */
  int32_t topk_groups; /* groups a token may use, 1..n_groups, with
                          top_k <= topk_groups * E / n_groups */
  int32_t combine;     /* moe_combine_form of moe_forward; 0 (auto) when zero-initialised.
                          Part of the shape, so moe_workspace_bytes accounts for it */
  int32_t hidden_split; /* SWIGLU: 0 = the hidden activation h = silu(x W1^T) * (x W3^T)
                           is rounded to bf16 before the down projection (the usual bf16
                           layer); 1 = compensated: h is kept as two bf16 terms, hi =
                           bf16(h) and lo = bf16(h - hi), and the down projection sums
                           both against W2 (h's rounding error about 2^-17 instead of
                           2^-9; twice the down projection's MFMA work and hidden-buffer
                           bytes) */
  int32_t router_packed; /* 1: the W_g argument of moe_route / moe_forward is the packed
                            router buffer written by moe_pack_router, not the fp32 [d, E]
                            matrix (needs bf16 x and d % 32 == 0) */
} moe_shape;

/* Expert weights [device].  Unused members may be NULL. */
typedef struct moe_weights {
  const void* W1;
  const void* W3;
  const void* W2;
  const float* s1;
  const float* s3;
  const float* s2;
  const void* W1s;
  const void* W3s;
  const void* W2s;
  const float* s1s;
  const float* s3s;
  const float* s2s;
  const float* W;
  const float* b;
} moe_weights;

/* Capacity per expert [host]: ceil(cf * T * k / E), evaluated in IEEE double in
 * that order, or -1 (unlimited) when cf <= 0.  The capacity factor is
 * max_tokens_per_expert / (tokens / num_experts) (fde-learning "MoE 并行",
 * Capacity Factor); with top-k routing an expert's tokens are drawn from the
 * T*k assignments.  Kernels only ever see this integer.  Returns -2 on
 * invalid T, E or k. */
int moe_capacity(int64_t T, int32_t E, int32_t k, double cf);

/* Bytes of device workspace moe_dispatch / moe_expert_ffn / moe_forward need
 * for `shape` (a safe upper bound that does not depend on the routing).
 * Returns 0 for an invalid shape.  The workspace must be 256-byte aligned. */
size_t moe_workspace_bytes(const moe_shape* shape);

/* Bytes of the packed router weights moe_pack_router writes for `shape` [host]:
 * three bf16 planes [3][E_pad][d] (E_pad = E rounded up to a power of two, at
 * least 16).  0 when the shape's router cannot use them (fp32 x, or d not a
 * multiple of 32) or the shape is invalid. */
size_t moe_router_packed_bytes(const moe_shape* shape);

/* One-time packing of the router's gate weights (iopenshare §2.1 TopKGating,
 * tutorial §4.1 gate Linear; the packed form is this library's): W_g [d, E]
 * fp32 is split exactly into three bf16 parts, hi + mid + lo = W_g, stored
 * transposed, which the MFMA router multiplies with the bf16 activations and
 * sums in fp32 (the logits keep fp32 accuracy).  moe_route and moe_forward
 * do this split on every call unless shape->router_packed is 1 and W_g points
 * to this buffer.
 *   W_g [device] fp32 [d, E]; packed [device] moe_router_packed_bytes(shape)
 *   bytes, 16-byte aligned, owned by the caller; enqueued on `stream`.
 * MOE_ERR_UNSUPPORTED when the shape's router does not take packed weights. */
moe_status moe_pack_router(const moe_shape* shape, const float* W_g, void* packed,
                           void* stream);

/* Router, stage 1 (iopenshare §2.1 TopKGating; tutorial §3.1 and §4.1 table
 * steps 1-3).  logits = x W_g (+ b_g) in fp32; the k largest logits are kept
 * (slot 0 the largest, equal logits: the lower expert index first, -0 == +0);
 * topk_w[t, j] = exp(l_j - l_max) / sum over the kept j' of exp(l_j' - l_max),
 * i.e. softmax over all experts, keep k, divide by their sum (tutorial Q1).
 * Group-limited routing (n_groups > 1; fde-learning "MoE 并行" Hierarchical
 * Routing, tutorial §5 device-limited routing): a group's score is its largest
 * logit, each token keeps its topk_groups best groups (equal scores: the lower
 * group), and the top-k is taken among those groups' experts only; the
 * weights follow the same rule.
 *   x [device] [T, d] (act_dtype); W_g [device] [d, E] fp32 (or, with
 *   shape->router_packed, moe_pack_router's buffer); b_g [device] [E] or NULL;
 *   logits [device] [T, E] fp32 output or NULL; topk_idx, topk_w [device] outputs;
 *   ws [device] workspace of moe_workspace_bytes(shape) bytes. */
moe_status moe_route(const moe_shape* shape, const void* x, const float* W_g,
                     const float* b_g, float* logits, int32_t* topk_idx,
                     float* topk_w, void* ws, void* stream);

/* Router selection alone, from given fp32 logits [device] [T, E] (the
 * logits-in form of the iopenshare §4.2 safe_topk_routing).  Same selection and
 * weights as moe_route; the selection is a pure function of the logits' bits. */
moe_status moe_route_from_logits(const moe_shape* shape, const float* logits,
                                 int32_t* topk_idx, float* topk_w, void* stream);

/* Overflow re-routing (fde-learning "MoE 并行", 推理时的负载均衡: when an expert
 * is over capacity, its token goes to the next expert; iopenshare §4.2 leaves
 * this step, redistribute, undefined).  Given the router's logits and top-k
 * selection, final_idx[t, j] is the expert assignment (t, j) ends at, or -1:
 *   - first pass: each expert keeps its first `capacity` assignments in token
 *     order (the same keep mask as moe_dispatch);
 *   - then `reroute_rounds` rounds (at most E - k do anything): every
 *     assignment still without an expert, in token order then slot order,
 *     asks for its token's next expert in logit order (equal logits: lower
 *     index first) that the token has neither held nor asked for; each expert
 *     admits the round's requests in that order while it has room;
 *   - assignments still waiting after the last round get -1.
 * A re-routed assignment keeps its routing weight topk_w[t, j].  With
 * capacity == -1 nothing overflows and final_idx = topk_idx.  Pass final_idx
 * to moe_dispatch (with the same shape) to group the rows; its -1 entries
 * are skipped there.  shape->overflow is not consulted.
 *   logits   [device] fp32 [T, E] (as moe_route writes them; the ranking is a pure
 *            function of their bits)
 *   topk_idx [device] int32 [T, k]; final_idx [device] int32 [T, k] output
 *   ws       [device] workspace of moe_workspace_bytes(shape) bytes
 * No host synchronisation. */
moe_status moe_reroute(const moe_shape* shape, const float* logits,
                       const int32_t* topk_idx, int32_t* final_idx, void* ws,
                       void* stream);

/* Load accounting and dispatch (tutorial §3.2 bincount; Q2 capacity and drop;
 * fde-learning Token Batching: group tokens by expert).
 *   counts[e]  [device] int32 [E]   assignments routed to e (before the drop)
 *   offsets    [device] int32 [E+1] exclusive prefix sum of min(counts, C)
 *   keep       [device] uint8 [T*k] 1 if assignment (t, j) is within capacity
 *              (its rank among the tokens choosing e, in token order, is < C), or NULL
 *   perm_token [device] int32 [P_max] token of grouped row p (P = offsets[E] rows used)
 *   perm_w     [device] fp32  [P_max] routing weight of grouped row p
 *   slot_pos   [device] int32 [T*k]   grouped row of (t, j), -1 if dropped
 *   x_perm     [device] [P_max, d] gathered rows x[perm_token[p]], or NULL
 * P_max = T*k without a capacity, min(T*k, E*capacity) with one.
 * The order is deterministic: within an expert, rows follow token order.
 * Expert ids outside [0, E) (such as moe_reroute's -1) stand for assignments
 * without an expert: counted nowhere, slot_pos -1, keep 0.  Capacity is applied
 * to the entries given, whatever shape->overflow says. */
moe_status moe_dispatch(const moe_shape* shape, const int32_t* topk_idx,
                        const float* topk_w, const void* x, int32_t* counts,
                        int32_t* offsets, uint8_t* keep, int32_t* perm_token,
                        float* perm_w, int32_t* slot_pos, void* x_perm,
                        void* ws, void* stream);

/* Grouped expert FFN over the dispatched rows (iopenshare §5.2 merged experts,
 * one GEMM per expert segment; fde-learning Expert 计算).  Row p of expert e's
 * segment [offsets[e], offsets[e+1]) is token perm_token[p].
 *   Exactly one of y_perm / y is non-NULL:
 *   y      [device] fp32 [T, d]: y[t] += perm_w[p] * expert_e(x[t]) for every grouped
 *          row (the combine fused into the last GEMM; y is NOT cleared here;
 *          the shared expert, if any, is added with weight 1 for every token;
 *          MOE_OVERFLOW_SHARED is not available in this form: MOE_ERR_UNSUPPORTED)
 *   y_perm [device] fp32 [P_max (+ T with a shared expert), d]:
 *          y_perm[p] = expert_e(x[perm_token[p]]) (no weight) for p < P_max, and
 *          y_perm[P_max + t] = shared(x[t]) when there is a shared expert; finish
 *          with moe_combine
 *   x is the original [T, d] activation (rows are gathered on load). */
moe_status moe_expert_ffn(const moe_shape* shape, const moe_weights* w,
                          const void* x, const int32_t* offsets,
                          const int32_t* perm_token, const float* perm_w,
                          float* y_perm, float* y, void* ws, void* stream);

/* Combine (MOE 学习笔记 输出聚合: weighted sum of the chosen experts' outputs):
 * y[t] = sum over kept j of topk_w[t, j] * y_perm[slot_pos[t, j]], in slot
 * order, then + y_perm[P_max + t] (weight 1) with a shared expert; dropped
 * assignments (slot_pos == -1) add nothing, except under MOE_OVERFLOW_SHARED,
 * where the shared row's weight is 1 + the sum of the token's dropped topk_w.  y_perm is laid out as
 * moe_expert_ffn writes it; y [device] fp32 [T, d] is overwritten.  The sum
 * order is fixed, so the result is deterministic. */
moe_status moe_combine(const moe_shape* shape, const float* y_perm,
                       const int32_t* slot_pos, const float* topk_w, float* y,
                       void* stream);

/* The whole layer: route, dispatch, grouped FFN, combine, shared expert,
 * with shape->overflow deciding what happens past capacity (re-routing as
 * moe_reroute describes; overflow to the shared expert as moe_combine does).
 * counts stays the router's loads before capacity; offsets are those of the
 * final grouping.
 * shape->combine picks the combine's form (moe_combine_form): fused into the
 * down projection as fp32 atomic adds into a cleared y, or a grouped fp32
 * output in the workspace summed by a combine pass in slot order (no
 * read-modify-write of y, and a deterministic result).  AUTO fuses it when
 * experts average 32 rows or fewer (P_max / E <= 32, decode-sized batches).  y [device] fp32 [T, d] is overwritten.  topk_idx, topk_w,
 * counts, offsets [device] are outputs as above; ws [device] holds
 * moe_workspace_bytes(shape) bytes.  No host synchronisation. */
moe_status moe_forward(const moe_shape* shape, const void* x, const float* W_g,
                       const float* b_g, const moe_weights* w, float* y,
                       int32_t* topk_idx, float* topk_w, int32_t* counts,
                       int32_t* offsets, void* ws, void* stream);

/* Size of the fixed device scratch moe_forward_noalloc uses: 64 MiB, one copy
 * per device the library runs on, held until the process ends. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* moe_forward without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops and harnesses
 * that forbid hipMalloc.  Same arguments, results and errors as moe_forward,
 * minus `ws`: the library's fixed scratch array of MOE_NOALLOC_SCRATCH_BYTES
 * on the current device stands in for it.  Shapes whose
 * moe_workspace_bytes() exceed that size are rejected with
 * MOE_ERR_UNSUPPORTED before anything is launched (decode-sized batches fit:
 * T = 64 at d = 4096, E = 8, d_ff = 14336 needs about 20 MiB).  This entry
 * point calls no allocating routine; the first call on a device looks up the
 * scratch array's device address once.  Every call on a device shares that
 * device's scratch: calls that overlap on one device (other streams, other
 * threads) race and must be serialised by the caller.  Nothing in the
 * scratch needs to start at zero; stage timing is not recorded. */
moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const float* W_g,
                               const float* b_g, const moe_weights* w, float* y,
                               int32_t* topk_idx, float* topk_w, int32_t* counts,
                               int32_t* offsets, void* stream);

/* Load imbalance [host] (tutorial §4.2 expert_imbalance):
 * max(load) / (min(load) + 1e-6).  Returns -1 for E <= 0 or load == NULL. */
double moe_load_imbalance(const int64_t* load, int32_t E);

/* Longest-processing-time-first packing [host] (tutorial §3.3 and §4.3
 * eplb_rebalance): experts in decreasing load order (equal loads: lower expert
 * first) each go to the lightest device (equal: lower device index).
 * assignment [host] int32 [E] receives the device of each expert, bin_load
 * [host] int64 [D] the device loads.  Returns MOE_ERR_INVALID on bad sizes. */
moe_status moe_lpt_pack(const int64_t* load, int32_t E, int32_t D,
                        int32_t* assignment, int64_t* bin_load);

/* Expert placement with hot-expert replication, on the device (fde-learning
 * "MoE 并行" Expert 复制: a popular expert gets a copy on several GPUs; tutorial
 * §3.3 / §4.3 LPT packing, §5 online EPLB).  From the per-expert loads:
 *   1. each expert has one replica; each of `extra` more goes to the expert
 *      with the largest load per replica (equal: the lower expert), at most D
 *      replicas per expert;
 *   2. an expert's load splits evenly over its replicas (the first load % r
 *      take one more); slot s numbers the replicas expert by expert;
 *   3. LPT over the slots: heaviest first (equal: lower expert, then lower
 *      replica), each to the lightest device that holds no copy of the same
 *      expert yet (equal: lower device).
 * With extra = 0 this is moe_lpt_pack.  Runs as one kernel on `stream`: the
 * loads can be moe_forward's counts of the same step, with no host round trip.
 *   counts      [device] int32 [E] loads, >= 0; E in [1, 1024]
 *   D           devices, 1..64;  extra  replicas beyond E, 0..1024, E + extra <= 2048
 *   replicas    [device] int32 [E] output
 *   slot_device [device] int32 [E + extra] output: device of slot s, -1 for
 *               unused slots (when every expert already has D replicas)
 *   slot_load   [device] int32 [E + extra] output: the slot's share of its
 *               expert's load (0 for unused slots)
 *   device_load [device] int64 [D] output
 * MOE_ERR_INVALID for sizes out of range or NULL pointers. */
moe_status moe_eplb_plan(const int32_t* counts, int32_t E, int32_t D, int32_t extra,
                         int32_t* replicas, int32_t* slot_device, int32_t* slot_load,
                         int64_t* device_load, void* stream);

/* Stage timing, for profiling.  While enabled, moe_forward records a HIP event
 * on its stream before its first kernel and after each stage: 0 router GEMM,
 * 1 top-k, 2 dispatch (histogram, scan, rank), 3 clearing y, 4 grouped
 * gate/up GEMM + SwiGLU, 5 grouped down GEMM + combine.  moe_timing_collect
 * [host] waits for the recorded events, writes the summed milliseconds of
 * each stage since the previous collect into ms[0..n) and the number of
 * timed calls into *calls, and returns the number of stages (6).  Disabled
 * by default; enabling adds one event record per stage boundary. */
moe_status moe_timing_enable(int on);
int moe_timing_collect(double* ms, int n, int* calls);
const char* moe_timing_stage_name(int stage);

/* Message of the last non-OK status on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
