// Load accounting and dispatch.
//
// adv12 MoE + EPLB tutorial §3.2 (bincount of the routed experts) and Q2
// (capacity: an expert takes at most C tokens, the overflow is dropped);
// fde-learning "MoE 并行" (Capacity Factor; Token Batching: group the tokens
// by expert).  The grouped order is deterministic: within an expert, rows
// follow token order, and an assignment is kept iff its rank (the number of
// earlier tokens that chose the same expert) is below C.
//
// Overflow re-routing reuses the same three steps, over each round's
// requests, against each expert's remaining room (see launch_reroute).
//
// Three small kernels over the flattened assignments a = t*k + j, in chunks
// of kDispatchChunk:
//   hist_kernel   per-chunk LDS histogram  -> chunk_hist[c][e]
//   scan_kernel   one workgroup: per-expert exclusive scan over chunks
//                 (chunk_base), counts, kept = min(count, C), and the
//                 exclusive scan of kept over experts (offsets)
//   rank_kernel   stable rank inside the chunk: per wave, lanes with the same
//                 expert are found with ballots over the expert-id bits, the
//                 rank is the popcount of lower such lanes; waves are ordered
//                 through an LDS table.  Writes perm_token / perm_w /
//                 slot_pos / keep.
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx, int64_t A,
                                                   int E, int32_t* __restrict__ chunk_hist) {
  extern __shared__ int32_t h[];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t a0 = (int64_t)blockIdx.x * kDispatchChunk;
  for (int i = threadIdx.x; i < kDispatchChunk; i += 256) {
    const int64_t a = a0 + i;
    if (a < A) {
      const int e = idx[a];
      if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);  // out-of-range ids are ignored
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    chunk_hist[(int64_t)blockIdx.x * E + e] = h[e];
}

// One workgroup of 1024 threads; E <= 1024.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ chunk_hist,
                                                    int nchunks, int E, int C,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ chunk_base) {
  __shared__ int32_t sc[1024];
  const int e = threadIdx.x;
  int32_t kept = 0;
  if (e < E) {
    int32_t run = 0;
    for (int c = 0; c < nchunks; ++c) {
      chunk_base[(int64_t)c * E + e] = run;
      run += chunk_hist[(int64_t)c * E + e];
    }
    counts[e] = run;
    kept = (C < 0) ? run : min(run, C);
  }
  sc[e] = kept;
  __syncthreads();
  // Hillis-Steele inclusive scan over 1024 entries.
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = (e >= off) ? sc[e - off] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  if (e < E) offsets[e + 1] = sc[e];
  if (e == 0) offsets[0] = 0;
}

// Stable ranks inside one chunk of assignments.  For every assignment a of
// this workgroup's chunk (a < A) calls f(a, e, rank) with e = ids[a] and rank
// = the number of earlier assignments that chose e (chunk_base holds the
// earlier chunks' share), or f(a, -1, -1) when ids[a] is outside [0, E).
// Per wave, lanes with the same expert are found with ballots over the
// expert-id bits; the rank is the popcount of the lower such lanes, and the
// waves are ordered through an LDS table.  All threads of the workgroup must
// call it.  LDS: 5 * E int32.
template <class F>
__device__ __forceinline__ void rank_chunk(const int32_t* __restrict__ ids, int64_t A, int E,
                                           int ebits, const int32_t* __restrict__ chunk_base,
                                           int32_t* sm, F&& f) {
  int32_t* run = sm;           // [E] running count of earlier sub-rounds
  int32_t* cnt = sm + E;       // [4][E] per-wave counts of this sub-round
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int e = tid; e < E; e += 256) run[e] = 0;
  const int64_t a0 = (int64_t)blockIdx.x * kDispatchChunk;
  const int32_t* base = chunk_base + (int64_t)blockIdx.x * E;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < kDispatchChunk / 256; ++r) {
    for (int i = tid; i < 4 * E; i += 256) cnt[i] = 0;
    __syncthreads();
    const int64_t a = a0 + r * 256 + tid;
    int e = (a < A) ? ids[a] : 0;
    const bool valid = (a < A) && (unsigned)e < (unsigned)E;
    if (!valid) e = 0;
    uint64_t mask = __ballot(valid);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      mask &= bit ? bb : ~bb;
    }
    const int rank_w = __popcll(mask & lt_mask);
    if (valid && rank_w == 0) cnt[wave * E + e] = __popcll(mask);
    __syncthreads();
    if (valid) {
      int32_t pre = run[e];
      for (int w2 = 0; w2 < wave; ++w2) pre += cnt[w2 * E + e];
      f(a, e, base[e] + pre + rank_w);
    } else if (a < A) {
      f(a, -1, -1);
    }
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += 256)
      run[e2] += cnt[e2] + cnt[E + e2] + cnt[2 * E + e2] + cnt[3 * E + e2];
    __syncthreads();
  }
}

// Grouped position of every assignment: kept iff its rank is below C.
// Writes perm_token / perm_w / slot_pos / keep; assignments without an
// expert get slot_pos -1 and keep 0.
__global__ __launch_bounds__(256) void rank_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ w, int64_t A, int k, int E,
    int ebits, int C, const int32_t* __restrict__ chunk_base,
    const int32_t* __restrict__ offsets, uint8_t* __restrict__ keep,
    int32_t* __restrict__ perm_token, float* __restrict__ perm_w,
    int32_t* __restrict__ slot_pos) {
  extern __shared__ int32_t sm[];
  rank_chunk(idx, A, E, ebits, chunk_base, sm, [&](int64_t a, int e, int32_t rank) {
    const bool kp = e >= 0 && ((C < 0) || (rank < C));
    if (kp) {
      const int32_t pos = offsets[e] + rank;
      perm_token[pos] = (int32_t)(a / k);
      perm_w[pos] = w[a];
      slot_pos[a] = pos;
    } else {
      slot_pos[a] = -1;
    }
    if (keep) keep[a] = kp ? 1 : 0;
  });
}

// ---------------------------------------------------------------- re-routing
// fde-learning "MoE 并行" (推理时的负载均衡): an assignment past its expert's
// capacity goes to its token's next expert.  State per assignment: fin[a] =
// the expert it holds, or kWaiting.  Each round is a request pass (one
// thread per token) followed by an admission pass that is the capacity drop
// again, over the requests, against each expert's remaining room: hist_kernel
// counts the requests per chunk, admit_scan_kernel turns the counts into
// chunk bases and rooms, admit_kernel ranks the requests in token order.
constexpr int32_t kWaiting = -2;

// One workgroup of 1024 threads; E <= 1024.  Per expert: exclusive scan of
// the chunk histograms (chunk_base), the requests n_e, the room left before
// this round (room_out; unlimited for C < 0) and the new fill (used).
// first: used starts at 0 and counts_out (if given) receives n_e.
__global__ __launch_bounds__(1024) void admit_scan_kernel(
    const int32_t* __restrict__ chunk_hist, int nchunks, int E, int C, int first,
    int32_t* __restrict__ chunk_base, int32_t* __restrict__ used,
    int32_t* __restrict__ room_out, int32_t* __restrict__ counts_out) {
  const int e = threadIdx.x;
  if (e >= E) return;
  int32_t run = 0;
  for (int c = 0; c < nchunks; ++c) {
    chunk_base[(int64_t)c * E + e] = run;
    run += chunk_hist[(int64_t)c * E + e];
  }
  if (counts_out) counts_out[e] = run;
  const int32_t u = first ? 0 : used[e];
  const int32_t room = C < 0 ? 0x7FFFFFFF : C - u;
  room_out[e] = room;
  used[e] = u + min(run, room);
}

// Admission: a request is granted iff its rank among the round's requests
// for its expert (token order, then slot order) is below the room left.
// write_all (the first pass): every assignment's state is written, granted
// or waiting; otherwise only granted requests change state.
__global__ __launch_bounds__(256) void admit_kernel(
    const int32_t* __restrict__ req, int64_t A, int E, int ebits,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ room,
    int write_all, int32_t* __restrict__ fin) {
  extern __shared__ int32_t sm[];
  rank_chunk(req, A, E, ebits, chunk_base, sm, [&](int64_t a, int e, int32_t rank) {
    const bool ok = e >= 0 && rank < room[e];
    if (ok) fin[a] = e;
    else if (write_all) fin[a] = kWaiting;
  });
}

// Requests of one round, one thread per token: each waiting slot, in slot
// order, asks for the token's next candidate (cand[t] lists the experts by
// decreasing logit; positions below nxt[t] have been held or asked for).
// A slot with no candidate left asks for nothing (req -1).  final_pass: no
// requests; slots still waiting become -1.
__global__ __launch_bounds__(256) void request_kernel(
    const int32_t* __restrict__ cand, int KR, int64_t T, int k, int first_round,
    int final_pass, int32_t* __restrict__ fin, int32_t* __restrict__ req,
    int32_t* __restrict__ nxt) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  if (final_pass) {
    for (int j = 0; j < k; ++j)
      if (fin[t * k + j] == kWaiting) fin[t * k + j] = -1;
    return;
  }
  int n = first_round ? k : nxt[t];
  for (int j = 0; j < k; ++j) {
    int32_t r = -1;
    if (fin[t * k + j] == kWaiting && n < KR) r = cand[t * KR + n++];
    req[t * k + j] = r;
  }
  nxt[t] = n;
}

// Overflow to the shared expert: shared_w[t] = 1 + the token's dropped
// routing weights, summed in slot order.
__global__ __launch_bounds__(256) void shared_weight_kernel(const int32_t* __restrict__ slot_pos,
                                                            const float* __restrict__ topk_w,
                                                            int64_t T, int k,
                                                            float* __restrict__ shared_w) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  float sw = 1.f;
  for (int j = 0; j < k; ++j)
    if (slot_pos[t * k + j] < 0) sw += topk_w[t * k + j];
  shared_w[t] = sw;
}

template <typename VT>
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ offsets, int E,
                                                     const int32_t* __restrict__ perm_token,
                                                     const VT* __restrict__ x,
                                                     VT* __restrict__ x_perm, int64_t P_max,
                                                     int vec_per_row) {
  const int64_t P = offsets[E];
  const int64_t n = (int64_t)P * vec_per_row;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t p = i / vec_per_row;
    const int c = (int)(i % vec_per_row);
    x_perm[i] = x[(int64_t)perm_token[p] * vec_per_row + c];
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float4* __restrict__ y, int64_t n4,
                                                        float* __restrict__ tail, int ntail) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    y[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0.f;
}

}  // namespace

hipError_t launch_dispatch(const moe_shape& s, const WsLayout& L, const int32_t* topk_idx,
                           const float* topk_w, int32_t* counts, int32_t* offsets,
                           uint8_t* keep, int32_t* perm_token, float* perm_w,
                           int32_t* slot_pos, int32_t* chunk_hist, int32_t* chunk_base,
                           hipStream_t st) {
  const int64_t A = s.T * (int64_t)s.top_k;
  int ebits = 0;
  while ((1 << ebits) < s.E) ++ebits;
  hist_kernel<<<L.nchunks, 256, s.E * sizeof(int32_t), st>>>(topk_idx, A, s.E, chunk_hist);
  scan_kernel<<<1, 1024, 0, st>>>(chunk_hist, L.nchunks, s.E, s.capacity, counts, offsets,
                                  chunk_base);
  rank_kernel<<<L.nchunks, 256, 5 * s.E * sizeof(int32_t), st>>>(
      topk_idx, topk_w, A, s.top_k, s.E, ebits, s.capacity, chunk_base, offsets, keep,
      perm_token, perm_w, slot_pos);
  return hipGetLastError();
}

int reroute_rounds_eff(const moe_shape& s) {
  return std::min(s.reroute_rounds, s.E - s.top_k);
}

int reroute_candidates(const moe_shape& s) {
  return (int)std::min<int64_t>(s.E, (int64_t)s.top_k * (1 + reroute_rounds_eff(s)));
}

hipError_t launch_reroute(const moe_shape& s, const WsLayout& L, const float* logits,
                          const int32_t* topk_idx, int32_t* fin, int32_t* counts,
                          const RerouteWs& R, int32_t* chunk_hist, int32_t* chunk_base,
                          hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  const int64_t A = s.T * (int64_t)s.top_k;
  int ebits = 0;
  while ((1 << ebits) < s.E) ++ebits;
  const int rounds = reroute_rounds_eff(s);
  const int KR = reroute_candidates(s);
  const unsigned tblocks = (unsigned)((s.T + 255) / 256);
  const size_t rank_lds = 5 * s.E * sizeof(int32_t);
  if (rounds > 0) {
    hipError_t err = launch_candidates(s, logits, KR, R.cand, st);
    if (err != hipSuccess) return err;
  }
  // first pass: every assignment asks for its own expert
  hist_kernel<<<L.nchunks, 256, s.E * sizeof(int32_t), st>>>(topk_idx, A, s.E, chunk_hist);
  admit_scan_kernel<<<1, 1024, 0, st>>>(chunk_hist, L.nchunks, s.E, s.capacity, 1, chunk_base,
                                        R.used, R.room, counts);
  admit_kernel<<<L.nchunks, 256, rank_lds, st>>>(topk_idx, A, s.E, ebits, chunk_base, R.room, 1,
                                                 fin);
  for (int r = 0; r < rounds; ++r) {
    request_kernel<<<tblocks, 256, 0, st>>>(R.cand, KR, s.T, s.top_k, r == 0, 0, fin, R.req,
                                            R.nxt);
    hist_kernel<<<L.nchunks, 256, s.E * sizeof(int32_t), st>>>(R.req, A, s.E, chunk_hist);
    admit_scan_kernel<<<1, 1024, 0, st>>>(chunk_hist, L.nchunks, s.E, s.capacity, 0,
                                          chunk_base, R.used, R.room, nullptr);
    admit_kernel<<<L.nchunks, 256, rank_lds, st>>>(R.req, A, s.E, ebits, chunk_base, R.room, 0,
                                                   fin);
  }
  request_kernel<<<tblocks, 256, 0, st>>>(R.cand, KR, s.T, s.top_k, 0, 1, fin, R.req, R.nxt);
  return hipGetLastError();
}

hipError_t launch_shared_weights(const moe_shape& s, const int32_t* slot_pos,
                                 const float* topk_w, float* shared_w, hipStream_t st) {
  shared_weight_kernel<<<(unsigned)((s.T + 255) / 256), 256, 0, st>>>(slot_pos, topk_w, s.T,
                                                                       s.top_k, shared_w);
  return hipGetLastError();
}

hipError_t launch_gather(const moe_shape& s, int64_t P_max, const int32_t* offsets,
                         const int32_t* perm_token, const void* x, void* x_perm,
                         hipStream_t st) {
  const int64_t row_bytes = (int64_t)s.d * (s.act_dtype == MOE_DT_F32 ? 4 : 2);
  if (P_max <= 0) return hipSuccess;  // nothing can be kept
  if (row_bytes % 16 == 0) {
    const int vpr = (int)(row_bytes / 16);
    const int64_t n = P_max * vpr;
    const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 8192);
    gather_kernel<uint4><<<blocks, 256, 0, st>>>(offsets, s.E, perm_token, (const uint4*)x,
                                                 (uint4*)x_perm, P_max, vpr);
  } else {
    const int vpr = (int)(row_bytes / 4);
    const int64_t n = P_max * vpr;
    const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 8192);
    gather_kernel<uint32_t><<<blocks, 256, 0, st>>>(offsets, s.E, perm_token,
                                                     (const uint32_t*)x, (uint32_t*)x_perm,
                                                     P_max, vpr);
  }
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* y, int64_t n, hipStream_t st) {
  const int64_t n4 = n / 4;
  const int ntail = (int)(n - n4 * 4);
  const unsigned blocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>((n4 + 255) / 256, 4096));
  fill_zero_kernel<<<blocks, 256, 0, st>>>((float4*)y, n4, y + n4 * 4, ntail);
  return hipGetLastError();
}

}  // namespace moe
