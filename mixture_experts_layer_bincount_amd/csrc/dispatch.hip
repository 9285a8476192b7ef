// Load accounting and dispatch.
//
// adv12 MoE + EPLB tutorial §3.2 (bincount of the routed experts) and Q2
// (capacity: an expert takes at most C tokens, the overflow is dropped);
// fde-learning "MoE 并行" (Capacity Factor; Token Batching: group the tokens
// by expert).  The grouped order is deterministic: within an expert, rows
// follow token order, and an assignment is kept iff its rank (the number of
// earlier tokens that chose the same expert) is below C.
//
// Overflow re-routing reuses the same steps, over each round's requests,
// against each expert's remaining room (see launch_reroute).
//
// Three small kernels over the flattened assignments a = t*k + j, in chunks
// of dispatch_chunk(k) <= kDispatchChunk assignments (a multiple of k, so a
// token's slots never straddle two chunks):
//   hist_kernel   per-chunk LDS histogram  -> chunk_hist[c][e]
//   scan_kernel   one workgroup: per-expert exclusive scan over chunks
//                 (chunk_base), counts, kept = min(count, C), and the
//                 exclusive scan of kept over experts (offsets)
//   rank_kernel   stable rank inside the chunk: per wave, lanes with the same
//                 expert are found with ballots over the expert-id bits, the
//                 rank is the popcount of lower such lanes; waves are ordered
//                 through an LDS table.  Writes perm_token / perm_w /
//                 slot_pos / keep.
// When all assignments fit one chunk, one workgroup does all three steps in
// a single launch (dispatch_one_chunk_kernel).
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx, int64_t A,
                                                   int E, int chunk,
                                                   int32_t* __restrict__ chunk_hist) {
  extern __shared__ int32_t h[];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t a0 = (int64_t)blockIdx.x * chunk;
  for (int i = threadIdx.x; i < chunk; i += 256) {
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

// Exclusive scan of expert e's chunk histograms into chunk_base; returns the
// total.  Loads are issued 8 chunks at a time (the chain of dependent adds
// is short; the load latency is what a serial loop would pay per chunk).
__device__ __forceinline__ int32_t scan_chunks(const int32_t* __restrict__ chunk_hist,
                                               int nchunks, int E, int e,
                                               int32_t* __restrict__ chunk_base) {
  int32_t run = 0;
  int c = 0;
  for (; c + 8 <= nchunks; c += 8) {
    int32_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = chunk_hist[(int64_t)(c + i) * E + e];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      chunk_base[(int64_t)(c + i) * E + e] = run;
      run += v[i];
    }
  }
  for (; c < nchunks; ++c) {
    const int32_t v = chunk_hist[(int64_t)c * E + e];
    chunk_base[(int64_t)c * E + e] = run;
    run += v;
  }
  return run;
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
    const int32_t run = scan_chunks(chunk_hist, nchunks, E, e, chunk_base);
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
// this workgroup's chunk calls f(a, r, e, rank) with r its sub-round (a =
// a0 + r * 256 + threadIdx.x), e = ids[a] and rank = the number of earlier
// assignments that chose e (chunk_base holds the earlier chunks' share), or
// f(a, r, -1, -1) when ids[a] is outside [0, E).  Per wave, lanes with the
// same expert are found with ballots over the expert-id bits; the rank is
// the popcount of the lower such lanes, and the waves are ordered through an
// LDS table.  The chunk's ids and bases are loaded up front.  All threads of
// the workgroup must call it; LDS the caller wrote before the call is
// visible inside f.  LDS: 5 * E int32.
constexpr int kSubRounds = kDispatchChunk / 256;

template <class F>
__device__ __forceinline__ void rank_chunk(const int32_t* ids, int64_t A, int E, int ebits,
                                           int chunk, const int32_t* __restrict__ chunk_base,
                                           int32_t* sm, F&& f) {
  int32_t* run = sm;           // [E] rank of the next assignment per expert
  int32_t* cnt = sm + E;       // [4][E] per-wave counts of this sub-round
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t a0 = (int64_t)blockIdx.x * chunk;
  const int64_t a_end = min(a0 + chunk, A);
  int ev[kSubRounds];
#pragma unroll
  for (int r = 0; r < kSubRounds; ++r) {
    const int64_t a = a0 + r * 256 + tid;
    ev[r] = (a < a_end) ? ids[a] : -1;
  }
  const int32_t* base = chunk_base + (int64_t)blockIdx.x * E;
  for (int e = tid; e < E; e += 256) run[e] = base[e];
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int r = 0; r < kSubRounds; ++r) {
    for (int i = tid; i < 4 * E; i += 256) cnt[i] = 0;
    __syncthreads();
    const int64_t a = a0 + r * 256 + tid;
    int e = ev[r];
    const bool valid = (a < a_end) && (unsigned)e < (unsigned)E;
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
      f(a, r, e, pre + rank_w);
    } else if (a < a_end) {
      f(a, r, -1, -1);
    }
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += 256)
      run[e2] += cnt[e2] + cnt[E + e2] + cnt[2 * E + e2] + cnt[3 * E + e2];
    __syncthreads();  // cnt is cleared next; the caller may read run or its LDS after return
  }
}

// Grouped position of every assignment: kept iff its rank is below C.
// Writes perm_token / perm_w / slot_pos / keep; assignments without an
// expert get slot_pos -1 and keep 0.
__global__ __launch_bounds__(256) void rank_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ w, int64_t A, int k, int E,
    int ebits, int chunk, int C, const int32_t* __restrict__ chunk_base,
    const int32_t* __restrict__ offsets, uint8_t* __restrict__ keep,
    int32_t* __restrict__ perm_token, float* __restrict__ perm_w,
    int32_t* __restrict__ slot_pos) {
  extern __shared__ int32_t sm[];
  int32_t* soff = sm + 5 * E;  // [E] the experts' first grouped rows
  for (int e = threadIdx.x; e < E; e += 256) soff[e] = offsets[e];
  float wv[kSubRounds];
  const int64_t a0 = (int64_t)blockIdx.x * chunk;
  const int64_t a_end = min(a0 + chunk, A);
#pragma unroll
  for (int r = 0; r < kSubRounds; ++r) {
    const int64_t a = a0 + r * 256 + threadIdx.x;
    wv[r] = (a < a_end) ? w[a] : 0.f;
  }
  rank_chunk(idx, A, E, ebits, chunk, chunk_base, sm, [&](int64_t a, int r, int e, int32_t rank) {
    const bool kp = e >= 0 && ((C < 0) || (rank < C));
    if (kp) {
      const int32_t pos = soff[e] + rank;
      perm_token[pos] = (int32_t)(a / k);
      perm_w[pos] = wv[r];
      slot_pos[a] = pos;
    } else {
      slot_pos[a] = -1;
    }
    if (keep) keep[a] = kp ? 1 : 0;
  });
}

// All assignments in one chunk (decode-sized batches): the histogram, the
// scan over experts and the stable ranks of the three kernels above in one
// workgroup and one launch.  LDS: (8 E + 256) int32.
__global__ __launch_bounds__(256) void dispatch_one_chunk_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ w, int64_t A, int k, int E,
    int ebits, int chunk, int C, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    uint8_t* __restrict__ keep, int32_t* __restrict__ perm_token, float* __restrict__ perm_w,
    int32_t* __restrict__ slot_pos) {
  extern __shared__ int32_t sm[];
  int32_t* soff = sm + 5 * E;  // [E] the experts' first grouped rows
  int32_t* zb = sm + 6 * E;    // [E] zeros: no earlier chunks
  int32_t* h = sm + 7 * E;     // [E] histogram
  int32_t* ss = sm + 8 * E;    // [256] scan of the per-thread sums
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) {
    h[e] = 0;
    zb[e] = 0;
  }
  __syncthreads();
  for (int64_t a = tid; a < A; a += 256) {
    const int e = idx[a];
    if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  // exclusive scan of kept = min(count, C) over the experts: thread tid owns
  // experts tid * per .. tid * per + per - 1
  const int per = (E + 255) / 256;
  int sum = 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < E) sum += (C < 0) ? h[e] : min(h[e], C);
  }
  ss[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int32_t v = (tid >= off) ? ss[tid - off] : 0;
    __syncthreads();
    ss[tid] += v;
    __syncthreads();
  }
  int32_t run = ss[tid] - sum;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < E) {
      counts[e] = h[e];
      soff[e] = run;
      offsets[e] = run;
      run += (C < 0) ? h[e] : min(h[e], C);
    }
  }
  if (tid == 255) offsets[E] = ss[255];
  float wv[kSubRounds];
#pragma unroll
  for (int r = 0; r < kSubRounds; ++r) {
    const int64_t a = r * 256 + tid;
    wv[r] = (a < A) ? w[a] : 0.f;
  }
  __syncthreads();  // soff, zb written
  rank_chunk(idx, A, E, ebits, chunk, zb, sm, [&](int64_t a, int r, int e, int32_t rank) {
    const bool kp = e >= 0 && ((C < 0) || (rank < C));
    if (kp) {
      const int32_t pos = soff[e] + rank;
      perm_token[pos] = (int32_t)(a / k);
      perm_w[pos] = wv[r];
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
// the expert it holds, or kWaiting.  A round is admit_scan_kernel (one
// workgroup: per-expert chunk bases of the round's requests and the room
// each expert has left) then admit_kernel (per chunk: stable ranks of the
// requests in token order, granted while below the room, then the next
// round's requests of the chunk's tokens and their histogram).  The first
// pass is the same round with every assignment asking for its own expert.
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
  const int32_t run = scan_chunks(chunk_hist, nchunks, E, e, chunk_base);
  if (counts_out) counts_out[e] = run;
  const int32_t u = first ? 0 : used[e];
  const int32_t room = C < 0 ? 0x7FFFFFFF : C - u;
  room_out[e] = room;
  used[e] = u + min(run, room);
}

// Admission of one round, then the chunk's part of what comes next.
//   1. A request (req[a] in [0, E)) is granted iff its rank among the
//      round's requests for its expert (token order, then slot order) is
//      below the room the expert has left.  Grants are staged in LDS.
//   2. For each token of the chunk (its slots all lie in the chunk), in slot
//      order: the slot's new state is the grant, or (first pass) waiting, or
//      its previous state.  Then either
//        next round: each waiting slot asks for the token's next candidate
//        (cand[t] lists the experts by decreasing logit; positions below
//        nxt[t] have been held or asked for), none if no candidate is left;
//        req is rewritten in place (only this workgroup reads its chunk);
//      or the last pass: waiting slots become -1.
//      The chunk's histogram of the new requests (or of the final experts,
//      for the grouping that follows) goes to chunk_hist.
// LDS: 7 * E + kDispatchChunk int32.
__global__ __launch_bounds__(256) void admit_kernel(
    const int32_t* req_in, int64_t A, int E, int ebits, int chunk, int k,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ room, int first_pass,
    int last_pass, const int32_t* __restrict__ cand, int KR, int32_t* __restrict__ fin,
    int32_t* req_out, int32_t* __restrict__ nxt,
    int32_t* __restrict__ chunk_hist) {
  extern __shared__ int32_t sm[];
  int32_t* hist = sm + 5 * E;              // [E]
  int32_t* sroom = sm + 6 * E;             // [E]
  int32_t* grant = sm + 7 * E;             // [chunk] granted expert, or -1
  const int tid = threadIdx.x;
  const int64_t a0 = (int64_t)blockIdx.x * chunk;
  const int n_a = (int)(min(a0 + chunk, A) - a0);
  for (int i = tid; i < n_a; i += 256) grant[i] = -1;
  for (int e = tid; e < E; e += 256) {
    hist[e] = 0;
    sroom[e] = room[e];
  }
  rank_chunk(req_in, A, E, ebits, chunk, chunk_base, sm,
             [&](int64_t a, int, int e, int32_t rank) {
               if (e >= 0 && rank < sroom[e]) grant[a - a0] = e;
             });
  // rank_chunk ends with a barrier: the grants are visible
  const int64_t t0 = a0 / k;
  const int ntok = n_a / k;
  for (int i = tid; i < ntok; i += 256) {
    const int64_t t = t0 + i;
    int n = first_pass ? k : (last_pass ? 0 : nxt[t]);
    for (int j = 0; j < k; ++j) {
      const int64_t a = t * k + j;
      const int g = grant[i * k + j];
      int32_t f = g >= 0 ? g : (first_pass ? kWaiting : fin[a]);
      if (last_pass) {
        if (f == kWaiting) f = -1;
        if (f >= 0) atomicAdd(&hist[f], 1);
      } else {
        int32_t r = -1;
        if (f == kWaiting && n < KR) r = cand[t * KR + n++];
        req_out[a] = r;
        if (r >= 0) atomicAdd(&hist[r], 1);
      }
      fin[a] = f;
    }
    if (!last_pass) nxt[t] = n;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) chunk_hist[(int64_t)blockIdx.x * E + e] = hist[e];
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

int dispatch_chunk(int k) { return kDispatchChunk / k * k; }

hipError_t launch_dispatch(const moe_shape& s, const WsLayout& L, const int32_t* topk_idx,
                           const float* topk_w, int32_t* counts, int32_t* offsets,
                           uint8_t* keep, int32_t* perm_token, float* perm_w,
                           int32_t* slot_pos, int32_t* chunk_hist, int32_t* chunk_base,
                           hipStream_t st, bool hist_ready) {
  const int64_t A = s.T * (int64_t)s.top_k;
  const int chunk = dispatch_chunk(s.top_k);
  int ebits = 0;
  while ((1 << ebits) < s.E) ++ebits;
  if (!hist_ready && L.nchunks == 1) {
    dispatch_one_chunk_kernel<<<1, 256, (8 * s.E + 256) * sizeof(int32_t), st>>>(
        topk_idx, topk_w, A, s.top_k, s.E, ebits, chunk, s.capacity, counts, offsets, keep,
        perm_token, perm_w, slot_pos);
    return hipGetLastError();
  }
  if (!hist_ready)
    hist_kernel<<<L.nchunks, 256, s.E * sizeof(int32_t), st>>>(topk_idx, A, s.E, chunk,
                                                               chunk_hist);
  scan_kernel<<<1, 1024, 0, st>>>(chunk_hist, L.nchunks, s.E, s.capacity, counts, offsets,
                                  chunk_base);
  rank_kernel<<<L.nchunks, 256, 6 * s.E * sizeof(int32_t), st>>>(
      topk_idx, topk_w, A, s.top_k, s.E, ebits, chunk, s.capacity, chunk_base, offsets, keep,
      perm_token, perm_w, slot_pos);
  return hipGetLastError();
}

int reroute_rounds_eff(const moe_shape& s) {
  return std::min(s.reroute_rounds, s.E - s.top_k);
}

int reroute_candidates(const moe_shape& s) {
  return (int)std::min<int64_t>(s.E, (int64_t)s.top_k * (1 + reroute_rounds_eff(s)));
}

hipError_t launch_reroute(const moe_shape& s, const WsLayout& L, const int32_t* topk_idx,
                          int32_t* fin, int32_t* counts, const RerouteWs& R,
                          int32_t* chunk_hist, int32_t* chunk_base, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  const int64_t A = s.T * (int64_t)s.top_k;
  const int chunk = dispatch_chunk(s.top_k);
  int ebits = 0;
  while ((1 << ebits) < s.E) ++ebits;
  const int rounds = s.capacity < 0 ? 0 : reroute_rounds_eff(s);  // nothing overflows
  const int KR = reroute_candidates(s);
  const size_t lds = (7 * s.E + kDispatchChunk) * sizeof(int32_t);
  // first pass: every assignment asks for its own expert
  hist_kernel<<<L.nchunks, 256, s.E * sizeof(int32_t), st>>>(topk_idx, A, s.E, chunk,
                                                             chunk_hist);
  for (int r = 0; r <= rounds; ++r) {
    admit_scan_kernel<<<1, 1024, 0, st>>>(chunk_hist, L.nchunks, s.E, s.capacity, r == 0,
                                          chunk_base, R.used, R.room, r == 0 ? counts : nullptr);
    admit_kernel<<<L.nchunks, 256, lds, st>>>(r == 0 ? topk_idx : R.req, A, s.E, ebits, chunk,
                                              s.top_k, chunk_base, R.room, r == 0, r == rounds,
                                              R.cand, KR, fin, R.req, R.nxt, chunk_hist);
  }
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
