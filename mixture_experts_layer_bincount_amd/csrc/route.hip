// Router: gate Linear (fp32 accumulate), then softmax / top-k / renormalise.
//
// iopenshare "MoE 混合专家架构" §2.1 (TopKGating: gate Linear without bias,
// top-k, softmax of the kept logits) and the adv12 MoE + EPLB tutorial §3.1 /
// §4.1 (softmax -> topk -> divide by the kept sum; Q1 explains the
// renormalisation).  Both formulations give the same weights; the selection is
// made on the logits (softmax is monotone), ties to the lower expert index.
//
// Stage A: split-K partial dot products written to partial[split][t][e].
//   bf16 activations (router_split_kernel + router_lds_kernel): the fp32
//   gate is split exactly into three bf16 parts and contracted on bf16 MFMA
//   with fp32 accumulation (fp32-GEMM accuracy at matrix-core speed).
//   fp32 activations (router_gemm_kernel): one workgroup = 64 tokens x all
//   experts x one K range; lane = token, each wave owns a contiguous group of
//   experts whose weights it reads with wave-uniform (scalar) loads.
// Stage B (topk_kernel): L lanes per token (L = min(64, pow2 >= E)) sum the
// partials in a fixed order (deterministic), add the bias, and run k rounds of
// a lane-group arg-max on a 64-bit key (ordered logit bits, then ~expert).
#include "moe_internal.h"

namespace moe {
namespace {

template <typename XT>
__device__ __forceinline__ float load_x(const XT* p);
template <>
__device__ __forceinline__ float load_x<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_x<uint16_t>(const uint16_t* p) {
  return bf16_bits_to_f32(*p);
}

template <typename XT, int EPW>
__global__ __launch_bounds__(256) void router_gemm_kernel(
    const XT* __restrict__ x, const float* __restrict__ W_g, float* __restrict__ partial,
    int64_t T, int d, int E, int kchunk) {
  __shared__ float xs[64][65];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int split = blockIdx.y;
  const int kbeg = split * kchunk;
  const int kend = min(d, kbeg + kchunk);
  const int e0 = wave * EPW;

  float acc[EPW];
#pragma unroll
  for (int i = 0; i < EPW; ++i) acc[i] = 0.f;

  const int lrow = tid >> 2;         // token row loaded by this thread
  const int lcol = (tid & 3) * 16;   // 16 k values loaded by this thread
  for (int k0 = kbeg; k0 < kend; k0 += 64) {
    const int64_t t = t0 + lrow;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = k0 + lcol + i;
      xs[lrow][lcol + i] = (t < T && k < kend) ? load_x<XT>(x + t * (int64_t)d + k) : 0.f;
    }
    __syncthreads();
    if (e0 < E) {
      const int kn = min(64, kend - k0);
      for (int kk = 0; kk < kn; ++kk) {
        const float xv = xs[lane][kk];
        const float* wrow = W_g + (size_t)(k0 + kk) * E + e0;
#pragma unroll
        for (int i = 0; i < EPW; ++i)
          if (e0 + i < E) acc[i] = fmaf(xv, wrow[i], acc[i]);
      }
    }
    __syncthreads();
  }
  const int64_t t = t0 + lane;
  if (t < T && e0 < E) {
    float* out = partial + ((int64_t)split * T + t) * E + e0;
#pragma unroll
    for (int i = 0; i < EPW; ++i)
      if (e0 + i < E) out[i] = acc[i];
  }
}

// ---- MFMA router for bf16 activations.
// The fp32 gate weights are split exactly into three bf16 parts,
// W = hi + mid + lo (each part takes the next 8 significand bits; the
// remainders are exact in fp32), stored transposed [3][E_pad][d].  Each
// product of a bf16 activation with a bf16 part is exact in fp32, and the
// MFMA accumulates in fp32, so the logits carry fp32-GEMM accuracy.
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ W_g, int d,
                                                           int E, int E_pad,
                                                           uint16_t* __restrict__ Wp) {
  const int64_t n = (int64_t)E_pad * d;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int e = (int)(i / d);
    const int k = (int)(i % d);
    const float w = (e < E) ? W_g[(int64_t)k * E + e] : 0.f;
    const uint32_t h = f32_to_bf16_bits(w);
    const float r1 = w - bf16_bits_to_f32(h);
    const uint32_t m = f32_to_bf16_bits(r1);
    const float r2 = r1 - bf16_bits_to_f32(m);
    const uint32_t l = f32_to_bf16_bits(r2);
    Wp[i] = (uint16_t)h;
    Wp[n + i] = (uint16_t)m;
    Wp[2 * n + i] = (uint16_t)l;
  }
}

// Blocks of up to 64 experts: every wave covers the block's experts for its
// own 64 rows (with at most 64 experts the activations are read once), and
// the four waves share each 32-deep step of the split weights through LDS;
// blockIdx.z selects the 64-expert block.  The step's 3 x 16*NJ weight rows are
// loaded cooperatively (16 bytes per thread and chunk) and stored in
// fragment order (fragment f = part * NJ + expert tile, lane-major), so a
// wave's fragment read is 64 consecutive 16-byte pieces.  Two LDS buffers:
// step s + 1 is loaded into registers while step s is computed, then
// written to the other buffer; one barrier per step.
template <int NJ>
__global__ __launch_bounds__(256) void router_lds_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ Wp,
                                                         float* __restrict__ partial, int64_t T,
                                                         int d, int E, int E_pad, int ksteps_per) {
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  constexpr int EP = 16 * NJ;
  constexpr int CHUNKS = 3 * EP * 4;                 // 16-byte chunks of one step
  constexpr int CPT = (CHUNKS + 255) / 256;          // per thread
  constexpr int BUF = 3 * NJ * 1024;                 // bytes of one step in LDS
  __shared__ __attribute__((aligned(16))) char sb[2][BUF];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * 256 + wave * 64;
  const int split = blockIdx.y;
  const int k0 = split * ksteps_per * 32;
  const int k1 = min(d, k0 + ksteps_per * 32);  // an empty last split stores zeros
  const int nsteps = k1 > k0 ? (k1 - k0) / 32 : 0;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  const int eb = blockIdx.z * EP;  // first expert of the block
  const uint16_t* arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = min(r0 + i * 16 + fr, T - 1);
    arow[i] = x + t * d + fk;
  }
  const int64_t plane = (int64_t)E_pad * d;
  // this thread's weight chunks: global source and LDS destination
  int bsrc[CPT];  // element offsets into Wp (3 * E_pad * d < 2^31)
  int bdst[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int q = tid + c * 256;
    const int kc = q & 3, pe = q >> 2;           // (part, expert) row, K chunk
    const int part = pe / EP, e = pe % EP;
    bsrc[c] = (int)(part * plane + (int64_t)(eb + e) * d + kc * 8);
    bdst[c] = (part * NJ + e / 16) * 1024 + (kc * 16 + e % 16) * 16;
  }
  f32x4 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // (the staged chunks live in a local array of each step, fully unrolled,
  // so they stay in registers)
  auto load_b = [&](int k, uint4 (&breg)[CPT]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      breg[c] = (CHUNKS % 256 == 0 || tid + c * 256 < CHUNKS)
                    ? *(const uint4*)(Wp + bsrc[c] + k) : make_uint4(0, 0, 0, 0);
  };
  auto store_b = [&](int buf, const uint4 (&breg)[CPT]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (CHUNKS % 256 == 0 || tid + c * 256 < CHUNKS) *(uint4*)(sb[buf] + bdst[c]) = breg[c];
  };
  auto load_a = [&](int k, bf16x8_t (&a)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8_t*)(arow[i] + k);
  };
  auto step = [&](int s, bf16x8_t (&a)[4], bf16x8_t (&an)[4]) __attribute__((always_inline)) {
    const bool more = s + 1 < nsteps;
    uint4 breg[CPT];
    if (more) {
      load_b(k0 + (s + 1) * 32, breg);
      load_a(k0 + (s + 1) * 32, an);
    }
    const char* buf = sb[s & 1];
#pragma unroll
    for (int part = 0; part < 3; ++part)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bf16x8_t b = *(const bf16x8_t*)(buf + (part * NJ + j) * 1024 + lane * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, acc[i][j], 0, 0, 0);
      }
    if (more) store_b((s + 1) & 1, breg);
    __syncthreads();
  };
  if (nsteps > 0) {
    bf16x8_t a0[4], a1[4];
    {
      uint4 breg[CPT];
      load_b(k0, breg);
      store_b(0, breg);
    }
    load_a(k0, a0);
    __syncthreads();
    int s = 0;
    for (; s + 2 <= nsteps; s += 2) {
      step(s, a0, a1);
      step(s + 1, a1, a0);
    }
    if (s < nsteps) step(s, a0, a1);
  }
  // acc[i][j][r]: row i*16 + (lane/16)*4 + r, expert eb + j*16 + lane%16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = r0 + i * 16 + (lane >> 4) * 4 + r;
      if (t >= T) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int e = eb + j * 16 + fr;
        if (e < E) partial[((int64_t)split * T + t) * E + e] = acc[i][j][r];
      }
    }
}

// Ordered key: larger logit -> larger key; equal logits -> lower expert larger.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0 compares equal to +0
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
  return __uint_as_float(u);
}

template <int L>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
#pragma unroll
  for (int off = L / 2; off > 0; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}
template <int L>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = L / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int L, int EPL>
__global__ __launch_bounds__(256) void topk_kernel(
    const float* __restrict__ partial, int splits, const float* __restrict__ b_g,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int64_t T, int E, int k, int32_t* __restrict__ cand, int KR,
    int G, int M) {
  const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = gt / L;
  const int sub = (int)(gt % L);
  const bool live = t < T;
  uint64_t keys[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = sub + i * L;
    keys[i] = 0;
    if (live && e < E) {
      float v = 0.f;
      for (int s = 0; s < splits; ++s) v += partial[((int64_t)s * T + t) * E + e];
      if (b_g) v += b_g[e];
      if (logits) logits[t * E + e] = v;
      keys[i] = topk_key(v, e);
    }
  }
  if (G > 1) {
    // group-limited routing: M rounds of the arg-max over the experts of the
    // groups not yet kept; each round keeps the winner's group (the group
    // with the best maximum; equal maxima: the lower expert, so the lower
    // group).  Then only the kept groups' experts stay selectable.
    const int gs = E / G;
    int grp[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) grp[i] = min((sub + i * L) / gs, 63);  // >= G: padding, key 0
    uint64_t kept = 0;
    for (int m = 0; m < M; ++m) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (!((kept >> grp[i]) & 1) && keys[i] > best) best = keys[i];
      best = group_max_u64<L>(best);
      if (best) kept |= 1ull << ((int)(0xFFFFFFFFu - (uint32_t)best) / gs);
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (!((kept >> grp[i]) & 1)) keys[i] = 0;
  }
  int my_e = -1;
  float my_v = 0.f, vmax = 0.f;
  const int rounds = cand ? max(k, KR) : k;
  for (int j = 0; j < rounds; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) best = keys[i] > best ? keys[i] : best;
    best = group_max_u64<L>(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    const float v = key_value(best);
    if (j == 0) vmax = v;  // the overall maximum (its group is always kept)
    if (sub == j && j < k) { my_e = e; my_v = v; }
    if (cand && live && sub == 0 && j < KR) cand[t * KR + j] = e;
    if ((e % L) == sub) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (i == e / L) keys[i] = 0;
    }
  }
  const float ex = (sub < k) ? expf(my_v - vmax) : 0.f;
  const float den = group_sum<L>(ex);
  if (live && sub < k && topk_idx) {
    topk_idx[t * k + sub] = my_e;
    topk_w[t * k + sub] = ex / den;
  }
}

template <typename XT>
hipError_t router_gemm_dispatch(const moe_shape& s, const XT* x, const float* W_g,
                                float* partial, int splits, hipStream_t st) {
  const int epw_need = (s.E + 3) / 4;
  const int kchunk = ((s.d + splits - 1) / splits + 63) / 64 * 64;
  dim3 grid((unsigned)((s.T + 63) / 64), (unsigned)splits);
#define MOE_RG(EPW)                                                                         \
  if (epw_need <= EPW) {                                                                    \
    router_gemm_kernel<XT, EPW><<<grid, 256, 0, st>>>(x, W_g, partial, s.T, s.d, s.E, kchunk); \
    return hipGetLastError();                                                               \
  }
  MOE_RG(1) MOE_RG(2) MOE_RG(4) MOE_RG(8) MOE_RG(16) MOE_RG(32) MOE_RG(64)
#undef MOE_RG
  return hipErrorInvalidValue;
}

}  // namespace

int router_mfma_epad(const moe_shape& s) {
  if (s.act_dtype != MOE_DT_BF16 || s.d % 32 != 0 || s.E > 1024) return 0;
  int e = 16;
  while (e < s.E) e *= 2;
  return e;
}

size_t router_split_bytes(const moe_shape& s) {
  const int ep = router_mfma_epad(s);
  return ep ? (size_t)3 * ep * s.d * sizeof(uint16_t) : 0;
}

// Expert blocks of the MFMA router (64 experts each beyond 64).
static int router_eblocks(int ep) { return ep <= 64 ? 1 : ep / 64; }

int router_splits_for(const moe_shape& s) {
  const int ep = router_mfma_epad(s);
  if (ep) {
    // about 512 workgroups (2048 waves), K pieces of at least 8 steps of 32
    const int64_t wgs = std::max<int64_t>(1, (s.T + 255) / 256) * router_eblocks(ep);  // T may be 0
    const int ksteps = s.d / 32;
    const int64_t want = (512 + wgs - 1) / wgs;
    return (int)std::max<int64_t>(1, std::min<int64_t>(want, std::max(1, ksteps / 8)));
  }
  const int64_t mt = (s.T + 63) / 64;
  const int kmax = std::max(1, (s.d + 63) / 64);
  return (int)std::max<int64_t>(1, std::min<int64_t>(kmax, (512 + mt - 1) / std::max<int64_t>(mt, 1)));
}

hipError_t launch_router_pack(const moe_shape& s, const float* W_g, void* packed, hipStream_t st) {
  const int ep = router_mfma_epad(s);
  if (!ep) return hipErrorInvalidValue;
  const int64_t n = (int64_t)ep * s.d;
  router_split_kernel<<<(unsigned)std::min<int64_t>((n + 255) / 256, 4096), 256, 0, st>>>(
      W_g, s.d, s.E, ep, (uint16_t*)packed);
  return hipGetLastError();
}

hipError_t launch_router_gemm(const moe_shape& s, const void* x, const float* W_g,
                              float* partial, int splits, void* split_ws, hipStream_t st) {
  const int ep = router_mfma_epad(s);
  if (ep) {
    // the split planes: packed once by the caller (moe_pack_router), or here
    const uint16_t* Wp = s.router_packed ? (const uint16_t*)W_g : (const uint16_t*)split_ws;
    if (!s.router_packed) {
      const hipError_t e = launch_router_pack(s, W_g, split_ws, st);
      if (e != hipSuccess) return e;
    }
    const int ksteps = s.d / 32;
    const int per = (ksteps + splits - 1) / splits;
    dim3 grid((unsigned)((s.T + 255) / 256), (unsigned)splits, (unsigned)router_eblocks(ep));
#define MOE_RL(EP, NJ)                                                                            \
  if (ep == EP) {                                                                                 \
    router_lds_kernel<NJ><<<grid, 256, 0, st>>>((const uint16_t*)x, Wp, partial, s.T, s.d, s.E,  \
                                                ep, per);                                         \
    return hipGetLastError();                                                                     \
  }
    MOE_RL(16, 1) MOE_RL(32, 2) MOE_RL(64, 4) MOE_RL(128, 4) MOE_RL(256, 4) MOE_RL(512, 4)
    MOE_RL(1024, 4)
#undef MOE_RL
    return hipErrorInvalidValue;
  }
  if (s.act_dtype == MOE_DT_F32)
    return router_gemm_dispatch<float>(s, (const float*)x, W_g, partial, splits, st);
  return router_gemm_dispatch<uint16_t>(s, (const uint16_t*)x, W_g, partial, splits, st);
}

hipError_t launch_topk(const moe_shape& s, const float* partial, int splits,
                       const float* b_g, float* logits, int32_t* topk_idx,
                       float* topk_w, hipStream_t st, int32_t* cand, int KR) {
  const int64_t threads_needed = s.T;  // multiplied by L below
#define MOE_TK(LL, EPL)                                                                    \
  {                                                                                        \
    const int64_t n = threads_needed * LL;                                                 \
    topk_kernel<LL, EPL><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(                     \
        partial, splits, b_g, logits, topk_idx, topk_w, s.T, s.E, s.top_k, cand, KR,       \
        s.n_groups, s.topk_groups);                                                        \
    return hipGetLastError();                                                              \
  }
  if (s.E <= 1) MOE_TK(1, 1)
  if (s.E <= 2) MOE_TK(2, 1)
  if (s.E <= 4) MOE_TK(4, 1)
  if (s.E <= 8) MOE_TK(8, 1)
  if (s.E <= 16) MOE_TK(16, 1)
  if (s.E <= 32) MOE_TK(32, 1)
  if (s.E <= 64) MOE_TK(64, 1)
  if (s.E <= 128) MOE_TK(64, 2)
  if (s.E <= 256) MOE_TK(64, 4)
  if (s.E <= 512) MOE_TK(64, 8)
  if (s.E <= 1024) MOE_TK(64, 16)
#undef MOE_TK
  return hipErrorInvalidValue;
}

}  // namespace moe
