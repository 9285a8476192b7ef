// Router: gate Linear (fp32 accumulate), then softmax / top-k / renormalise.
//
// iopenshare "MoE 混合专家架构" §2.1 (TopKGating: gate Linear without bias,
// top-k, softmax of the kept logits) and the adv12 MoE + EPLB tutorial §3.1 /
// §4.1 (softmax -> topk -> divide by the kept sum; Q1 explains the
// renormalisation).  Both formulations give the same weights; the selection is
// made on the logits (softmax is monotone), ties to the lower expert index.
//
// Stage A (router_gemm_kernel): split-K partial dot products written to
// partial[split][t][e].  One workgroup = 64 tokens x all experts x one K
// range; lane = token, each wave owns a contiguous group of experts whose
// weights it reads with wave-uniform (scalar) loads.
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
    float* __restrict__ topk_w, int64_t T, int E, int k) {
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
  int my_e = -1;
  float my_v = 0.f, vmax = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) best = keys[i] > best ? keys[i] : best;
    best = group_max_u64<L>(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    const float v = key_value(best);
    if (j == 0) vmax = v;
    if (sub == j) { my_e = e; my_v = v; }
    if ((e % L) == sub) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (i == e / L) keys[i] = 0;
    }
  }
  const float ex = (sub < k) ? expf(my_v - vmax) : 0.f;
  const float den = group_sum<L>(ex);
  if (live && sub < k) {
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

hipError_t launch_router_gemm(const moe_shape& s, const void* x, const float* W_g,
                              float* partial, int splits, hipStream_t st) {
  if (s.act_dtype == MOE_DT_F32)
    return router_gemm_dispatch<float>(s, (const float*)x, W_g, partial, splits, st);
  return router_gemm_dispatch<uint16_t>(s, (const uint16_t*)x, W_g, partial, splits, st);
}

hipError_t launch_topk(const moe_shape& s, const float* partial, int splits,
                       const float* b_g, float* logits, int32_t* topk_idx,
                       float* topk_w, hipStream_t st) {
  const int64_t threads_needed = s.T;  // multiplied by L below
#define MOE_TK(LL, EPL)                                                                    \
  {                                                                                        \
    const int64_t n = threads_needed * LL;                                                 \
    topk_kernel<LL, EPL><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(                     \
        partial, splits, b_g, logits, topk_idx, topk_w, s.T, s.E, s.top_k);                \
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
