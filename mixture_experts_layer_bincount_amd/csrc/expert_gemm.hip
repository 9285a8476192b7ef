// Grouped expert FFN on bf16 MFMA (gfx950 v_mfma_f32_16x16x32_bf16).
//
// The experts' weights are merged per projection ([E, out, in], the
// MergedExpertLayer layout of the iopenshare page §5.2) and each expert runs
// one GEMM over its contiguous segment of grouped rows, the tile schedule
// being read from the device-side offsets (no host synchronisation).
//
//   MODE_GATEUP  H[p, :] = silu(x_p W1_e^T) * (x_p W3_e^T)       (bf16 out)
//                rows are gathered on load: x_p = x[perm_token[p]]
//   MODE_DOWN    y[perm_token[p], :] += perm_w[p] * (H[p, :] W2_e^T)
//                the combine (MOE 学习笔记 输出聚合: weighted sum of the k
//                expert outputs) fused into the epilogue with fp32 atomics
//   MODE_DOWN_PERM  y_perm[p, :] = H[p, :] W2_e^T                (no weight)
//
// A shared expert (iopenshare §1.4: always-active experts) is expert index E
// with T rows, row t = token t, weight 1, H rows P_max .. P_max + T.
//
// Tile: 128 rows x 256 weight rows x 64 K per step, 256 threads = 2x2 waves,
// each wave 64 rows x 128 weight rows = 4 x 8 MFMA 16x16 tiles.  For
// MODE_GATEUP the 256 weight rows are 128 rows of W1 and the same 128 rows of
// W3, split so that each wave holds matching gate and up columns; the SwiGLU
// is computed in registers.  Operands go global -> registers -> LDS (padded
// rows) -> MFMA fragments, with the next K step's global loads in flight
// during the current step's MFMAs.
#include "moe_internal.h"

namespace moe {
namespace {

enum { MODE_GATEUP = 0, MODE_DOWN = 1, MODE_DOWN_PERM = 2 };

constexpr int BM = 128;
constexpr int BNB = 256;  // weight rows per tile
constexpr int BK = 64;
constexpr int LDSK = BK + 8;  // padded LDS row (bf16 elements)

struct GemmParams {
  const uint16_t* A;          // GATEUP: x [T, K]; DOWN*: H [H_rows, K]
  const int32_t* perm_token;  // [P_max]
  const float* perm_w;        // [P_max]
  const int32_t* offsets;     // [E+1]
  const void* B0;             // GATEUP: W1 [E, N, K]; DOWN*: W2 [E, N, K]
  const void* B1;             // GATEUP: W3 [E, N, K]
  const void* B0s;            // shared expert versions [N, K]
  const void* B1s;
  const float* sc0;           // fp8 scales [E, N/128] (or NULL)
  const float* sc1;
  const float* sc0s;          // shared fp8 scales [N/128]
  const float* sc1s;
  uint16_t* H;                // GATEUP output [H_rows, N]
  float* y;                   // DOWN output [T, N]
  float* y_perm;              // DOWN_PERM output [P_max, N]
  int64_t T;
  int64_t P_max;
  int E;
  int has_shared;
  int K;
  int N;
};

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

// fp8 e4m3 (OCP) -> bf16 bits, exact.  Subnormal codes (exponent field 0)
// are m * 2^-9 and are normalised here.
__device__ __forceinline__ uint32_t e4m3_to_bf16_bits(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 8;
  const uint32_t em = c & 0x7Fu;
  if (em == 0) return s;
  const uint32_t e = em >> 3, m = em & 7u;
  if (e != 0) return s | ((e + 120u) << 7) | (m << 4);
  // subnormal: value = m * 2^-9; m in 1..7
  const int lz = __clz(m) - 29;           // leading zeros within 3 bits
  const uint32_t mn = (m << (lz + 1)) & 7u;  // drop the leading one
  const uint32_t eb = 127u - 9u + (2u - (uint32_t)lz);  // exponent of the leading one
  return s | (eb << 7) | (mn << 4);
}

template <bool FP8>
__device__ __forceinline__ uint4 load_b8(const void* base, int64_t elem_off) {
  if constexpr (!FP8) {
    return *(const uint4*)((const uint16_t*)base + elem_off);
  } else {
    const uint2 q = *(const uint2*)((const uint8_t*)base + elem_off);
    uint4 r;
    r.x = e4m3_to_bf16_bits(q.x & 0xFF) | (e4m3_to_bf16_bits((q.x >> 8) & 0xFF) << 16);
    r.y = e4m3_to_bf16_bits((q.x >> 16) & 0xFF) | (e4m3_to_bf16_bits(q.x >> 24) << 16);
    r.z = e4m3_to_bf16_bits(q.y & 0xFF) | (e4m3_to_bf16_bits((q.y >> 8) & 0xFF) << 16);
    r.w = e4m3_to_bf16_bits((q.y >> 16) & 0xFF) | (e4m3_to_bf16_bits(q.y >> 24) << 16);
    return r;
  }
}

template <int MODE, bool FP8>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDSK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BNB * LDSK];
  __shared__ int s_scan[8];
  __shared__ int s_e, s_m0, s_rows, s_seg;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nseg = p.E + (p.has_shared ? 1 : 0);

  // ---- map this workgroup's m-slot to (expert, first row) from the offsets.
  {
    const int per = (nseg + 255) / 256;
    const int e_lo = tid * per;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int e = e_lo + i;
      if (e < nseg) {
        const int64_t rows = (e < p.E) ? (int64_t)(p.offsets[e + 1] - p.offsets[e]) : p.T;
        local += (int)((rows + BM - 1) / BM);
      }
    }
    const int incl = wave_incl_scan(local, lane);
    if (lane == 63) s_scan[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w2 = 0; w2 < wave; ++w2) before += s_scan[w2];
    const int total = s_scan[0] + s_scan[1] + s_scan[2] + s_scan[3];
    int excl = before + incl - local;
    const int slot = blockIdx.y;
    if (tid == 0 && slot >= total) s_e = -1;
    if (slot >= excl && slot < excl + local) {
      for (int i = 0; i < per; ++i) {
        const int e = e_lo + i;
        if (e >= nseg) break;
        const int64_t rows = (e < p.E) ? (int64_t)(p.offsets[e + 1] - p.offsets[e]) : p.T;
        const int nt = (int)((rows + BM - 1) / BM);
        if (slot < excl + nt) {
          s_e = e;
          s_m0 = (slot - excl) * BM;
          s_rows = (int)rows;
          s_seg = (e < p.E) ? p.offsets[e] : 0;
          break;
        }
        excl += nt;
      }
    }
    __syncthreads();
  }
  const int e = s_e;
  if (e < 0) return;
  const int m0 = s_m0, rows = s_rows, seg = s_seg;
  const bool shared_e = (e == p.E);
  const int K = p.K, N = p.N;

  // ---- per-thread global source rows.
  const int lr = tid >> 3;        // 0..31
  const int kc = (tid & 7) * 8;   // bf16 element offset within BK
  const uint16_t* a_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = min(m0 + lr + 32 * i, rows - 1);
    int64_t arow;
    if (MODE == MODE_GATEUP)
      arow = shared_e ? (int64_t)m : (int64_t)p.perm_token[seg + m];
    else
      arow = shared_e ? p.P_max + m : (int64_t)seg + m;
    a_src[i] = p.A + arow * K + kc;
  }
  const int n0 = (MODE == MODE_GATEUP) ? blockIdx.x * (BNB / 2) : blockIdx.x * BNB;
  const void* b_base[8];
  int64_t b_off[8];
  const int64_t estride = (int64_t)N * K;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int br = lr + 32 * i;  // 0..255
    if (MODE == MODE_GATEUP) {
      const bool up = br >= BNB / 2;
      const int n = n0 + (up ? br - BNB / 2 : br);
      b_base[i] = shared_e ? (up ? p.B1s : p.B0s) : (up ? p.B1 : p.B0);
      b_off[i] = (shared_e ? 0 : (int64_t)e * estride) + (int64_t)n * K + kc;
    } else {
      b_base[i] = shared_e ? p.B0s : p.B0;
      b_off[i] = (shared_e ? 0 : (int64_t)e * estride) + (int64_t)(n0 + br) * K + kc;
    }
  }

  // ---- wave tile
  const int wm = wave >> 1, wn = wave & 1;
  int brow[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (MODE == MODE_GATEUP)
      brow[j] = (j < 4) ? (wn * 64 + j * 16) : (BNB / 2 + wn * 64 + (j - 4) * 16);
    else
      brow[j] = wn * 128 + j * 16;
  }
  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 ra[4], rb[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) ra[i] = *(const uint4*)(a_src[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) rb[i] = load_b8<FP8>(b_base[i], b_off[i]);

  const int nk = K / BK;
  const int frow = lane & 15;
  const int fk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) *(uint4*)&As[(lr + 32 * i) * LDSK + kc] = ra[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) *(uint4*)&Bs[(lr + 32 * i) * LDSK + kc] = rb[i];
    __syncthreads();
    if (kt + 1 < nk) {
      const int64_t ko = (int64_t)(kt + 1) * BK;
#pragma unroll
      for (int i = 0; i < 4; ++i) ra[i] = *(const uint4*)(a_src[i] + ko);
#pragma unroll
      for (int i = 0; i < 8; ++i) rb[i] = load_b8<FP8>(b_base[i], b_off[i] + ko);
    }
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8 af[4], bfr[8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *(const bf16x8*)&As[(wm * 64 + i * 16 + frow) * LDSK + kk + fk];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        bfr[j] = *(const bf16x8*)&Bs[(brow[j] + frow) * LDSK + kk + fk];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue.  acc[i][j][r] is row wm*64 + i*16 + (lane>>4)*4 + r,
  // weight row brow[j] + (lane & 15).
  const int col_l = lane & 15;
  const int row_l = (lane >> 4) * 4;
  if (MODE == MODE_GATEUP) {
    const int64_t hbase = shared_e ? p.P_max : (int64_t)seg;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + j * 16 + col_l;
      float sg = 1.f, su = 1.f;
      if (FP8) {
        const int gi = n / kFp8Group;
        sg = shared_e ? p.sc0s[gi] : p.sc0[(int64_t)e * (N / kFp8Group) + gi];
        su = shared_e ? p.sc1s[gi] : p.sc1[(int64_t)e * (N / kFp8Group) + gi];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm * 64 + i * 16 + row_l + r;
          if (m < rows) {
            const float a = acc[i][j][r] * sg;
            const float g = acc[i][j + 4][r] * su;
            const float h = a / (1.f + __expf(-a)) * g;
            p.H[(hbase + m) * N + n] = (uint16_t)f32_to_bf16_bits(h);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 64 + i * 16 + row_l + r;
        if (m >= rows) continue;
        float wgt = 1.f;
        int64_t orow;
        if (MODE == MODE_DOWN) {
          if (shared_e) {
            orow = m;
          } else {
            orow = p.perm_token[seg + m];
            wgt = p.perm_w[seg + m];
          }
        } else {
          orow = (int64_t)seg + m;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int n = n0 + brow[j] + col_l;
          float v = acc[i][j][r];
          if (FP8) {
            const int gi = n / kFp8Group;
            v *= shared_e ? p.sc0s[gi] : p.sc0[(int64_t)e * (N / kFp8Group) + gi];
          }
          if (MODE == MODE_DOWN)
            atomicAdd(&p.y[orow * N + n], wgt * v);
          else
            p.y_perm[orow * N + n] = v;
        }
      }
    }
  }
}

// Linear+bias experts in fp32 (the tutorial's nn.Linear(d, d) experts, §4.1).
// One thread per (grouped row, output feature); MODE_DOWN adds w * out into y.
template <int MODE>
__global__ __launch_bounds__(256) void linear_bias_kernel(
    const float* __restrict__ x, const float* __restrict__ W, const float* __restrict__ b,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm_token,
    const float* __restrict__ perm_w, float* __restrict__ y, float* __restrict__ y_perm,
    int E, int d, int64_t P_max) {
  const int64_t P = offsets[E];
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < P * d;
       i += (int64_t)gridDim.x * 256) {
    const int64_t pr = i / d;
    const int n = (int)(i % d);
    int lo = 0, hi = E;  // find e with offsets[e] <= pr < offsets[e+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (offsets[mid] <= pr) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int64_t t = perm_token[pr];
    const float* wr = W + ((int64_t)e * d + n) * d;
    const float* xr = x + t * d;
    float acc = 0.f;
    for (int c = 0; c < d; ++c) acc = fmaf(xr[c], wr[c], acc);
    acc += b[(int64_t)e * d + n];
    if (MODE == MODE_DOWN)
      atomicAdd(&y[t * d + n], perm_w[pr] * acc);
    else
      y_perm[pr * d + n] = acc;
  }
}

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ slot_pos,
                                                      const float* __restrict__ topk_w,
                                                      float* __restrict__ y, int64_t T, int k,
                                                      int d) {
  const int64_t n = T * d;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / d;
    const int c = (int)(i % d);
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const int32_t pos = slot_pos[t * k + j];
      if (pos >= 0) acc += topk_w[t * k + j] * y_perm[(int64_t)pos * d + c];
    }
    y[i] = acc;
  }
}

template <int MODE, bool FP8>
hipError_t launch_gemm(const GemmParams& p, int64_t mtiles_max, int ntiles, hipStream_t st) {
  if (mtiles_max <= 0 || ntiles <= 0) return hipSuccess;
  dim3 grid((unsigned)ntiles, (unsigned)mtiles_max);
  grouped_gemm_kernel<MODE, FP8><<<grid, 256, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expert_ffn(const moe_shape& s, const WsLayout& L, const moe_weights& w,
                             const void* x, const int32_t* offsets, const int32_t* perm_token,
                             const float* perm_w, float* y_perm, float* y, void* H,
                             hipStream_t st, hipEvent_t ev_mid) {
  if (s.kind == MOE_EXPERT_LINEAR_BIAS) {
    const int64_t n = L.P_max * s.d;
    const unsigned blocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 4096));
    if (y)
      linear_bias_kernel<MODE_DOWN><<<blocks, 256, 0, st>>>((const float*)x, w.W, w.b, offsets,
                                                            perm_token, perm_w, y, nullptr, s.E,
                                                            s.d, L.P_max);
    else
      linear_bias_kernel<MODE_DOWN_PERM><<<blocks, 256, 0, st>>>((const float*)x, w.W, w.b,
                                                                 offsets, perm_token, perm_w,
                                                                 nullptr, y_perm, s.E, s.d,
                                                                 L.P_max);
    return hipGetLastError();
  }
  const bool fp8 = s.w_dtype == MOE_DT_FP8_E4M3;
  const int has_sh = s.has_shared ? 1 : 0;
  // Upper bound of m-tiles: sum_e ceil(rows_e / BM) <= P_max / BM + E (+ shared).
  const int64_t mt_max = (L.P_max + BM - 1) / BM + s.E + (has_sh ? (s.T + BM - 1) / BM : 0);

  GemmParams g{};
  g.perm_token = perm_token;
  g.perm_w = perm_w;
  g.offsets = offsets;
  g.T = s.T;
  g.P_max = L.P_max;
  g.E = s.E;
  g.has_shared = has_sh;

  // gate / up
  g.A = (const uint16_t*)x;
  g.B0 = w.W1; g.B1 = w.W3; g.B0s = w.W1s; g.B1s = w.W3s;
  g.sc0 = w.s1; g.sc1 = w.s3; g.sc0s = w.s1s; g.sc1s = w.s3s;
  g.H = (uint16_t*)H;
  g.K = s.d;
  g.N = s.d_ff;
  hipError_t err = fp8 ? launch_gemm<MODE_GATEUP, true>(g, mt_max, s.d_ff / (BNB / 2), st)
                       : launch_gemm<MODE_GATEUP, false>(g, mt_max, s.d_ff / (BNB / 2), st);
  if (err != hipSuccess) return err;
  if (ev_mid) {
    err = hipEventRecord(ev_mid, st);
    if (err != hipSuccess) return err;
  }

  // down (+ combine)
  GemmParams g2 = g;
  g2.A = (const uint16_t*)H;
  g2.B0 = w.W2; g2.B1 = nullptr; g2.B0s = w.W2s; g2.B1s = nullptr;
  g2.sc0 = w.s2; g2.sc1 = nullptr; g2.sc0s = w.s2s; g2.sc1s = nullptr;
  g2.H = nullptr;
  g2.y = y;
  g2.y_perm = y_perm;
  g2.K = s.d_ff;
  g2.N = s.d;
  if (y)
    return fp8 ? launch_gemm<MODE_DOWN, true>(g2, mt_max, s.d / BNB, st)
               : launch_gemm<MODE_DOWN, false>(g2, mt_max, s.d / BNB, st);
  return fp8 ? launch_gemm<MODE_DOWN_PERM, true>(g2, mt_max, s.d / BNB, st)
             : launch_gemm<MODE_DOWN_PERM, false>(g2, mt_max, s.d / BNB, st);
}

hipError_t launch_combine(const moe_shape& s, const float* y_perm, const int32_t* slot_pos,
                          const float* topk_w, float* y, hipStream_t st) {
  const int64_t n = s.T * s.d;
  const unsigned blocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 8192));
  combine_kernel<<<blocks, 256, 0, st>>>(y_perm, slot_pos, topk_w, y, s.T, s.top_k, s.d);
  return hipGetLastError();
}

}  // namespace moe
