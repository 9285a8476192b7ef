// Grouped expert FFN on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// The experts' weights are merged per projection ([E, out, in], the
// MergedExpertLayer layout of the iopenshare page §5.2) and each expert runs
// one GEMM over its contiguous segment of grouped rows; the tile schedule is
// read from the device-side offsets (no host synchronisation).
//
//   MODE_GATEUP  H[p, :] = silu(x_p W1_e^T) * (x_p W3_e^T)       (bf16 out)
//                rows are gathered on load: x_p = x[perm_token[p]]
//   MODE_DOWN    y[perm_token[p], :] += perm_w[p] * (H[p, :] W2_e^T)
//                the combine (MOE 学习笔记 输出聚合: weighted sum of the k
//                expert outputs) fused into the epilogue with fp32 atomics
//   MODE_DOWN_PERM  y_perm[p, :] = H[p, :] W2_e^T                (no weight)
//
// A shared expert (iopenshare §1.4: always-active experts) is expert index E
// with T rows, row t = token t, weight 1, hidden rows P_max .. P_max + T.
//
// Workgroup tile: 128 activation rows x 512 weight rows, K in steps of 32;
// 256 threads = 4 waves, each wave all 128 rows x its own 128 weight rows =
// 4 x 4 MFMA tiles of 32x32 (256 accumulators per lane).  In MODE_GATEUP a
// wave's 128 weight rows are 64 rows of W1 and the same 64 rows of W3, so the
// SwiGLU happens in registers; the product is computed transposed
// (weights as the MFMA A operand) so each lane holds 4 consecutive hidden
// columns of one row and stores them as one 8-byte write.
// Pipeline: double-buffered LDS (padded rows, conflict-free 16-byte fragment
// reads) fed from three register stages, so each global load has two K steps
// of MFMAs to land; fragments of the next 16 K are read from LDS under the
// current MFMAs; one barrier per K step.
// Tile order: a 1-D grid remapped so that the workgroups one XCD runs at the
// same time cover an 8 (row tiles) x 4 (weight tiles) block, sharing both
// operands in that XCD's L2.  The down projection may split K across
// workgroups when the tile grid is small (decode); partial sums are added
// by the same atomics.
#include "moe_internal.h"

namespace moe {
namespace {

enum { MODE_GATEUP = 0, MODE_DOWN = 1, MODE_DOWN_PERM = 2 };

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;       // activation rows per tile
constexpr int BNB = 512;      // weight rows per tile
constexpr int BK = 32;        // K per step
constexpr int LDSK = BK + 8;  // padded LDS row, bf16 elements (80 bytes)
constexpr int A_STAGE = BM * LDSK;
constexpr int B_STAGE = BNB * LDSK;
constexpr int GROUP_M = 8;    // row tiles per XCD block
constexpr int GROUP_N = 4;    // weight tiles per XCD block
constexpr int NUM_XCD = 8;

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
  int64_t A_bytes;            // size of the A operand buffer (< 2^31)
  int64_t T;
  int64_t P_max;
  int E;
  int has_shared;
  int K;
  int N;
  int mt_max;                 // row-tile slots in the grid
  int nt;                     // weight tiles
  int ksplit;                 // K ranges (DOWN only)
};

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

// fp8 e4m3 (OCP) -> bf16 bits, exact and branch-free.  Normal codes move
// exponent and mantissa fields (bias 7 -> 127); subnormal codes (exponent
// field 0) are m * 2^-9, formed exactly in fp32 and truncated to bf16 (at
// most 3 significant bits, so nothing is lost).
__device__ __forceinline__ uint32_t e4m3_to_bf16_bits(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 8;
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  const uint32_t normal = ((e + 120u) << 7) | (m << 4);
  const uint32_t sub = __float_as_uint((float)m * 0x1p-9f) >> 16;
  return s | (e ? normal : sub);
}

constexpr int kBufferWord3 = 0x00020000;  // gfx9-family raw buffer descriptor word 3

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// 8 weight elements as bf16 bits: 16 bytes of bf16, or 8 fp8 codes widened.
template <bool FP8>
__device__ __forceinline__ uint4 load_b8(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  if constexpr (!FP8) {
    return buf_load16(r, voff, soff);
  } else {
    const u32x2 q = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    uint4 o;
    o.x = e4m3_to_bf16_bits(q[0] & 0xFF) | (e4m3_to_bf16_bits((q[0] >> 8) & 0xFF) << 16);
    o.y = e4m3_to_bf16_bits((q[0] >> 16) & 0xFF) | (e4m3_to_bf16_bits(q[0] >> 24) << 16);
    o.z = e4m3_to_bf16_bits(q[1] & 0xFF) | (e4m3_to_bf16_bits((q[1] >> 8) & 0xFF) << 16);
    o.w = e4m3_to_bf16_bits((q[1] >> 16) & 0xFF) | (e4m3_to_bf16_bits(q[1] >> 24) << 16);
    return o;
  }
}

template <int MODE, bool FP8>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t* As = lds;                    // [2][BM][LDSK]
  uint16_t* Bs = lds + 2 * A_STAGE;      // [2][BNB][LDSK]
  __shared__ int s_scan[4];
  __shared__ int s_e, s_m0, s_rows, s_seg;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- XCD-aware tile order.  Workgroup ids are dealt round-robin to the 8
  // XCDs; give each XCD a contiguous range of logical tiles, ordered in
  // GROUP_M x GROUP_N blocks (row-tile groups fastest).
  const int ksplit = (MODE == MODE_GATEUP) ? 1 : p.ksplit;
  const int mgroups = (p.mt_max + GROUP_M - 1) / GROUP_M;
  const int ngroups = (p.nt + GROUP_N - 1) / GROUP_N;
  const int64_t tiles_per_k = (int64_t)mgroups * ngroups * (GROUP_M * GROUP_N);
  const int64_t G = tiles_per_k * ksplit;
  const int64_t chunk = (G + NUM_XCD - 1) / NUM_XCD;
  const int64_t Lg = (int64_t)(blockIdx.x % NUM_XCD) * chunk + blockIdx.x / NUM_XCD;
  if (Lg >= G) return;
  const int ks = (int)(Lg / tiles_per_k);
  const int64_t L = Lg % tiles_per_k;
  const int64_t blk = L / (GROUP_M * GROUP_N);
  const int rr = (int)(L % (GROUP_M * GROUP_N));
  const int mslot = __builtin_amdgcn_readfirstlane((int)(blk % mgroups) * GROUP_M + rr % GROUP_M);
  const int ntile = __builtin_amdgcn_readfirstlane((int)(blk / mgroups) * GROUP_N + rr / GROUP_M);
  if (mslot >= p.mt_max || ntile >= p.nt) return;

  // ---- map the row-tile slot to (expert, first row) from the offsets.
  const int nseg = p.E + (p.has_shared ? 1 : 0);
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
    if (tid == 0 && mslot >= total) s_e = -1;
    if (mslot >= excl && mslot < excl + local) {
      for (int i = 0; i < per; ++i) {
        const int e = e_lo + i;
        if (e >= nseg) break;
        const int64_t rows = (e < p.E) ? (int64_t)(p.offsets[e + 1] - p.offsets[e]) : p.T;
        const int nt = (int)((rows + BM - 1) / BM);
        if (mslot < excl + nt) {
          s_e = e;
          s_m0 = (mslot - excl) * BM;
          s_rows = (int)rows;
          s_seg = (e < p.E) ? p.offsets[e] : 0;
          break;
        }
        excl += nt;
      }
    }
    __syncthreads();
  }
  // The LDS values are the same in every lane; say so to the compiler so the
  // buffer resources built from them live in scalar registers.
  const int e = __builtin_amdgcn_readfirstlane(s_e);
  if (e < 0) return;
  const int m0 = __builtin_amdgcn_readfirstlane(s_m0);
  const int rows = __builtin_amdgcn_readfirstlane(s_rows);
  const int seg = __builtin_amdgcn_readfirstlane(s_seg);
  const bool shared_e = (e == p.E);
  const int K = p.K, N = p.N;

  // ---- K range of this workgroup (split-K for the down projection).
  const int ksteps_all = K / BK;
  // (uniform values that went through 64-bit VALU arithmetic: pin them to
  // scalar registers so buffer offsets need no per-lane loops)
  const int kbeg = __builtin_amdgcn_readfirstlane((int)((int64_t)ksteps_all * ks / ksplit));
  const int kend = __builtin_amdgcn_readfirstlane((int)((int64_t)ksteps_all * (ks + 1) / ksplit));
  const int nk = kend - kbeg;

  // ---- operand sources as buffer loads: one scalar resource per operand
  // (and per expert matrix), a 32-bit byte offset per thread and row that
  // stays fixed over K, and the K step in the scalar offset.
  constexpr int WB = FP8 ? 1 : 2;  // bytes per weight element
  const int lr = tid >> 2;         // 0..63: rows lr + 64 i
  const int kc = (tid & 3) * 8;    // element offset within BK
  const __amdgpu_buffer_rsrc_t rsA =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.A, (short)0, (int)p.A_bytes, kBufferWord3);
  uint32_t voA[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = min(m0 + lr + 64 * i, rows - 1);
    int64_t ar;
    if (MODE == MODE_GATEUP)
      ar = shared_e ? (int64_t)m : (int64_t)p.perm_token[seg + m];
    else
      ar = shared_e ? p.P_max + m : (int64_t)seg + m;
    voA[i] = (uint32_t)((ar * K + kc) * 2);
  }
  // B row r (0..511) of the tile.  GATEUP: rows 0..255 are W1 rows n0 + r,
  // rows 256..511 are W3 rows n0 + r - 256 (n0 = ntile * 256).  DOWN: W2 rows
  // n0 + r (n0 = ntile * 512).  Rows past N are clamped (outputs masked).
  const int n0 = (MODE == MODE_GATEUP) ? ntile * (BNB / 2) : ntile * BNB;
  const int64_t ebytes = (int64_t)N * K * WB;  // one expert matrix (< 2^31)
  const char* bptr0 = (const char*)(shared_e ? p.B0s : p.B0) + (shared_e ? 0 : (int64_t)e * ebytes);
  const __amdgpu_buffer_rsrc_t rsB0 =
      __builtin_amdgcn_make_buffer_rsrc((void*)bptr0, (short)0, (int)ebytes, kBufferWord3);
  __amdgpu_buffer_rsrc_t rsB1 = rsB0;
  if (MODE == MODE_GATEUP) {
    const char* bptr1 = (const char*)(shared_e ? p.B1s : p.B1) + (shared_e ? 0 : (int64_t)e * ebytes);
    rsB1 = __builtin_amdgcn_make_buffer_rsrc((void*)bptr1, (short)0, (int)ebytes, kBufferWord3);
  }
  uint32_t voB[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = lr + 64 * i;
    int n = (MODE == MODE_GATEUP) ? n0 + (r & (BNB / 2 - 1)) : n0 + r;
    n = min(n, N - 1);
    voB[i] = (uint32_t)((n * K + kc) * WB);
  }
  // In GATEUP, B loads i = 0..3 come from W1 and i = 4..7 from W3.

  // Three register stages of global loads (A: 2 x 16 B, B: 8 x 16 B per
  // thread and K step), so a load has two K steps of MFMAs to land.
  uint4 ra_0[2], rb_0[8], ra_1[2], rb_1[8], ra_2[2], rb_2[8];
#define MOE_LOAD_STAGE(S, KT)                                                   \
  do {                                                                          \
    const int kstep_ = __builtin_amdgcn_readfirstlane(kbeg + (KT));             \
    ra_##S[0] = buf_load16(rsA, voA[0], kstep_ * BK * 2);                       \
    ra_##S[1] = buf_load16(rsA, voA[1], kstep_ * BK * 2);                       \
    _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_)                            \
      rb_##S[i_] = load_b8<FP8>((MODE == MODE_GATEUP && i_ >= 4) ? rsB1 : rsB0, \
                                voB[i_], kstep_ * BK * WB);                     \
  } while (0)
#define MOE_STORE_STAGE(S, BUF)                                           \
  do {                                                                    \
    uint16_t* a_ = As + (BUF) * A_STAGE;                                  \
    uint16_t* b_ = Bs + (BUF) * B_STAGE;                                  \
    *(uint4*)&a_[lr * LDSK + kc] = ra_##S[0];                             \
    *(uint4*)&a_[(lr + 64) * LDSK + kc] = ra_##S[1];                      \
    _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_)                      \
      *(uint4*)&b_[(lr + 64 * i_) * LDSK + kc] = rb_##S[i_];              \
  } while (0)

  // ---- the wave's weight rows: 4 tiles of 32.
  int brow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (MODE == MODE_GATEUP)
      brow[j] = (j < 2) ? (wave * 64 + j * 32) : (BNB / 2 + wave * 64 + (j - 2) * 32);
    else
      brow[j] = wave * 128 + j * 32;
  }

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int frow = lane & 31;
  const int fk = (lane >> 5) * 8;
  auto compute = [&](int buf) {
    const uint16_t* a = As + buf * A_STAGE;
    const uint16_t* b = Bs + buf * B_STAGE;
    bf16x8 af[2][4], bfr[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[0][i] = *(const bf16x8*)&a[(i * 32 + frow) * LDSK + fk];
#pragma unroll
    for (int j = 0; j < 4; ++j) bfr[0][j] = *(const bf16x8*)&b[(brow[j] + frow) * LDSK + fk];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < BK / 16) {  // fragments of the next 16 K, read under this step's MFMAs
        const int ko = (kk + 1) * 16 + fk;
#pragma unroll
        for (int i = 0; i < 4; ++i) af[cur ^ 1][i] = *(const bf16x8*)&a[(i * 32 + frow) * LDSK + ko];
#pragma unroll
        for (int j = 0; j < 4; ++j) bfr[cur ^ 1][j] = *(const bf16x8*)&b[(brow[j] + frow) * LDSK + ko];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (MODE == MODE_GATEUP)  // transposed: acc[i][j] holds [weight row][act row]
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[cur][j], af[cur][i], acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
        }
    }
  };

  // ---- main loop, unrolled by the three register stages.  At step kt the
  // LDS buffer kt & 1 holds step kt, stage (kt + 1) % 3 holds step kt + 1 and
  // stage (kt + 2) % 3 step kt + 2 (both possibly in flight).  After the
  // MFMAs, stage kt + 1 goes to the other LDS buffer and stage kt % 3 is
  // reloaded with step kt + 3.  One barrier per step.
  if (nk > 0) {
    MOE_LOAD_STAGE(0, 0);
    if (nk > 1) MOE_LOAD_STAGE(1, 1);
    if (nk > 2) MOE_LOAD_STAGE(2, 2);
    MOE_STORE_STAGE(0, 0);
    __syncthreads();
#define MOE_STEP(S0, S1)                                   \
  {                                                        \
    const int k_ = kt + (S0);                              \
    if (k_ >= nk) break;                                   \
    compute(k_ & 1);                                       \
    if (k_ + 1 < nk) MOE_STORE_STAGE(S1, (k_ + 1) & 1);    \
    __syncthreads();                                       \
    if (k_ + 3 < nk) MOE_LOAD_STAGE(S0, k_ + 3);           \
  }
    for (int kt = 0; kt < nk; kt += 3) {
      MOE_STEP(0, 1)
      MOE_STEP(1, 2)
      MOE_STEP(2, 0)
    }
#undef MOE_STEP
  }
#undef MOE_LOAD_STAGE
#undef MOE_STORE_STAGE

  // ---- epilogue.  32x32 accumulator register r of lane l is row
  // (r/4)*8 + (l/32)*4 + r%4, column l%32 of the 32x32 tile.
  const int ccol = lane & 31;
  const int rbase = (lane >> 5) * 4;
  if (MODE == MODE_GATEUP) {
    // acc[i][j]: weight row brow[j] + R, activation row i*32 + ccol.
    const int64_t hbase = shared_e ? p.P_max : (int64_t)seg;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_barrier(0);  // keep the accumulator reads incremental
      const int m = m0 + i * 32 + ccol;
      if (m >= rows) continue;
      uint16_t* hrow = p.H + (hbase + m) * N;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wave * 64 + j * 32 + q * 8 + rbase;  // 4 consecutive columns
          if (n >= N) continue;
          float sg = 1.f, su = 1.f;
          if (FP8) {
            const int gi = n / kFp8Group;
            sg = shared_e ? p.sc0s[gi] : p.sc0[(int64_t)e * (N / kFp8Group) + gi];
            su = shared_e ? p.sc1s[gi] : p.sc1[(int64_t)e * (N / kFp8Group) + gi];
          }
          uint32_t hb[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = acc[i][j][q * 4 + r] * sg;
            const float g = acc[i][j + 2][q * 4 + r] * su;
            hb[r] = f32_to_bf16_bits(a / (1.f + __expf(-a)) * g);
          }
          uint2 v;
          v.x = hb[0] | (hb[1] << 16);
          v.y = hb[2] | (hb[3] << 16);
          *(uint2*)(hrow + n) = v;
        }
      }
    }
  } else {
    // acc[i][j]: activation row i*32 + R, weight row (output column) brow[j] + ccol.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_barrier(0);  // keep the accumulator reads incremental
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + i * 32 + q * 8 + rbase + r;
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
          for (int j = 0; j < 4; ++j) {
            const int n = n0 + brow[j] + ccol;
            if (n >= N) continue;
            float v = acc[i][j][q * 4 + r];
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
}

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

constexpr size_t kGemmLds = (size_t)2 * (A_STAGE + B_STAGE) * sizeof(uint16_t);

template <int MODE, bool FP8>
hipError_t launch_gemm(const GemmParams& p, hipStream_t st) {
  if (p.mt_max <= 0 || p.nt <= 0) return hipSuccess;
  const int64_t mg = (p.mt_max + GROUP_M - 1) / GROUP_M;
  const int64_t ng = (p.nt + GROUP_N - 1) / GROUP_N;
  const int64_t G = mg * ng * GROUP_M * GROUP_N * (MODE == MODE_GATEUP ? 1 : p.ksplit);
  static bool attr_set = false;  // opt in to more than 64 KiB of LDS, once per process
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute((const void*)grouped_gemm_kernel<MODE, FP8>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)kGemmLds);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  const int64_t chunk = (G + NUM_XCD - 1) / NUM_XCD;
  grouped_gemm_kernel<MODE, FP8><<<(unsigned)(chunk * NUM_XCD), 256, kGemmLds, st>>>(p);
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
    hipError_t err = hipGetLastError();
    if (err == hipSuccess && ev_mid) err = hipEventRecord(ev_mid, st);
    return err;
  }
  const bool fp8 = s.w_dtype == MOE_DT_FP8_E4M3;
  const int has_sh = s.has_shared ? 1 : 0;
  // Upper bound of row tiles: sum_e ceil(rows_e / BM) <= P_max / BM + E (+ shared).
  const int64_t mt_max = (L.P_max + BM - 1) / BM + s.E + (has_sh ? (s.T + BM - 1) / BM : 0);

  GemmParams g{};
  g.perm_token = perm_token;
  g.perm_w = perm_w;
  g.offsets = offsets;
  g.T = s.T;
  g.P_max = L.P_max;
  g.E = s.E;
  g.has_shared = has_sh;
  g.mt_max = (int)mt_max;
  g.ksplit = 1;

  // gate / up
  g.A = (const uint16_t*)x;
  g.A_bytes = s.T * (int64_t)s.d * 2;
  g.B0 = w.W1; g.B1 = w.W3; g.B0s = w.W1s; g.B1s = w.W3s;
  g.sc0 = w.s1; g.sc1 = w.s3; g.sc0s = w.s1s; g.sc1s = w.s3s;
  g.H = (uint16_t*)H;
  g.K = s.d;
  g.N = s.d_ff;
  g.nt = (s.d_ff + BNB / 2 - 1) / (BNB / 2);
  hipError_t err = fp8 ? launch_gemm<MODE_GATEUP, true>(g, st)
                       : launch_gemm<MODE_GATEUP, false>(g, st);
  if (err != hipSuccess) return err;
  if (ev_mid) {
    err = hipEventRecord(ev_mid, st);
    if (err != hipSuccess) return err;
  }

  // down (+ combine)
  GemmParams g2 = g;
  g2.A = (const uint16_t*)H;
  g2.A_bytes = L.H_rows * (int64_t)s.d_ff * 2;
  g2.B0 = w.W2; g2.B1 = nullptr; g2.B0s = w.W2s; g2.B1s = nullptr;
  g2.sc0 = w.s2; g2.sc1 = nullptr; g2.sc0s = w.s2s; g2.sc1s = nullptr;
  g2.H = nullptr;
  g2.y = y;
  g2.y_perm = y_perm;
  g2.K = s.d_ff;
  g2.N = s.d;
  g2.nt = (s.d + BNB - 1) / BNB;
  // Split K when the tile grid would leave CUs idle (decode-sized T); only
  // with the atomic combine, whose adds also take the partial sums.
  if (y) {
    const int64_t tiles = (int64_t)(L.P_max / BM + std::min<int64_t>(s.E, L.P_max) + has_sh) * g2.nt;
    const int ksteps = s.d_ff / BK;
    int ks = 1;
    while (tiles * ks < 512 && ks * 2 <= ksteps / 8) ks *= 2;
    g2.ksplit = ks;
  }
  if (y)
    return fp8 ? launch_gemm<MODE_DOWN, true>(g2, st) : launch_gemm<MODE_DOWN, false>(g2, st);
  return fp8 ? launch_gemm<MODE_DOWN_PERM, true>(g2, st)
             : launch_gemm<MODE_DOWN_PERM, false>(g2, st);
}

hipError_t launch_combine(const moe_shape& s, const float* y_perm, const int32_t* slot_pos,
                          const float* topk_w, float* y, hipStream_t st) {
  const int64_t n = s.T * s.d;
  const unsigned blocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 8192));
  combine_kernel<<<blocks, 256, 0, st>>>(y_perm, slot_pos, topk_w, y, s.T, s.top_k, s.d);
  return hipGetLastError();
}

}  // namespace moe
