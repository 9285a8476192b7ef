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
// Two kernels.  The ping-pong kernel (grouped_gemm_pp_kernel, described at
// its definition) takes bf16 weights and, for experts of 256 or more rows,
// 8-bit weights on 256 x 256 tiles with 8 waves; the down projection of
// 8-bit weights at 33..255 rows per expert takes its 128 x 512 tiles.  The
// four-wave kernel (grouped_gemm_dma_kernel) takes the rest: workgroup tile
// 256 activation rows x 256 weight rows, K in steps of 64; 256 threads = 4
// waves of 128 x 128 (4 x 4 MFMA tiles of 32x32, 256 fp32 accumulators per
// lane).  Decode-sized batches (32 or fewer rows per expert on average) use
// 64- or 32-row activation tiles instead, so two workgroups share a CU.  A wave's activation rows are the 32-row granules
// wm, wm + 2, wm + 4, wm + 6 of the tile, and it runs only the granules that
// hold rows of the segment (partial tiles cost in proportion to their rows).
// In MODE_GATEUP a wave's 128 weight rows are 64 rows of W1 and the same 64
// rows of W3, so the SwiGLU happens in registers; the product is computed
// transposed (weights as the MFMA A operand) so each lane holds 4
// consecutive hidden columns of one row and stores them as one 8-byte write.
// Operands move global -> LDS by buffer_load ... lds (two 64-deep stages;
// for decode-sized batches two or three stages, see launch_gemm;
// XOR-swizzled rows, no bank conflicts on the 16-byte fragment reads; no
// loads for activation rows past the segment's end); the next 32-deep
// slice's fragments are read under the current slice's MFMAs; one barrier
// per step.  Quantised weights (OCP fp8 e4m3, symmetric int8, or symmetric
// int4 as offset-binary nibbles) land in LDS as codes and are widened
// exactly to bf16 in registers; their per-128-row scales apply in the
// epilogue.  With 8-bit weights each workgroup starts its
// K walk at its own offset (K rotation).
// Tile order (tile_sched.h): the real tiles, counted on the device, are dealt
// evenly to the XCDs in expert-aligned blocks, so the workgroups one XCD runs
// at the same time share operands in its L2.  The tiles of the last, partial
// round may be split over K: their partial sums are added by the atomic
// combine, or (grouped output) summed from a partial-tile slab by a fixup
// pass.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "moe_internal.h"
#include "tile_sched.h"

#ifndef MOE_SCHED_GN
#define MOE_SCHED_GN 8
#endif
#ifndef MOE_SCHED_NFAST
#define MOE_SCHED_NFAST 0
#endif
#ifndef MOE_GEMM_PF
#define MOE_GEMM_PF 0
#endif
#ifndef MOE_GEMM_PP
#define MOE_GEMM_PP 1
#endif
#ifndef MOE_PP8_ROWS
#define MOE_PP8_ROWS 256
#endif
#ifndef MOE_PP8_WIDE
#define MOE_PP8_WIDE 6  // bit (1 << MODE): the launches that take 128 x 512 tiles
#endif
#ifndef MOE_PP_KROT
#define MOE_PP_KROT 1
#endif
#ifndef MOE_B_NT
#define MOE_B_NT 1
#endif
#ifndef MOE_DECODE_NS
#define MOE_DECODE_NS 2
#endif
#ifndef MOE_DECODE_PF
#define MOE_DECODE_PF 0
#endif
#ifndef MOE_DECODE_GU_SPLIT
#define MOE_DECODE_GU_SPLIT 0
#endif

namespace moe {
namespace {

enum { MODE_GATEUP = 0, MODE_DOWN = 1, MODE_DOWN_PERM = 2 };

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Tiles: 256 activation rows x 256 weight rows (four waves of 128 x 128);
// K is counted in units of BK (the schedule's K pieces are whole multiples).
constexpr int BK = 32;

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
  const float* shared_w;      // MODE_DOWN: per-token weight of the shared expert (NULL: 1)
  int64_t A_bytes;            // size of the A operand buffer (< 2^31)
  int64_t T;
  int64_t P_max;
  int E;
  int has_shared;
  int K;                      // A row length and K extent (elements)
  int kb_len;                 // B row length (elements): K, or K/2 when A holds two
                              // terms per hidden unit (hi | lo) against the same B
  int N;
  int h_ld;                   // GATEUP: H row stride (N, or 2N with the lo terms after)
  int h_split;                // GATEUP: also store lo = bf16(h - bf16(h)) at column N + n
  int mt_max;                 // upper bound of the row tiles (grid size)
  int nt;                     // weight tiles
  int split_max;              // K ranges a tail tile may be cut into (1: none)
  int kunit;                  // K steps of BK per unit of the schedule
  int slots;                  // workgroups one XCD runs at once
  float* tail_slab;           // fp32 partial tiles of split tail tiles (GATEUP, DOWN_PERM)
  int64_t slab_floats;        //   its size in floats
  int slab_piece;             //   floats per partial tile: activation-tile rows x 256
  int group_n;                // weight tiles per expert-aligned block of the tile order
  int nfast;                  // tile order inside a block: weight tiles fastest (1) or row tiles
  int krot;                   // K walk start of workgroup b: (b * krot) mod (its K steps); 0 = none
  int b_nt;                   // weight loads of a tile whose expert fits in that one row tile
                              // (so no other tile reads its weight panel) as non-temporal
  float* zero_out;            // zero_n floats (16-byte aligned) the workgroups clear first, or NULL
  int64_t zero_n;             //   (the atomic combine's y, cleared by the gate/up launch)
};

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, expanded at
// compile time.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

constexpr int kBufferWord3 = 0x00020000;  // gfx9-family raw buffer descriptor word 3

// A raw buffer resource over [ptr, ptr + bytes) built from values the caller
// knows to be wave-uniform, pinned to scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* ptr, int64_t bytes) {
  const uint64_t a = (uint64_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), kBufferWord3);
}

// Where a workgroup's tile lies: expert segment, rows, weight tile, K range.
struct TileMap {
  int e;         // expert (E = the shared expert)
  int m0;        // first row of the tile within the expert's segment
  int rows;      // rows in the expert's segment
  int seg;       // first grouped row of the segment (routed experts)
  int ntile;     // weight tile
  int kbeg, nk;  // K steps of this workgroup
  bool shared_e;
  int slab;      // MODE_DOWN_PERM piece of a split tail tile: its partial-tile
                 // slot in p.tail_slab (-1: the tile is stored directly)
};

// The workgroup's unit of the tile schedule (tile_sched.h): the segments'
// row tiles are counted and scanned from the device-side offsets into an LDS
// prefix array, which the expert-aligned tile map then searches.  Returns
// false when the workgroup has no unit.  Must be called by all threads of
// the workgroup.
constexpr int kMaxSegments = 1025;  // routed experts (at most 1024) + shared

// Row tiles per segment (routed experts, then the shared expert), counted
// from the device-side offsets and scanned into s_pre (s_pre[nseg] = total).
// Must be called by all threads of the workgroup; returns the total.
template <int BM, int NT = 256>
__device__ __forceinline__ int seg_prefix(const GemmParams& p, int* s_pre, int* s_scan) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nseg = p.E + (p.has_shared ? 1 : 0);
  const int per = (nseg + NT - 1) / NT;
  const int e_lo = tid * per;
  auto seg_tiles = [&](int e) {
    const int64_t rows = (e < p.E) ? (int64_t)(p.offsets[e + 1] - p.offsets[e]) : p.T;
    return (int)((rows + BM - 1) / BM);
  };
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (e_lo + i < nseg) local += seg_tiles(e_lo + i);
  const int incl = wave_incl_scan(local, lane);
  if (lane == 63) s_scan[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w2 = 0; w2 < wave; ++w2) before += s_scan[w2];
  int run = before + incl - local;
  for (int i = 0; i < per; ++i) {
    const int e = e_lo + i;
    if (e < nseg) {
      s_pre[e] = run;
      run += seg_tiles(e);
    }
  }
  if (tid == 0) {
    int total = 0;
    for (int w2 = 0; w2 < NT / 64; ++w2) total += s_scan[w2];
    s_pre[nseg] = total;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(s_pre[nseg]);
}

// Segment, first row and weight tile of tile q (uniform values).
template <int BM>
__device__ __forceinline__ void tile_place(const GemmParams& p, const int* s_pre, int64_t q,
                                           TileMap& t) {
  const int nseg = p.E + (p.has_shared ? 1 : 0);
  int seg = 0, mslot = 0, ntile = 0;
  sched_tile_of(q, s_pre, nseg, p.nt, p.group_n, seg, mslot, ntile, p.nfast != 0);
  t.e = __builtin_amdgcn_readfirstlane(seg);
  t.ntile = __builtin_amdgcn_readfirstlane(ntile);
  t.m0 = __builtin_amdgcn_readfirstlane((mslot - s_pre[seg]) * BM);
  t.shared_e = (t.e == p.E);
  t.rows = __builtin_amdgcn_readfirstlane(t.shared_e ? (int)p.T
                                                     : p.offsets[t.e + 1] - p.offsets[t.e]);
  t.seg = __builtin_amdgcn_readfirstlane(t.shared_e ? 0 : p.offsets[t.e]);
}

// The workgroup's unit of the tile schedule (tile_sched.h) over the
// expert-aligned tile order.  Returns false when the workgroup has no unit.
// Must be called by all threads of the workgroup.
template <int MODE, int BM, int NT = 256>
__device__ __forceinline__ bool map_tile(const GemmParams& p, TileMap& t) {
  __shared__ int s_scan[NT / 64];
  __shared__ int s_pre[kMaxSegments + 1];
  const int Mreal = seg_prefix<BM, NT>(p, s_pre, s_scan);
  SchedUnit u{};
  const int kunits = p.K / BK / p.kunit;
  const int xcd = (int)(blockIdx.x % kNumXcd);
  if (!sched_unit((int64_t)Mreal * p.nt, kunits, p.slots, p.split_max, xcd,
                  (int64_t)(blockIdx.x / kNumXcd), u))
    return false;
  tile_place<BM>(p, s_pre, u.q, t);
  t.kbeg = __builtin_amdgcn_readfirstlane(u.kbeg * p.kunit);
  t.nk = __builtin_amdgcn_readfirstlane(u.nk * p.kunit);
  t.slab = ((MODE == MODE_DOWN_PERM || MODE == MODE_GATEUP) && u.tail >= 0)
               ? __builtin_amdgcn_readfirstlane(xcd * p.slots + u.tail)
               : -1;
  return true;
}

// Row (in elements of K) of activation row m of the tile's segment in the A
// operand: gathered token rows of x for GATEUP, hidden rows for DOWN*.
template <int MODE>
__device__ __forceinline__ int64_t a_row(const GemmParams& p, const TileMap& t, int m) {
  if (MODE == MODE_GATEUP) return t.shared_e ? (int64_t)m : (int64_t)p.perm_token[t.seg + m];
  return t.shared_e ? p.P_max + m : (int64_t)t.seg + m;
}

// Four consecutive hidden values h[0..3] of one row at column n: their bf16
// roundings hi, and with `split` also lo = bf16(h - hi) at column N + n (the
// compensated form, h = hi + lo to about 2^-17 relative).
__device__ __forceinline__ void store_h4(uint16_t* hrow, int n, int N, const float (&h)[4],
                                         int split) {
  uint32_t hb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) hb[r] = f32_to_bf16_bits(h[r]);
  *(uint2*)(hrow + n) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
  if (split) {
    uint32_t lb[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lb[r] = f32_to_bf16_bits(h[r] - bf16_bits_to_f32(hb[r]));
    *(uint2*)(hrow + N + n) = make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
  }
}

// Epilogue.  32x32 accumulator register r of lane l is row (r/4)*8 +
// (l/32)*4 + r%4, column l%32 of the 32x32 tile.  arow0: the wave's first
// activation row in the tile, its i-th 32-row granule starting RS rows
// further per i (32: contiguous rows, 64: granules interleaved with the other
// row wave); brow: its four 32-row weight tiles; n0: first output column of
// the tile; wn: the wave's column group.  CORR (int4 weights): ctab[i * 32
// + R] is the amount to take off every accumulator of row R of granule i
// (136 times the row's activation sum), before the scale.  GI: the wave's
// granules in the tile (4 in a 256-row tile, 1 in a 64-row one); rows past
// them belong to the next tile.
template <int MODE, bool FP8, int RS, int BMT, bool CORR = false, int GI = 4, int TR = 256>
__device__ __forceinline__ void store_tile(const GemmParams& p, f32x16 (&acc)[4][4],
                                           const TileMap& t, int arow0, int n0, int wn,
                                           const int (&brow)[4], const float* ctab = nullptr) {
  const int lane = threadIdx.x & 63;
  const int ccol = lane & 31;
  const int rbase = (lane >> 5) * 4;
  const int N = p.N;
  if (MODE == MODE_GATEUP) {
    // transposed product: acc[i][j] holds weight row brow[j] + R, activation
    // row arow0 + i*RS + ccol; tiles j and j + 2 are the gate and up halves.
    const int64_t hbase = t.shared_e ? p.P_max : (int64_t)t.seg;
#pragma unroll
    for (int i = 0; i < GI; ++i) {
      __builtin_amdgcn_sched_barrier(0);  // keep the accumulator reads incremental
      const int m = t.m0 + arow0 + i * RS + ccol;
      if (m >= t.rows || m - t.m0 >= TR) continue;
      const float cr = CORR ? ctab[i * 32 + ccol] : 0.f;
      uint16_t* hrow = p.H + (hbase + m) * p.h_ld;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * 64 + j * 32 + q * 8 + rbase;  // 4 consecutive columns
          if (n >= N) continue;
          float sg = 1.f, su = 1.f;
          if (FP8) {
            const int gi = n / kFp8Group;
            sg = t.shared_e ? p.sc0s[gi] : p.sc0[(int64_t)t.e * (N / kFp8Group) + gi];
            su = t.shared_e ? p.sc1s[gi] : p.sc1[(int64_t)t.e * (N / kFp8Group) + gi];
          }
          if (t.slab >= 0) {  // piece of a split tail tile: gate and up partial sums
            float* sl = p.tail_slab + (int64_t)t.slab * p.slab_piece + (int64_t)(m - t.m0) * 256 + (n - n0);
            *(float4*)sl = make_float4(
                (acc[i][j][q * 4] - cr) * sg, (acc[i][j][q * 4 + 1] - cr) * sg,
                (acc[i][j][q * 4 + 2] - cr) * sg, (acc[i][j][q * 4 + 3] - cr) * sg);
            *(float4*)(sl + 128) = make_float4(
                (acc[i][j + 2][q * 4] - cr) * su, (acc[i][j + 2][q * 4 + 1] - cr) * su,
                (acc[i][j + 2][q * 4 + 2] - cr) * su, (acc[i][j + 2][q * 4 + 3] - cr) * su);
            continue;
          }
          float hv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = (acc[i][j][q * 4 + r] - cr) * sg;
            const float g = (acc[i][j + 2][q * 4 + r] - cr) * su;
            hv[r] = a / (1.f + __expf(-a)) * g;
          }
          store_h4(hrow, n, N, hv, p.h_split);
        }
      }
    }
  } else {
    // acc[i][j]: activation row arow0 + i*RS + R, output column brow[j] + ccol.
#pragma unroll
    for (int i = 0; i < GI; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_barrier(0);  // keep the accumulator reads incremental
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = t.m0 + arow0 + i * RS + q * 8 + rbase + r;
          if (m >= t.rows || m - t.m0 >= TR) continue;
          const float cr = CORR ? ctab[i * 32 + q * 8 + rbase + r] : 0.f;
          float wgt = 1.f;
          int64_t orow;
          if (MODE == MODE_DOWN) {
            if (t.shared_e) {
              orow = m;
              if (p.shared_w) wgt = p.shared_w[m];
            } else {
              orow = p.perm_token[t.seg + m];
              wgt = p.perm_w[t.seg + m];
            }
          } else {
            orow = t.shared_e ? p.P_max + m : (int64_t)t.seg + m;
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = n0 + brow[j] + ccol;
            if (n >= N) continue;
            float v = acc[i][j][q * 4 + r] - cr;
            if (FP8) {
              const int gi = n / kFp8Group;
              v *= t.shared_e ? p.sc0s[gi] : p.sc0[(int64_t)t.e * (N / kFp8Group) + gi];
            }
            if (MODE == MODE_DOWN)
              atomicAdd(&p.y[orow * N + n], wgt * v);
            else if (t.slab >= 0)  // piece of a split tail tile: its partial tile
              p.tail_slab[(int64_t)t.slab * p.slab_piece + (int64_t)(m - t.m0) * 256 + (n - n0)] = v;
            else
              p.y_perm[orow * N + n] = v;
          }
        }
      }
    }
  }
}

// The wave's four 32-row weight tiles.  GATEUP: 64 gate rows then the same
// 64 up rows (which sit BNB/2 further in the tile); DOWN*: 128 rows.
template <int MODE, int BNB>
__device__ __forceinline__ void wave_brows(int wn, int (&brow)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (MODE == MODE_GATEUP)
      brow[j] = (j < 2) ? (wn * 64 + j * 32) : (BNB / 2 + wn * 64 + (j - 2) * 32);
    else
      brow[j] = wn * 128 + j * 32;
  }
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// ---------------------------------------------------------------------------
// LDS-DMA kernel for bf16 weights: 256 x 256 tiles (2 x 2 waves of 128 x 128),
// operands moved global -> LDS by buffer_load ... lds (no register staging,
// no LDS write instructions), NS stage buffers of KB-deep K steps, filled
// NS - 1 steps ahead.  Rows are KB*2 bytes; their 16-byte chunks are
// XOR-swizzled by (row / rows-per-256-bytes) % chunks-per-row, so the 16-byte
// fragment reads of 32 consecutive rows hit distinct banks while each
// wave-level DMA instruction still writes 1 KiB contiguously.
constexpr int DMA_BM = 256;
// cache policy of a DMA load (the buffer instruction's aux operand): 1 for the
// operand panels that tiles share through L2, kAuxStream (the non-temporal
// bit) for weight panels that only one row tile reads, which then do not
// push the shared activation rows out of L2
constexpr int kAuxStream = 2;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int KB, int NS, int WBITS, int BMA = 256, int BNT = 256>
struct DmaCfg {
  // activation (A) tile: 256 rows of KB bf16
  static constexpr int RB = KB * 2;                 // bytes per A row and stage
  static constexpr int CPR = RB / 16;               // 16-byte chunks per A row
  static constexpr int RPS = 256 / RB;              // A rows per 256-byte bank sweep
  static constexpr int ROWS_PER_INST = 1024 / RB;   // A rows one wave-level DMA fills
  static constexpr int NI = BMA / 2 / ROWS_PER_INST;  // A DMA instructions per wave and stage
  static constexpr int TILE_BYTES = BMA * RB;         // the A tile (BMA activation rows)
  // weight (B) tile: BNT rows (256, or 512 under 128-row activation tiles)
  // of KB weights of WBITS bits (16 bf16, 8 or 4)
  static constexpr int RBB = KB * WBITS / 8;         // bytes per B row and stage
  static constexpr int CPRB = RBB / 16;
  static constexpr int RPSB = 256 / RBB;
  static constexpr int ROWS_PER_INST_B = 1024 / RBB;
  static constexpr int NIB = 128 / ROWS_PER_INST_B; // B DMA instructions per wave and stage
  static constexpr int B_TILE_BYTES = BNT * RBB;
  static constexpr int STAGE_BYTES = TILE_BYTES + B_TILE_BYTES;
  static constexpr int NI_MAX = NI > NIB ? NI : NIB;
  static constexpr size_t LDS = (size_t)NS * STAGE_BYTES;
  static_assert(KB % 32 == 0 && NS >= 2 && NS <= 4 && RBB >= 16, "DMA pipeline shape");
  static_assert((BMA == 256 || BMA == 128 || BMA == 64 || BMA == 32) && NI >= 1,
                "activation tile rows");
  static_assert(BNT == 256 || (BNT == 512 && BMA == 128), "weight tile rows");
  static_assert(LDS <= 150 * 1024, "LDS budget (with the static tile-map arrays)");
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt left at their maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 8 OCP e4m3 codes (K order, low byte first) -> 8 bf16, exactly: the gfx950
// scaled conversion with scale 1 (e4m3 values are all representable in bf16).
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint2 q) {
  const bf16x2v p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, false);
  const bf16x2v p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, true);
  const bf16x2v p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, false);
  const bf16x2v p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// 8 symmetric int8 codes (K order, low byte first) -> 8 bf16, exactly: each
// code (|q| <= 127) has at most 7 significant bits.  Sign-extending byte
// conversions to fp32, then pairs packed to bf16.
__device__ __forceinline__ bf16x8 int8x8_to_bf16x8(uint2 q) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (__bf16)(float)(int8_t)(q.x >> (8 * i));
#pragma unroll
  for (int i = 0; i < 4; ++i) r[4 + i] = (__bf16)(float)(int8_t)(q.y >> (8 * i));
  return r;
}

// One group of 8 int4 codes (offset binary c = n + 8; byte b holds input b
// in its low nibble and input b + 4 in its high nibble) -> the 8 bf16 values
// 128 + c = 136 + n, exactly: the bf16 pattern 0x43cc is 128 + c for c < 16,
// so after splitting the nibbles into bytes each pair of values is one byte
// permute with the constant 0x43.  The MFMA then sums a * (136 + n); the
// epilogue takes 136 * (sum of a) off (int4_rowsum below).
__device__ __forceinline__ bf16x8 int4x8_to_bf16x8(uint32_t q) {
  const uint32_t lo = q & 0x0F0F0F0Fu;         // c of inputs 0..3, one per byte
  const uint32_t hi = (q >> 4) & 0x0F0F0F0Fu;  // c of inputs 4..7
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  u32x4v r;
  // v_perm_b32: selector bytes 0..3 pick bytes of the second source, 4..7
  // bytes of the first (the constant)
  r.x = __builtin_amdgcn_perm(0x43434343u, lo, 0x04010400u);
  r.y = __builtin_amdgcn_perm(0x43434343u, lo, 0x04030402u);
  r.z = __builtin_amdgcn_perm(0x43434343u, hi, 0x04010400u);
  r.w = __builtin_amdgcn_perm(0x43434343u, hi, 0x04030402u);
  return __builtin_bit_cast(bf16x8, r);
}
// The offset the int4 widening adds to every code.
constexpr float kInt4Offset = 136.f;

// Sum of the 8 bf16 activations of a fragment, added to acc (fp32 dot
// products with ones).
__device__ __forceinline__ float int4_rowsum(bf16x8 a, float acc) {
  typedef __bf16 bf16x2v2 __attribute__((ext_vector_type(2)));
  const bf16x2v2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7), one, acc, false);
  return acc;
}

// Weight formats of the GEMM: bf16, or 8-bit / 4-bit codes with fp32 scales
// per 128 output rows (OCP fp8 e4m3, symmetric int8, symmetric int4 as
// offset-binary nibbles in groups of 8 inputs).
enum { WQ_BF16 = 0, WQ_FP8 = 1, WQ_INT8 = 2, WQ_INT4 = 3 };
constexpr int wq_bits(int wq) { return wq == WQ_BF16 ? 16 : (wq == WQ_INT4 ? 4 : 8); }

// wait_vmcnt for a count known only at run time (wave-uniform, 0..NMAX):
// s_waitcnt takes an immediate, so one branch per possible count.
template <int NMAX>
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  static_for<NMAX + 1>([&](auto c) {
    if (n == decltype(c)::value) wait_vmcnt<decltype(c)::value>();
  });
}

// s_waitcnt with only the LDS counter constrained: lgkmcnt(0).
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}

// L2 prefetch (PF = d > 0): when a workgroup issues the DMA of K step s, it
// also touches every 128-byte line of step s + d of its weight rows (and, in
// 256-row tiles, of its activation rows) with one 4-byte DMA per row into a
// sink in LDS that nothing reads, so those lines are on their way to L2 d
// steps before their DMA.  A 64-deep bf16 step of a row is exactly one line,
// so 128 rows take 2 instructions per wave, and the sink is 2 KiB.
constexpr int kPfSinkBytes = 2048;

template <int MODE, int KB, int NS, int MOE_AUX, int WQ, int BMA, int PF = 0>
__global__ __launch_bounds__(256, 1) void grouped_gemm_dma_kernel(GemmParams p) {
  static_assert(!PF || (KB * 2 == 128 && WQ == WQ_BF16 && NS == 2), "prefetch: 64-deep bf16 steps, two stages");
  constexpr bool FP8 = WQ != WQ_BF16;  // quantised weight codes with scales
  constexpr int WBITS = wq_bits(WQ);
  using C = DmaCfg<KB, NS, WBITS, BMA>;
  constexpr int BNB = 256;
  extern __shared__ __attribute__((aligned(1024))) char dlds[];
  if (p.zero_out) {  // every workgroup clears its share, with or without a tile
    const int64_t n4 = p.zero_n / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
      ((float4*)p.zero_out)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (blockIdx.x == 0 && (int64_t)threadIdx.x < p.zero_n - n4 * 4) p.zero_out[n4 * 4 + threadIdx.x] = 0.f;
  }
  TileMap t;
  if (!map_tile<MODE, BMA>(p, t)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = p.K, N = p.N, KW = p.kb_len;
  // K steps of KB (the workgroup's K range is given in steps of BK)
  const int kbeg_el = t.kbeg * BK;
  const int nk = (t.nk * BK) / KB;
  // B's K steps: step kabs of A reads B step kabs mod nkw (A holding two
  // terms per hidden unit reads B twice)
  const int nkw = KW / KB;
  const int kbeg_st = kbeg_el / KB;

  // ---- DMA sources.  Waves 0, 1 fill the A tile, waves 2, 3 the B tile
  // (in GATEUP wave 2 the W1 rows, wave 3 the W3 rows).  A wave's
  // instruction j fills 1 KiB: tile rows ((w & 1) * NI + j) * ROWS_PER_INST +
  // lane / CPR (B: the _B / CPRB / NIB counterparts); lane i writes chunk slot
  // i % CPR, which holds K chunk (i % CPR) ^ swz(row).
  const int n0 = (MODE == MODE_GATEUP) ? t.ntile * (BNB / 2) : t.ntile * BNB;
  const int64_t ebytes = (int64_t)N * KW * WBITS / 8;
  const int64_t eoff = t.shared_e ? 0 : (int64_t)t.e * ebytes;
  // the B wave's own weight matrix (GATEUP: wave 3 reads W3, wave 2 W1), as
  // one resource built from a pointer chosen up front (a select between two
  // resources would go through scratch memory)
  const bool w3 = (MODE == MODE_GATEUP) && wave == 3;
  const void* bsrc = w3 ? (t.shared_e ? p.B1s : p.B1) : (t.shared_e ? p.B0s : p.B0);
  // each wave's one DMA source (A waves: the activations)
  const bool a_wave = wave < 2;
  const __amdgpu_buffer_rsrc_t rsW =
      uniform_rsrc(a_wave ? (const char*)p.A : (const char*)bsrc + eoff, a_wave ? p.A_bytes : ebytes);
  // Rows past the segment's end (or past N) get an offset beyond the buffer:
  // the buffer range check turns their loads into zeros with no memory
  // traffic (operands are below 2 GiB, so 2^31 plus the K offset is out of
  // range and does not wrap).  Those rows' results are never stored.
  constexpr uint32_t kOobOff = 0x80000000u;
  uint32_t voff[C::NI_MAX];
  static_for<C::NI_MAX>([&](auto j) {
    if (wave < 2) {
      const int r = ((wave & 1) * C::NI + j) * C::ROWS_PER_INST + lane / C::CPR;  // 0..BMA-1
      const int chunk = (lane % C::CPR) ^ ((r / C::RPS) % C::CPR);
      const int m = t.m0 + min(r, BMA - 1);
      voff[j] = m < t.rows
                    ? (uint32_t)((a_row<MODE>(p, t, m) * K + kbeg_el) * 2 + chunk * 16)
                    : kOobOff;
    } else {
      const int r = ((wave & 1) * C::NIB + j) * C::ROWS_PER_INST_B + lane / C::CPRB;
      const int chunk = (lane % C::CPRB) ^ ((r / C::RPSB) % C::CPRB);
      const int n = (MODE == MODE_GATEUP) ? n0 + (r & (BNB / 2 - 1)) : n0 + min(r, 255);
      voff[j] = n < N ? (uint32_t)((int64_t)n * KW * WBITS / 8 + chunk * 16) : kOobOff;
    }
  });
  // prefetch rows: B waves their 128 weight rows, A waves (256-row tiles
  // only) their 128 activation rows, lane + 64 j for j = 0, 1
  constexpr bool kPfA = BMA == 256;
  const bool has_pf = PF != 0 && (!a_wave || kPfA);
  uint32_t pfoff[2] = {kOobOff, kOobOff};
  if constexpr (PF != 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = (wave & 1) * 128 + j * 64 + lane;
      if (a_wave) {
        const int m = t.m0 + r;
        pfoff[j] = m < t.rows ? (uint32_t)((a_row<MODE>(p, t, m) * K + kbeg_el) * 2) : kOobOff;
      } else {
        const int n = (MODE == MODE_GATEUP) ? n0 + (r & (BNB / 2 - 1)) : n0 + r;
        pfoff[j] = n < N ? (uint32_t)((int64_t)n * KW * WBITS / 8) : kOobOff;
      }
    }
  }
  // Branching on the (scalar) wave index keeps each resource in scalar registers.
  // Activation DMA instructions whose rows all lie past the segment's end
  // are not issued at all.  A wave's rows are contiguous, so its valid
  // instructions are a prefix, a_valid of them at every step; the waits for
  // "k steps still in flight" count them.
  const int a_valid = [&] {
    if (!a_wave) return C::NI;
    const int left = t.rows - t.m0 - (wave & 1) * C::NI * C::ROWS_PER_INST;
    return __builtin_amdgcn_readfirstlane(
        max(0, min(C::NI, (left + C::ROWS_PER_INST - 1) / C::ROWS_PER_INST)));
  }();
  // the weight panel of an expert that fits in this one row tile is read by
  // this workgroup only: its loads may stream past L2
  const bool b_nt = p.b_nt && t.rows <= BMA;
  // K rotation: the workgroup walks its K steps from a start of its own, so
  // concurrent workgroups streaming rows of the same pitch (a power of two
  // in the usual shapes) do not all address the same offset within their
  // rows, which would load a few memory channels only.  The sum over K is
  // the same up to fp32 rounding order.
  const int krot = p.krot ? __builtin_amdgcn_readfirstlane(
                                (int)(((uint32_t)blockIdx.x * (uint32_t)p.krot) % (uint32_t)max(nk, 1)))
                          : 0;
  auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
    const int kr = kt + krot < nk ? kt + krot : kt + krot - nk;
    char* gbase = dlds + stage * C::STAGE_BYTES +
                  (a_wave ? (wave & 1) * (C::TILE_BYTES / 2)
                          : C::TILE_BYTES + (wave & 1) * (C::B_TILE_BYTES / 2));
    int kb = kbeg_st + kr;  // B: the absolute step, wrapped
    kb = kb >= nkw ? kb - nkw : kb;
    const int soff = __builtin_amdgcn_readfirstlane(a_wave ? kr * C::RB : kb * C::RBB);
    // the streaming hint on the step that reads the last part of each
    // 128-byte weight line (every step for bf16 rows)
    const bool nt_now = b_nt && (C::RBB >= 128 || (kb + 1) % (128 / C::RBB) == 0);
    if constexpr (C::NI == C::NIB) {
      if (!a_wave && nt_now)
        static_for<C::NIB>([&](auto j) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsW, (lds_ptr_t)(gbase + j * 1024), 16, voff[j], soff, 0, kAuxStream);
        });
      else
        static_for<C::NI>([&](auto j) {
          if (j < a_valid)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsW, (lds_ptr_t)(gbase + j * 1024), 16, voff[j], soff, 0, MOE_AUX);
        });
    } else if (a_wave) {
      static_for<C::NI>([&](auto j) {
        if (j < a_valid)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsW, (lds_ptr_t)(gbase + j * 1024), 16, voff[j], soff, 0, MOE_AUX);
      });
    } else if (nt_now) {
      static_for<C::NIB>([&](auto j) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsW, (lds_ptr_t)(gbase + j * 1024), 16, voff[j], soff, 0, kAuxStream);
      });
    } else {
      static_for<C::NIB>([&](auto j) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsW, (lds_ptr_t)(gbase + j * 1024), 16, voff[j], soff, 0, MOE_AUX);
      });
    }
    if constexpr (PF != 0) {
      // the lines of step kt + PF (issued after this step's DMA, so waiting
      // for this step leaves these two in flight)
      if (has_pf && kt + PF < nk) {
        const int kq = kt + PF + krot < nk ? kt + PF + krot : kt + PF + krot - nk;
        int kbq = kbeg_st + kq;
        kbq = kbq >= nkw ? kbq - nkw : kbq;
        const int spf = __builtin_amdgcn_readfirstlane(a_wave ? kq * C::RB : kbq * C::RBB);
        char* sink = dlds + C::LDS + wave * 512;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsW, (lds_ptr_t)sink, 4, pfoff[0], spf, 0, MOE_AUX);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsW, (lds_ptr_t)(sink + 256), 4, pfoff[1], spf, 0, MOE_AUX);
      }
    }
  };

  // Wave (wm, wn) owns the 32-row granules wm, wm + 2, wm + 4, wm + 6 of the
  // tile (interleaved, so a partial tile's valid granules split evenly over
  // the two row waves) and 128 weight rows.  Only the granules that hold rows
  // of the segment are computed: a wave runs the main loop compiled for its
  // count NG (0..4) of valid granules; every wave still takes part in the DMA
  // and the barriers.
  const int wm = wave >> 1, wn = wave & 1;
  const int arow0 = wm * 32;
  int brow[4];
  wave_brows<MODE, BNB>(wn, brow);
  f32x16 acc[4][4];
  zero_acc(acc);
  // int4: the lane's partial sums of its activation rows over its K halves
  float rs[4] = {0.f, 0.f, 0.f, 0.f};
  const int vg = min(BMA / 32, (t.rows - t.m0 + 31) / 32);  // valid granules of the tile
  const int ng = __builtin_amdgcn_readfirstlane(vg > wm ? (vg - wm + 1) / 2 : 0);

  // fragment reads: tile rows are 32-aligned, so swz(row) = (frow / RPS) % CPR
  const int frow = lane & 31;
  const int fhalf = lane >> 5;
  const int swz = (frow / C::RPS) % C::CPR;

  // ---- pipeline over 32-deep K slices (HPS per DMA step).  The fragments of
  // slice s + 1 are read from LDS while the MFMAs of slice s run (two
  // fragment buffers, LDS reads interleaved with the MFMAs).  Before the
  // first read of a new step t, each wave has finished its reads of step
  // t - 1 (lgkmcnt 0) and waited for its own DMA of step t; one barrier then
  // makes step t visible to all waves and frees the stage of step t - 1, which
  // is refilled with step t + NS - 1.  (A bare s_barrier: the fence of
  // __syncthreads would wait for all DMA.)
  constexpr int HPS = KB / 32;
  const int nsl = nk * HPS;
  // per-lane LDS byte offsets of the fragment rows (stage 0, chunk slot 0)
  // and of the swizzled 16-byte chunk for each (half, kk) of a step
  const int a_row_off = (arow0 + frow) * C::RB;
  // 8-bit weight codes (K8): K is permuted within each 32-deep slice so that
  // a lane's 16 codes of one 16-byte LDS read serve both MFMAs of the slice:
  // MFMA kk, lane half g takes the 8 K positions 32h + 16g + 8kk + 0..7, and
  // the activation fragment the same 8 (an 8-byte read per MFMA conflicts
  // in the LDS banks; the sums are the same up to the order of the adds)
  constexpr bool K8 = WBITS == 8;
  int col_off[HPS][2];
  static_for<HPS>([&](auto h) {
    static_for<2>([&](auto kk) {
      col_off[h][kk] = (((h * 4 + (K8 ? fhalf * 2 + kk : kk * 2 + fhalf)) ^ swz) * 16);
    });
  });
  // quantised weight rows: 8 codes (8 or 4 bytes) per fragment, part of a
  // swizzled 16-byte chunk; the B tile rows are 32-aligned as well
  const int swzb = FP8 ? (frow / C::RPSB) % C::CPRB : 0;
  // step boundary before slice sl (sl % HPS == 0, sl > 0): see above
  // a wave's DMA instructions per step: NI (activation waves) or NIB (weight
  // waves; fewer with fp8 weights), so "k steps still in flight" is a
  // different count per wave kind
  auto wait_steps = [&](auto KS) __attribute__((always_inline)) {
    constexpr int k = decltype(KS)::value;
    if constexpr (k == 0)
      wait_vmcnt<0>();
    else if (a_wave)
      wait_vmcnt_dyn<k * C::NI>(k * a_valid);
    else
      wait_vmcnt<k * C::NIB>();
  };
  auto step_sync = [&](int sl) __attribute__((always_inline)) {
    const int t = sl / HPS;
    wait_lgkm0();
    // steady state: the NS - 2 later steps may stay in flight; near the end
    // (fewer issued) wait for everything.  With the prefetch the two touches
    // of step t + 1, issued after step t's DMA, may stay in flight.
    if (PF != 0 && has_pf && t + PF < nk)
      wait_vmcnt<2>();
    else if (t + NS - 2 <= nk - 1)
      wait_steps(std::integral_constant<int, NS - 2>{});
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (t + NS - 1 < nk) issue(t + NS - 1, (t + NS - 1) % NS);
  };
  auto run = [&](auto NGc) __attribute__((always_inline)) {
    constexpr int NG = decltype(NGc)::value;
    constexpr int NGA = NG > 0 ? NG : 1;
    // weight fragments: bf16, or the raw fp8 codes, widened just before their
    // MFMAs (so the LDS reads of the next slice need not land early)
    using BFrag = std::conditional_t<WBITS == 16, bf16x8, std::conditional_t<WBITS == 8, uint2, uint32_t>>;
    bf16x8 fa0[2][NGA], fa1[2][NGA];
    BFrag fb0[2][4], fb1[2][4];
    auto read_slice = [&](int sl, bf16x8 (&fa)[2][NGA], BFrag (&fb)[2][4]) __attribute__((always_inline)) {
      if constexpr (NG > 0) {
        const int stage = (sl / HPS) % NS;
        const int h = sl % HPS;
        const char* a = dlds + stage * C::STAGE_BYTES;
        const char* b = a + C::TILE_BYTES;
        static_for<2>([&](auto kk) {
          const int co = (HPS == 1 || h == 0) ? col_off[0][kk] : col_off[HPS - 1][kk];
#pragma unroll
          for (int i = 0; i < NG; ++i)
            fa[kk][i] = *(const bf16x8*)(a + a_row_off + i * 64 * C::RB + co);
          if constexpr (!FP8) {
#pragma unroll
            for (int j = 0; j < 4; ++j) fb[kk][j] = *(const bf16x8*)(b + (brow[j] + frow) * C::RB + co);
          } else if constexpr (K8) {
            // 16 codes (K 32h + 16 fhalf + 0..15) per lane, read once for both MFMAs
            if (kk == 0) {
              const int cb = (((h * 2 + fhalf) ^ swzb) << 4);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const uint4 q = *(const uint4*)(b + (brow[j] + frow) * C::RBB + cb);
                fb[0][j] = make_uint2(q.x, q.y);
                fb[1][j] = make_uint2(q.z, q.w);
              }
            }
          } else {
            // the lane's 8 codes: K offset h*32 + kk*16 + fhalf*8 of the step
            const int bo = (h * 32 + kk * 16 + fhalf * 8) * WBITS / 8;
            const int cb = (((bo >> 4) ^ swzb) << 4) + (bo & 15);
#pragma unroll
            for (int j = 0; j < 4; ++j) fb[kk][j] = *(const BFrag*)(b + (brow[j] + frow) * C::RBB + cb);
          }
        });
      }
    };
    // MFMAs of one slice from (fa, fb) with the reads of slice `next` into
    // (ga, gb) interleaved.  `next` may be past the end: it then rereads a
    // valid stage and the values go unused.
    auto slice = [&](bf16x8 (&fa)[2][NGA], BFrag (&fb)[2][4], int next, bf16x8 (&ga)[2][NGA],
                     BFrag (&gb)[2][4]) __attribute__((always_inline)) {
      if constexpr (NG > 0) {
        read_slice(next < nsl ? next : nsl - 1, ga, gb);
        static_for<2>([&](auto kk) {
          if constexpr (!FP8) {
#pragma unroll
            for (int i = 0; i < NG; ++i)
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                if (MODE == MODE_GATEUP)
                  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk][j], fa[kk][i], acc[i][j], 0, 0, 0);
                else
                  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][i], fb[kk][j], acc[i][j], 0, 0, 0);
              }
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              bf16x8 bv;
              if constexpr (WQ == WQ_INT4) {
                bv = int4x8_to_bf16x8(fb[kk][j]);
                // the row sums ride on the j loop: granule j's fragment
                if (j < NG) rs[j] = int4_rowsum(fa[kk][j], rs[j]);
              } else if constexpr (WQ == WQ_INT8) {
                bv = int8x8_to_bf16x8(fb[kk][j]);
              } else {
                bv = fp8x8_to_bf16x8(fb[kk][j]);
              }
#pragma unroll
              for (int i = 0; i < NG; ++i) {
                if (MODE == MODE_GATEUP)
                  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv, fa[kk][i], acc[i][j], 0, 0, 0);
                else
                  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][i], bv, acc[i][j], 0, 0, 0);
              }
            }
          }
        });
        constexpr int NR = 2 * NG + (K8 ? 4 : 8), NM = 8 * NG, MPR = (NM + NR - 1) / NR;
        static_for<NR>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // one LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, MPR, 0);  // MFMAs
        });
      }
    };
    static_for<NS - 1>([&](auto s) {
      if (s < nk) issue(s, s);
    });
    if (PF != 0 && has_pf && PF < nk)
      wait_vmcnt<2>();
    else if (NS - 2 >= 2 && nk > 2)
      wait_steps(std::integral_constant<int, 2>{});
    else if (NS - 2 >= 1 && nk > 1)
      wait_steps(std::integral_constant<int, 1>{});
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (NS - 1 < nk) issue(NS - 1, (NS - 1) % NS);
    read_slice(0, fa0, fb0);
    // two slices per iteration (fragment buffers 0 and 1); single exit
    int sl = 0;
    for (; sl + 2 <= nsl; sl += 2) {
      if ((sl + 1) % HPS == 0) step_sync(sl + 1);
      slice(fa0, fb0, sl + 1, fa1, fb1);
      if ((sl + 2) % HPS == 0 && sl + 2 < nsl) step_sync(sl + 2);
      slice(fa1, fb1, sl + 2, fa0, fb0);
    }
    if (sl < nsl) slice(fa0, fb0, nsl, fa1, fb1);
  };
  if (nk > 0) {
    if (BMA > 64 && ng >= 4)
      run(std::integral_constant<int, (BMA > 64 ? 4 : 1)>{});
    else if (BMA > 64 && ng == 3)
      run(std::integral_constant<int, (BMA > 64 ? 3 : 1)>{});
    else if (BMA > 64 && ng == 2)
      run(std::integral_constant<int, (BMA > 64 ? 2 : 1)>{});
    else if (ng == 1)
      run(std::integral_constant<int, 1>{});
    else
      run(std::integral_constant<int, 0>{});
  }
  if constexpr (WQ == WQ_INT4) {
    // full row sums (the lane pair l, l ^ 32 holds the two K halves of row
    // l & 31 of each granule), times the widening's offset, per wave in LDS
    __shared__ float s_corr[4][4][32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float full = rs[i] + __shfl_xor(rs[i], 32);
      if (lane < 32) s_corr[wave][i][lane] = kInt4Offset * full;
    }
    __syncthreads();
    store_tile<MODE, FP8, 64, DMA_BM, true, (BMA + 63) / 64, BMA>(p, acc, t, arow0, n0, wn, brow,
                                                      &s_corr[wave][0][0]);
  } else {
    store_tile<MODE, FP8, 64, DMA_BM, false, (BMA + 63) / 64, BMA>(p, acc, t, arow0, n0, wn, brow);
  }
}


// Epilogue of the ping-pong kernel: the wave's NG granules (activation rows
// arow0 + RS i + 0..31) x its two 32-row weight tiles.  MODE_GATEUP
// (transposed product): acc[i][0] / acc[i][1] hold gate / up rows wn*32 + R of
// the weight tile, R = (r / 4) * 8 + (lane / 32) * 4 + r % 4, for activation
// row arow0 + RS i + lane % 32; DOWN*: acc[i][j] holds activation row
// arow0 + RS i + R, output column wn*64 + 32 j + lane % 32.  Quantised
// weights (QS): the per-128-output scales multiply the sums here.  BNB:
// weight rows of the tile (output columns of a partial-tile slab row).
template <int MODE, int NG, bool QS, int RS = 64, int BNB = 256>
__device__ __forceinline__ void store_tile_pp(const GemmParams& p, f32x16 (&acc)[NG][2],
                                              const TileMap& t, int arow0, int n0, int wn) {
  const int lane = threadIdx.x & 63;
  const int ccol = lane & 31;
  const int rbase = (lane >> 5) * 4;
  const int N = p.N;
  const int64_t sbase = t.shared_e ? 0 : (int64_t)t.e * (N / kFp8Group);
  if (MODE == MODE_GATEUP) {
    const int64_t hbase = t.shared_e ? p.P_max : (int64_t)t.seg;
    // the wave's 32 hidden columns share one scale group
    float sg = 1.f, su = 1.f;
    if (QS) {
      const int gi = (n0 + wn * 32) / kFp8Group;
      sg = (t.shared_e ? p.sc0s : p.sc0 + sbase)[gi];
      su = (t.shared_e ? p.sc1s : p.sc1 + sbase)[gi];
    }
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const int m = t.m0 + arow0 + i * RS + ccol;
      if (m >= t.rows) continue;
      uint16_t* hrow = p.H + (hbase + m) * p.h_ld;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 32 + q * 8 + rbase;  // 4 consecutive hidden columns
        if (n >= N) continue;
        if (t.slab >= 0) {  // piece of a split tail tile: gate and up partial sums
          float* sl = p.tail_slab + (int64_t)t.slab * p.slab_piece + (int64_t)(m - t.m0) * BNB + (n - n0);
          *(float4*)sl = make_float4(acc[i][0][q * 4] * sg, acc[i][0][q * 4 + 1] * sg,
                                     acc[i][0][q * 4 + 2] * sg, acc[i][0][q * 4 + 3] * sg);
          *(float4*)(sl + BNB / 2) = make_float4(acc[i][1][q * 4] * su, acc[i][1][q * 4 + 1] * su,
                                             acc[i][1][q * 4 + 2] * su, acc[i][1][q * 4 + 3] * su);
          continue;
        }
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = acc[i][0][q * 4 + r] * sg;
          hv[r] = a / (1.f + __expf(-a)) * (acc[i][1][q * 4 + r] * su);
        }
        store_h4(hrow, n, N, hv, p.h_split);
      }
    }
  } else {
    float sc[2] = {1.f, 1.f};
    if (QS) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + j * 32;
        sc[j] = n < N ? (t.shared_e ? p.sc0s : p.sc0 + sbase)[n / kFp8Group] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < NG; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = t.m0 + arow0 + i * RS + q * 8 + rbase + r;
          if (m >= t.rows) continue;
          float wgt = 1.f;
          int64_t orow;
          if (MODE == MODE_DOWN) {
            if (t.shared_e) {
              orow = m;
              if (p.shared_w) wgt = p.shared_w[m];
            } else {
              orow = p.perm_token[t.seg + m];
              wgt = p.perm_w[t.seg + m];
            }
          } else {
            orow = t.shared_e ? p.P_max + m : (int64_t)t.seg + m;
          }
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 64 + j * 32 + ccol;
            if (n >= N) continue;
            const float v = acc[i][j][q * 4 + r] * sc[j];
            if (MODE == MODE_DOWN)
              atomicAdd(&p.y[orow * N + n], wgt * v);
            else if (t.slab >= 0)
              p.tail_slab[(int64_t)t.slab * p.slab_piece + (int64_t)(m - t.m0) * BNB + (n - n0)] = v;
            else
              p.y_perm[orow * N + n] = v;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Ping-pong kernel: 512 threads = 8 waves, two per SIMD (wave w runs on SIMD
// w % 4), over 256 x 256 tiles or (BMT = 128) tiles of 128 activation rows x
// 512 weight rows.  256-row tiles: wave w computes 128 activation rows (the
// 32-row granules (w & 1) + 2i) x 64 weight rows (quarter w >> 1); 128-row
// tiles: all four granules x 64 weight rows (eighth w).  In MODE_GATEUP a
// wave's 64 weight rows are 32 rows of W1 and the same 32 rows of W3.  Each
// wave alternates a read phase (the fragments of one 32-deep K slice, LDS ->
// registers; 8-bit weight codes are widened exactly to bf16 here) and a
// compute phase (16 MFMAs 32x32x16 on them); waves 4..7 run one phase behind
// waves 0..3, so on every SIMD one wave's MFMAs issue back to back while the
// other's LDS reads and conversions are in flight.  A barrier separates the
// phases.  Operands move global -> LDS by buffer_load ... lds into NS stages
// of 64-deep steps (the XOR-swizzled row layout of DmaCfg).  256-row tiles:
// waves 0..3 fetch the weight tile, waves 4..7 the activation tile; 128-row
// tiles: every wave fetches 64 weight rows and 16 activation rows.  A wave
// issues its loads of step s + NS - 1 during its read of slice 2s (waves
// 4..7 one phase after waves 0..3) and waits for its own loads of a step at
// the end of the phase before that step is first read.  Tile map, K split,
// K rotation and the partial-tile slab are those of grouped_gemm_dma_kernel.
// The 128 x 512 shape serves experts of about 128 rows (a 256-row tile would
// be half empty): per MFMA it moves fewer operand bytes into LDS and widens
// fewer weight codes.
template <int MODE, int WQ, int NS, int BMT = 256>
__global__ __launch_bounds__(512, 1) void grouped_gemm_pp_kernel(GemmParams p) {
  static_assert(WQ == WQ_BF16 || WQ == WQ_FP8 || WQ == WQ_INT8, "bf16 or 8-bit weights");
  static_assert(BMT == 256 || BMT == 128, "activation tile rows");
  constexpr bool QW = WQ != WQ_BF16;  // weight codes with scales
  constexpr int WBITS = wq_bits(WQ);
  constexpr bool WIDE = BMT == 128;
  constexpr int BNB = WIDE ? 512 : 256;  // weight rows of the tile
  using C = DmaCfg<64, NS, WBITS, BMT, BNB>;
  constexpr int NT = 512;
  constexpr int NIB = 64 / C::ROWS_PER_INST_B;   // B DMA instructions per loading wave and step
  constexpr int AROWS = WIDE ? 16 : 64;          // activation rows per loading wave
  constexpr int NIA = AROWS / C::ROWS_PER_INST;  // A DMA instructions per loading wave and step
  constexpr int NV = WIDE ? NIB + NIA : (NIB > NIA ? NIB : NIA);  // most per wave and step
  constexpr int RS = WIDE ? 32 : 64;             // activation rows between a wave's granules
  extern __shared__ __attribute__((aligned(1024))) char dlds[];
  if (p.zero_out) {  // every workgroup clears its share, with or without a tile
    const int64_t n4 = p.zero_n / 4;
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n4; i += (int64_t)gridDim.x * NT)
      ((float4*)p.zero_out)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (blockIdx.x == 0 && (int64_t)threadIdx.x < p.zero_n - n4 * 4) p.zero_out[n4 * 4 + threadIdx.x] = 0.f;
  }
  TileMap t;
  if (!map_tile<MODE, BMT, NT>(p, t)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, widx = wave & 3;
  const int K = p.K, N = p.N, KW = p.kb_len;
  const int kbeg_el = t.kbeg * BK;
  const int nk = (t.nk * BK) / 64;       // 64-deep steps
  const int nkw = KW / 64;              // B's steps (A may hold two terms per unit: wrap)
  const int kbeg_st = kbeg_el / 64;
  const int n0 = (MODE == MODE_GATEUP) ? t.ntile * (BNB / 2) : t.ntile * BNB;
  const int64_t ebytes = (int64_t)N * KW * WBITS / 8;
  const int64_t eoff = t.shared_e ? 0 : (int64_t)t.e * ebytes;

  // ---- DMA.  The wave's weight rows brow0 .. +64 of the B tile (MODE_GATEUP:
  // the first half of the tile's rows are W1 rows, the second half the same
  // rows of W3) and activation rows arow_ld .. +AROWS of the A tile; an
  // instruction fills 1 KiB.
  const bool b_loader = WIDE || grp == 0;
  const bool a_loader = WIDE || grp == 1;
  const int brow0 = (WIDE ? wave : widx) * 64;
  const int arow_ld = (WIDE ? wave : widx) * AROWS;
  const bool w3 = (MODE == MODE_GATEUP) && brow0 >= BNB / 2;
  const void* bsrc = w3 ? (t.shared_e ? p.B1s : p.B1) : (t.shared_e ? p.B0s : p.B0);
  const __amdgpu_buffer_rsrc_t rsB = uniform_rsrc((const char*)bsrc + eoff, ebytes);
  const __amdgpu_buffer_rsrc_t rsA = uniform_rsrc(p.A, p.A_bytes);
  constexpr uint32_t kOobOff = 0x80000000u;
  uint32_t voffb[NIB], voffa[NIA];
#pragma unroll
  for (int j = 0; j < NIB; ++j) {
    const int r = brow0 + j * C::ROWS_PER_INST_B + lane / C::CPRB;  // tile row, 0 .. BNB-1
    const int chunk = (lane % C::CPRB) ^ ((r / C::RPSB) % C::CPRB);
    const int n = (MODE == MODE_GATEUP) ? n0 + (r & (BNB / 2 - 1)) : n0 + r;
    voffb[j] = n < N ? (uint32_t)((int64_t)n * KW * WBITS / 8 + chunk * 16) : kOobOff;
  }
#pragma unroll
  for (int j = 0; j < NIA; ++j) {
    const int r = arow_ld + j * C::ROWS_PER_INST + lane / C::CPR;
    const int chunk = (lane % C::CPR) ^ ((r / C::RPS) % C::CPR);
    const int m = t.m0 + r;
    voffa[j] = m < t.rows ? (uint32_t)((a_row<MODE>(p, t, m) * K + kbeg_el) * 2 + chunk * 16)
                          : kOobOff;
  }
  // activation instructions whose rows all lie past the segment's end are
  // not issued (a prefix of the wave's NIA is)
  const int n_inst_a = a_loader ? __builtin_amdgcn_readfirstlane(max(
                                      0, min(NIA, (t.rows - t.m0 - arow_ld + C::ROWS_PER_INST - 1) /
                                                      C::ROWS_PER_INST)))
                                : 0;
  const int per_step = (b_loader ? NIB : 0) + n_inst_a;  // the wave's loads per step
  // the weight panel of an expert that fits in this one row tile is read by
  // this workgroup only: its loads may stream past L2
  const bool b_nt = p.b_nt && t.rows <= BMT;
  // K rotation: the workgroup walks its K steps from a start of its own
  // (concurrent workgroups then stream different offsets of their rows)
  const int krot = p.krot ? __builtin_amdgcn_readfirstlane(
                                (int)(((uint32_t)blockIdx.x * (uint32_t)p.krot) % (uint32_t)max(nk, 1)))
                          : 0;
  auto issue = [&](int kt) __attribute__((always_inline)) {
    char* sbase = dlds + (kt % NS) * C::STAGE_BYTES;
    const int kr = kt + krot < nk ? kt + krot : kt + krot - nk;
    int kb = kbeg_st + kr;
    kb = kb >= nkw ? kb - nkw : kb;
    if (b_loader) {
      char* dst = sbase + C::TILE_BYTES + brow0 * C::RBB;
      const int soff = __builtin_amdgcn_readfirstlane(kb * C::RBB);
      // the streaming hint on the step that reads the last part of each
      // 128-byte weight line (every step for bf16 rows)
      if (b_nt && (C::RBB >= 128 || (kb + 1) % (128 / C::RBB) == 0))
        static_for<NIB>([&](auto j) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_ptr_t)(dst + j * 1024), 16, voffb[j],
                                                   soff, 0, kAuxStream);
        });
      else
        static_for<NIB>([&](auto j) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_ptr_t)(dst + j * 1024), 16, voffb[j],
                                                   soff, 0, 1);
        });
    }
    if (a_loader) {
      char* dst = sbase + arow_ld * C::RB;
      const int soff = __builtin_amdgcn_readfirstlane(kr * C::RB);
      static_for<NIA>([&](auto j) {
        if (j < n_inst_a)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_ptr_t)(dst + j * 1024), 16, voffa[j],
                                                   soff, 0, 1);
      });
    }
  };
  // "every load of step u has landed": the loads of the later steps issued
  // so far (up to step min(u + NS - 2, nk - 1)) may stay in flight
  auto wait_step = [&](int u) __attribute__((always_inline)) {
    const int later = min(u + NS - 2, nk - 1) - u;
    if (NS == 2 || later <= 0)
      wait_vmcnt<0>();
    else
      wait_vmcnt_dyn<NV * (NS - 2)>(later * per_step);
  };

  // ---- the wave's tile
  const int wm = WIDE ? 0 : (wave & 1), wn = WIDE ? wave : (wave >> 1);
  const int frow = lane & 31, fhalf = lane >> 5;
  const int swz = (frow / C::RPS) % C::CPR;     // fragment rows are 32-aligned + frow
  const int swzb = (frow / C::RPSB) % C::CPRB;
  const int arow0 = wm * 32;
  int b_row[2];
  b_row[0] = (MODE == MODE_GATEUP) ? wn * 32 + frow : wn * 64 + frow;
  b_row[1] = (MODE == MODE_GATEUP) ? BNB / 2 + wn * 32 + frow : wn * 64 + 32 + frow;
  const int vg = min(BMT / 32, (t.rows - t.m0 + 31) / 32);  // valid granules of the tile
  const int ng = __builtin_amdgcn_readfirstlane(WIDE ? vg : (vg > wm ? (vg - wm + 1) / 2 : 0));

  if (nk <= 0) return;  // (every unit of the schedule has at least one step)
  // prologue: steps 0 .. NS - 2 in flight, wait for step 0
  static_for<NS - 1>([&](auto u) {
    if (u < nk) issue(u);
  });
  wait_step(0);
  __builtin_amdgcn_s_barrier();

  auto bar = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto run = [&](auto NGc) __attribute__((always_inline)) {
    constexpr int NG = decltype(NGc)::value;
    constexpr int NGA = NG > 0 ? NG : 1;
    f32x16 acc[NGA][2];
#pragma unroll
    for (int i = 0; i < NGA; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    bf16x8 fa[2][NGA], fb[2][2];
    using BCode = std::conditional_t<QW, uint2, bf16x8>;
    BCode fq[2][2];
    const int nsl = nk * 2;
    int stage = 0;  // st % NS
    if (grp == 1) bar();
    for (int sl = 0; sl < nsl; ++sl) {
      // read phase: slice sl (with, on even slices, the DMA of step st + NS - 1)
      const int st = sl >> 1;
      if ((sl & 1) == 0 && st + NS - 1 < nk) issue(st + NS - 1);
      if constexpr (NG > 0) {
        const char* a = dlds + stage * C::STAGE_BYTES;
        const char* b = a + C::TILE_BYTES;
        static_for<2>([&](auto kk) {
          // 8-bit codes: K permuted within the slice as in grouped_gemm_dma_kernel
          // (MFMA kk, lane half g: K positions 32h + 16g + 8kk + 0..7), so one
          // 16-byte read of codes serves both MFMAs
          const int co = QW ? (((((sl & 1) * 4 + fhalf * 2 + kk) ^ swz) * 16))
                            : (((((sl & 1) * 4 + kk * 2 + fhalf) ^ swz) * 16));
#pragma unroll
          for (int i = 0; i < NG; ++i)
            fa[kk][i] = *(const bf16x8*)(a + (arow0 + i * RS + frow) * C::RB + co);
          if constexpr (!QW) {
#pragma unroll
            for (int j = 0; j < 2; ++j) fq[kk][j] = *(const bf16x8*)(b + b_row[j] * C::RBB + co);
          } else if (kk == 0) {
            // the lane's 16 codes: K offset (sl & 1) * 32 + fhalf * 16 of the step
            const int cb = ((((sl & 1) * 2 + fhalf) ^ swzb) << 4);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const uint4 q = *(const uint4*)(b + b_row[j] * C::RBB + cb);
              fq[0][j] = make_uint2(q.x, q.y);
              fq[1][j] = make_uint2(q.z, q.w);
            }
          }
        });
      }
      wait_lgkm0();
      if constexpr (NG > 0) {
        static_for<2>([&](auto kk) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if constexpr (WQ == WQ_FP8)
              fb[kk][j] = fp8x8_to_bf16x8(fq[kk][j]);
            else if constexpr (WQ == WQ_INT8)
              fb[kk][j] = int8x8_to_bf16x8(fq[kk][j]);
            else
              fb[kk][j] = fq[kk][j];
          }
        });
      }
      // activation loaders: their loads of step st + 1 have landed before
      // slice sl + 1 = 2 (st + 1) is read
      if (grp == 1 && (sl & 1) && st + 1 < nk) wait_step(st + 1);
      bar();
      // compute phase
      if constexpr (NG > 0) {
        static_for<2>([&](auto kk) {
#pragma unroll
          for (int i = 0; i < NG; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              if (MODE == MODE_GATEUP)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk][j], fa[kk][i], acc[i][j], 0, 0, 0);
              else
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][i], fb[kk][j], acc[i][j], 0, 0, 0);
            }
        });
      }
      // weight loaders: the same, at the end of their compute phase
      if (grp == 0 && (sl & 1) && st + 1 < nk) wait_step(st + 1);
      if (sl & 1) stage = stage + 1 == NS ? 0 : stage + 1;
      bar();
    }
    if (grp == 0) bar();
    if constexpr (NG > 0) store_tile_pp<MODE, NG, QW, RS, BNB>(p, acc, t, arow0, n0, wn);
  };
  if (ng >= 4)
    run(std::integral_constant<int, 4>{});
  else if (ng == 3)
    run(std::integral_constant<int, 3>{});
  else if (ng == 2)
    run(std::integral_constant<int, 2>{});
  else if (ng == 1)
    run(std::integral_constant<int, 1>{});
  else
    run(std::integral_constant<int, 0>{});
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

// Tail fixup: the pieces of a split tail tile left fp32 partial tiles in
// p.tail_slab (GATEUP: [row][128 gate | 128 up] sums, already scaled;
// DOWN_PERM: [row][256 outputs]); sum them in piece order and finish the
// tile's valid rows (GATEUP: SwiGLU into H; DOWN_PERM: the grouped output).
// One workgroup per band of 16 rows (BM / 16 bands per tile, at most
// kFixBands): workgroup b is XCD b % 8, then (tail tile, band) of b / 8 (the
// same schedule arithmetic as the GEMM, from the same offsets).
constexpr int kFixBands = 16;
template <int MODE, int BM>
__global__ __launch_bounds__(256) void tail_fixup_kernel(GemmParams p) {
  constexpr int ROWS = DMA_BM / kFixBands;  // rows per band (16)
  __shared__ int s_scan[4];
  __shared__ int s_pre[kMaxSegments + 1];
  constexpr int NB = BM / ROWS < kFixBands ? BM / ROWS : kFixBands;  // bands of a tile
  const int xcd = (int)(blockIdx.x % kNumXcd);
  const int r = (int)(blockIdx.x / kNumXcd / NB);
  const int band = (int)(blockIdx.x / kNumXcd % NB);
  const int Mreal = seg_prefix<BM>(p, s_pre, s_scan);
  int64_t qtail = 0;
  int rem = 0, S = 1;
  sched_tail_of_xcd((int64_t)Mreal * p.nt, xcd, p.slots, p.split_max, qtail, rem, S);
  if (r >= rem || S <= 1) return;
  TileMap t;
  tile_place<BM>(p, s_pre, qtail + r, t);
  if (band * ROWS >= t.rows - t.m0) return;  // the band holds no rows of the segment
  const float* slab = p.tail_slab + (int64_t)(xcd * p.slots + r * S) * p.slab_piece;
  const int64_t obase = (t.shared_e ? p.P_max : (int64_t)t.seg) + t.m0;
  // ROWS x 256 floats per band: 16 rows x 64 float4 = 4 float4 per thread;
  // GATEUP pairs the gate float4 at column c with the up float4 at c + 128
  constexpr int NV = (MODE == MODE_GATEUP) ? 2 : 4;
  float4 a[NV], u[NV];
  int row[NV], col[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int it = v * 256 + (int)threadIdx.x;  // GATEUP: 16 rows x 32 float4 of gate
    row[v] = band * ROWS + (MODE == MODE_GATEUP ? it / 32 : it / 64);
    col[v] = (MODE == MODE_GATEUP ? it % 32 : it % 64) * 4;
    const float* src = slab + row[v] * 256 + col[v];
    a[v] = *(const float4*)src;
    if (MODE == MODE_GATEUP) u[v] = *(const float4*)(src + 128);
  }
  for (int pc = 1; pc < S; ++pc) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const float* src = slab + (int64_t)pc * p.slab_piece + row[v] * 256 + col[v];
      const float4 b = *(const float4*)src;
      a[v].x += b.x; a[v].y += b.y; a[v].z += b.z; a[v].w += b.w;
      if (MODE == MODE_GATEUP) {
        const float4 c = *(const float4*)(src + 128);
        u[v].x += c.x; u[v].y += c.y; u[v].z += c.z; u[v].w += c.w;
      }
    }
  }
  const int n0 = (MODE == MODE_GATEUP) ? t.ntile * 128 : t.ntile * 256;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    if (t.m0 + row[v] >= t.rows || n0 + col[v] >= p.N) continue;
    if (MODE == MODE_GATEUP) {
      const float g[4] = {a[v].x, a[v].y, a[v].z, a[v].w};
      const float up[4] = {u[v].x, u[v].y, u[v].z, u[v].w};
      float hv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) hv[q] = g[q] / (1.f + __expf(-g[q])) * up[q];
      store_h4(p.H + (obase + row[v]) * p.h_ld, n0 + col[v], p.N, hv, p.h_split);
    } else {
      *(float4*)(p.y_perm + (obase + row[v]) * p.N + n0 + col[v]) = a[v];
    }
  }
}

// Combine: y[t] = sum over kept j (in slot order) of topk_w[t, j] *
// y_perm[slot_pos[t, j]], then + sw * y_shared[t] when there is a shared
// expert, with sw = 1, or with overflow to the shared expert 1 + the token's
// dropped weights (summed in slot order).  One thread per 4 consecutive
// outputs when d % 4 == 0.
template <int V>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const float* __restrict__ y_shared,
                                                      const int32_t* __restrict__ slot_pos,
                                                      const float* __restrict__ topk_w,
                                                      float* __restrict__ y, int64_t T, int k,
                                                      int d, int shared_overflow) {
  const int dv = d / V;
  const int64_t n = T * dv;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / dv;
    const int c = (int)(i - t * dv) * V;
    float acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = 0.f;
    float sw = 1.f;
    for (int j = 0; j < k; ++j) {
      const int32_t pos = slot_pos[t * k + j];
      const float w = topk_w[t * k + j];
      if (pos < 0) {
        sw += w;  // used only with overflow to the shared expert
        continue;
      }
      const float* src = y_perm + (int64_t)pos * d + c;
      if constexpr (V == 4) {
        const float4 v4 = *(const float4*)src;
        acc[0] += w * v4.x; acc[1] += w * v4.y; acc[2] += w * v4.z; acc[3] += w * v4.w;
      } else {
        acc[0] += w * src[0];
      }
    }
    if (y_shared) {
      const float* src = y_shared + t * d + c;
      if (!shared_overflow) sw = 1.f;
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] += sw * src[v];
    }
    if constexpr (V == 4)
      *(float4*)(y + t * d + c) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    else
      y[t * d + c] = acc[0];
  }
}

// Workgroups one XCD runs at once for a kernel of 256 threads and `lds`
// bytes of LDS (after its LDS opt-in) on device `dev`.
int xcd_slots(const void* kernel, size_t lds, int dev) {
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, 256, lds) != hipSuccess)
    occ = 1;
  return std::max(1, device_cus(dev) / kNumXcd) * std::max(1, occ);
}

// Per-device launch facts of one kernel instantiation (its LDS opt-in and
// the workgroups an XCD runs at once), set up once per device.
struct KernelSlots {
  std::once_flag once[kMaxDevices];
  hipError_t err[kMaxDevices] = {};
  int slots[kMaxDevices] = {};
};

// Grid of the tile schedule: kNumXcd x the bound of any XCD's units.
inline unsigned sched_grid(const GemmParams& p) {
  return (unsigned)(kNumXcd * sched_units_bound((int64_t)p.mt_max * p.nt, p.slots));
}


// The LDS-DMA kernel: KB-deep K steps in NS stages over tiles of BMA
// activation rows (launch_gemm picks the shape).  Two 64-deep stages keep
// one step in flight while one is computed, with few barriers per K; tiles
// with few rows have little compute to hide the operand latency behind and
// take smaller activation tiles, which leave LDS for more stages or a second
// workgroup per CU.
template <int MODE, int WQ, int KB, int NS, int BMA = 256, int PF = 0>
hipError_t launch_gemm_dma(const GemmParams& p0, hipStream_t st) {
  if (p0.mt_max <= 0 || p0.nt <= 0) return hipSuccess;
  using C = DmaCfg<KB, NS, wq_bits(WQ), BMA>;
  constexpr size_t kLds = C::LDS + (PF ? kPfSinkBytes : 0);
  const void* kern = (const void*)grouped_gemm_dma_kernel<MODE, KB, NS, 1, WQ, BMA, PF>;
  static KernelSlots ks;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(ks.once[dev], [&] {
    ks.err[dev] = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
    if (ks.err[dev] == hipSuccess) ks.slots[dev] = xcd_slots(kern, kLds, dev);
  });
  if (ks.err[dev] != hipSuccess) return ks.err[dev];
  const int slots = ks.slots[dev];
  GemmParams p = p0;
  p.kunit = KB / BK;
  p.slots = slots;
  p.slab_piece = BMA * 256;
  constexpr bool slab_mode = (MODE == MODE_DOWN_PERM || MODE == MODE_GATEUP);
  if (slab_mode && (!p.tail_slab || (int64_t)kNumXcd * slots * p.slab_piece > p.slab_floats))
    p.split_max = 1;
  // row tiles of BMA rows: sum_e ceil(rows_e / BMA) <= P_max / BMA + E (+ shared)
  p.mt_max = (int)((p.P_max + BMA - 1) / BMA + p.E + (p.has_shared ? (p.T + BMA - 1) / BMA : 0));
  grouped_gemm_dma_kernel<MODE, KB, NS, 1, WQ, BMA, PF><<<sched_grid(p), 256, kLds, st>>>(p);
  if (slab_mode && p.split_max > 1)
    // split tail tiles exist only with S >= 2 pieces, so rem <= slots / 2 of
    // them per XCD; bands past BMA rows hold nothing
    tail_fixup_kernel<MODE, BMA><<<(unsigned)(kNumXcd * std::max(1, slots / 2) *
                                              std::min(kFixBands, BMA / (DMA_BM / kFixBands))),
                                   256, 0, st>>>(p);
  return hipGetLastError();
}



// The ping-pong kernel: 512 threads, NS 64-deep stages (256 x 256 tiles:
// bf16 weights two stages of 64 KiB, 8-bit weights three of 48 KiB; 128 x 512
// tiles, 8-bit weights only: three stages of 48 KiB).  The 128 x 512 shape
// takes no K split of tail tiles.
template <int MODE, int WQ, int NS, int BMT = 256>
hipError_t launch_gemm_pp(const GemmParams& p0, hipStream_t st) {
  if (p0.mt_max <= 0 || p0.nt <= 0) return hipSuccess;
  constexpr int BNB = BMT == 128 ? 512 : 256;
  using C = DmaCfg<64, NS, wq_bits(WQ), BMT, BNB>;
  constexpr size_t kLds = C::LDS;
  const void* kern = (const void*)grouped_gemm_pp_kernel<MODE, WQ, NS, BMT>;
  static KernelSlots ks;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(ks.once[dev], [&] {
    ks.err[dev] = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
    if (ks.err[dev] == hipSuccess) {
      int occ = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, 512, kLds) != hipSuccess) occ = 1;
      ks.slots[dev] = std::max(1, device_cus(dev) / kNumXcd) * std::max(1, occ);
    }
  });
  if (ks.err[dev] != hipSuccess) return ks.err[dev];
  const int slots = ks.slots[dev];
  GemmParams p = p0;
  p.kunit = 64 / BK;
  p.slots = slots;
  p.slab_piece = BMT * BNB;
  if (WQ == WQ_BF16 || !MOE_PP_KROT) p.krot = 0;
  if (BMT != 256) {
    // weight tiles of the wider shape; no tail split (the fixup pass sums
    // 256-column pieces)
    p.nt = (MODE == MODE_GATEUP) ? (p.N + BNB / 2 - 1) / (BNB / 2) : (p.N + BNB - 1) / BNB;
    p.split_max = 1;
  }
  constexpr bool slab_mode = (MODE == MODE_DOWN_PERM || MODE == MODE_GATEUP);
  if (slab_mode && (!p.tail_slab || (int64_t)kNumXcd * slots * p.slab_piece > p.slab_floats))
    p.split_max = 1;
  p.mt_max = (int)((p.P_max + BMT - 1) / BMT + p.E + (p.has_shared ? (p.T + BMT - 1) / BMT : 0));
  grouped_gemm_pp_kernel<MODE, WQ, NS, BMT><<<sched_grid(p), 512, kLds, st>>>(p);
  if (slab_mode && p.split_max > 1)
    tail_fixup_kernel<MODE, 256><<<(unsigned)(kNumXcd * std::max(1, slots / 2) * kFixBands), 256, 0,
                                   st>>>(p);
  return hipGetLastError();
}

// Runtime weight format and pipeline shape -> the kernel instantiation.
template <int MODE>
// rows: the average rows per expert (decode-sized batches: 32 or fewer).
hipError_t launch_gemm(int wq, int64_t rows, const GemmParams& p, hipStream_t st) {
  const bool deep = rows <= 32;
  if (deep) {
    // 64-row activation tiles: a smaller LDS footprint, so two workgroups
    // share a CU.  Quantised weights with 64-deep steps in three stages
    // (measured at 16 rows per expert against 256-row tiles with 32-deep
    // steps: the fp8 layer 0.598 -> 0.362 ms, int4 0.38 -> 0.30 ms); bf16
    // weights with 32-deep ones (0.591 -> 0.582 ms; 64-deep steps, which
    // leave room for one workgroup per CU only, were slower there)
    if (wq == WQ_FP8) return launch_gemm_dma<MODE, WQ_FP8, 64, 3, 64>(p, st);
    if (wq == WQ_INT8) return launch_gemm_dma<MODE, WQ_INT8, 64, 3, 64>(p, st);
    if (wq == WQ_INT4) return launch_gemm_dma<MODE, WQ_INT4, 64, 3, 64>(p, st);
    // bf16 weights at 16 or fewer rows per expert: 32-row tiles with two
    // 64-deep stages, two workgroups per CU (decode at 16 rows per expert
    // 0.576 -> 0.542 ms)
    if (rows <= 16) return launch_gemm_dma<MODE, WQ_BF16, 64, MOE_DECODE_NS, 32, MOE_DECODE_PF>(p, st);
    return launch_gemm_dma<MODE, WQ_BF16, 32, 3, 64>(p, st);
  }
  // 8-bit weights: the ping-pong kernel on 256 x 256 tiles when experts fill
  // whole 256-row tiles; with about 128 rows per expert the half-empty
  // tiles make its phases short and their barriers dominate (measured on the
  // 256-expert layer: fp8 6.41 ms with the four-wave kernel against 7.26 ms).
  // There its 128 x 512 shape keeps the phases full: the down projection
  // 2.75 -> 2.46 ms (fp8), 2.87 -> 2.64 ms (int8); not the gate/up
  // projection (3.55 -> 4.0 ms), which keeps the four-wave kernel
  // (MOE_PP8_WIDE: bit 1 << MODE per launch).  For that kernel, 128-row
  // activation tiles (two, three or four stages) and three stages of 256
  // rows measured slower (3.63 -> 4.9..5.2 and 3.9 ms)
  const bool pp8 = MOE_GEMM_PP && rows >= MOE_PP8_ROWS;
  const bool pp8w = MOE_GEMM_PP && ((MOE_PP8_WIDE >> MODE) & 1) && !pp8;
  if (wq == WQ_FP8)
    return pp8    ? launch_gemm_pp<MODE, WQ_FP8, 3>(p, st)
           : pp8w ? launch_gemm_pp<MODE, WQ_FP8, 3, 128>(p, st)
                  : launch_gemm_dma<MODE, WQ_FP8, 64, 2>(p, st);
  if (wq == WQ_INT8)
    return pp8    ? launch_gemm_pp<MODE, WQ_INT8, 3>(p, st)
           : pp8w ? launch_gemm_pp<MODE, WQ_INT8, 3, 128>(p, st)
                  : launch_gemm_dma<MODE, WQ_INT8, 64, 2>(p, st);
  if (wq == WQ_INT4) return launch_gemm_dma<MODE, WQ_INT4, 64, 2>(p, st);
  if (MOE_GEMM_PP) return launch_gemm_pp<MODE, WQ_BF16, 2>(p, st);
  return launch_gemm_dma<MODE, WQ_BF16, 64, 2, 256, MOE_GEMM_PF>(p, st);
}

}  // namespace

int device_cus(int dev) {
  static std::once_flag once[kMaxDevices];
  static int cus[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(once[dev], [&] {
    int n = 0;
    cus[dev] = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                n > 0)
                   ? n
                   : 256;
  });
  return cus[dev];
}

int current_device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  return device_cus(dev);
}

size_t gemm_slab_floats(const moe_shape& s, int64_t P_max) {
  if (s.kind != MOE_EXPERT_SWIGLU || s.E <= 0) return 0;
  // the launches that may split tail tiles through the slab: gate/up for
  // d >= 4096, the grouped-output down projection for d_ff >= 4096
  if (s.d < 4096 && s.d_ff < 4096) return 0;
  const int64_t rows_avg = P_max / s.E;
  // activation-tile rows and workgroups per CU of launch_gemm's choice
  int bma = 256, per_cu = 1;
  if (rows_avg <= 32) {
    bma = (s.w_dtype == MOE_DT_BF16 && rows_avg <= 16) ? 32 : 64;
    per_cu = 2;
  }
  const int cus = current_device_cus();
  return (size_t)kNumXcd * std::max(1, cus / kNumXcd) * per_cu * bma * 256;
}

hipError_t launch_expert_ffn(const moe_shape& s, const WsLayout& L, const moe_weights& w,
                             const void* x, const int32_t* offsets, const int32_t* perm_token,
                             const float* perm_w, float* y_perm, float* y, void* H,
                             hipStream_t st, hipEvent_t ev_mid, const float* shared_w,
                             bool zero_y) {
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
  const int wq = s.w_dtype == MOE_DT_FP8_E4M3 ? WQ_FP8
                 : s.w_dtype == MOE_DT_INT8   ? WQ_INT8
                 : s.w_dtype == MOE_DT_INT4   ? WQ_INT4
                                              : WQ_BF16;
  const int has_sh = s.has_shared ? 1 : 0;
  float* tail_slab = (H && L.slab_floats) ? (float*)((char*)H + (L.off_slab - L.off_H)) : nullptr;
  // Upper bound of row tiles: sum_e ceil(rows_e / BM) <= P_max / BM + E (+ shared).
  constexpr int BM = DMA_BM;
  const int64_t mt_bound = (L.P_max + BM - 1) / BM + s.E + (has_sh ? (s.T + BM - 1) / BM : 0);

  GemmParams g{};
  g.perm_token = perm_token;
  g.perm_w = perm_w;
  g.offsets = offsets;
  g.T = s.T;
  g.P_max = L.P_max;
  g.E = s.E;
  g.has_shared = has_sh;
  g.mt_max = (int)mt_bound;
  g.tail_slab = tail_slab;
  g.slab_floats = L.slab_floats;
  g.group_n = MOE_SCHED_GN;  // weight tiles per expert-aligned block of the tile order
  g.nfast = MOE_SCHED_NFAST;

  // gate / up (it also clears y for the atomic combine when asked)
  if (zero_y && y) {
    g.zero_out = y;
    g.zero_n = s.T * (int64_t)s.d;
  }
  g.A = (const uint16_t*)x;
  g.A_bytes = s.T * (int64_t)s.d * 2;
  g.B0 = w.W1; g.B1 = w.W3; g.B0s = w.W1s; g.B1s = w.W3s;
  g.sc0 = w.s1; g.sc1 = w.s3; g.sc0s = w.s1s; g.sc1s = w.s3s;
  g.H = (uint16_t*)H;
  g.K = s.d;
  g.kb_len = s.d;
  g.N = s.d_ff;
  g.h_split = s.hidden_split ? 1 : 0;
  g.h_ld = s.d_ff * (g.h_split ? 2 : 1);
  const int bn1 = 128;  // hidden columns per gate/up tile (128 of W1 + 128 of W3)
  g.nt = (s.d_ff + bn1 - 1) / bn1;
  // tail tiles split over K through the slab + fixup (SwiGLU needs whole
  // sums), for long K loops only, as in the down projection
  g.split_max = s.d >= 4096 ? std::max(1, s.d / BK / 8) : 1;
  if (!MOE_DECODE_GU_SPLIT && L.P_max / s.E <= 32) g.split_max = 1;
  // few rows per expert (decode-sized batches): smaller activation tiles and
  // deeper weight pipelines (launch_gemm; slower at 128 rows and more)
  const int64_t rows_avg = L.P_max / s.E;
  const bool deep = rows_avg <= 32;
  // 8-bit weights outside decode-sized batches: K rotation (measured on the
  // 256-expert layer: 5-6% faster for fp8 and int8, neutral for int4, slower
  // for bf16 weights and for decode-sized batches)
  g.krot = (!deep && (wq == WQ_FP8 || wq == WQ_INT8)) ? 7 : 0;
  // bf16 weight panels read by a single row tile (the tile's expert has no
  // more rows than the tile; decided per tile on the device): their loads
  // stream past L2.  Measured: the 256-expert layer 5.94 -> 5.72 ms, decode
  // at 16 rows per expert 0.525 -> 0.485 ms; applied to all tiles of the
  // Mixtral-shaped layer (four row tiles per expert) 2.5% slower.  Not for
  // 8-bit or 4-bit codes: a 64-deep step reads only part of each 128-byte
  // line, and the next step finds the rest in L2 only if the line stayed
  // (fp8 256-expert layer 6.14 -> 7.35 ms, decode 0.32 -> 0.43 ms with the
  // streaming hint on every step; on the step that reads a line's last part
  // only, no change either way)
  g.b_nt = (wq == WQ_BF16 && MOE_B_NT) ? 1 : 0;
  hipError_t err = launch_gemm<MODE_GATEUP>(wq, rows_avg, g, st);
  if (err != hipSuccess) return err;
  if (ev_mid) {
    err = hipEventRecord(ev_mid, st);
    if (err != hipSuccess) return err;
  }

  // down (+ combine)
  GemmParams g2 = g;
  g2.zero_out = nullptr;
  g2.zero_n = 0;
  g2.A = (const uint16_t*)H;
  g2.A_bytes = L.H_rows * (int64_t)g.h_ld * 2;
  g2.B0 = w.W2; g2.B1 = nullptr; g2.B0s = w.W2s; g2.B1s = nullptr;
  g2.sc0 = w.s2; g2.sc1 = nullptr; g2.sc0s = w.s2s; g2.sc1s = nullptr;
  g2.H = nullptr;
  g2.y = y;
  g2.y_perm = y_perm;
  g2.shared_w = shared_w;
  g2.K = g.h_ld;  // hi | lo: K = 2 d_ff over the same W2 rows
  g2.kb_len = s.d_ff;
  g2.N = s.d;
  g2.h_split = 0;
  const int bn2 = 256;  // output columns per down tile
  g2.nt = (s.d + bn2 - 1) / bn2;
  g2.mt_max = (int)mt_bound;
  // The tiles of the last, partial round of the schedule may be split over K
  // (pieces of at least 8 steps): with the atomic combine the partial sums
  // add up in y; with the grouped output they go to the tail slab and a
  // fixup pass sums them, which pays only for long K loops (measured: a loss
  // at d_ff = 1408 and 2048, a gain at 14336).
  g2.split_max = (y || s.d_ff >= 4096) ? std::max(1, s.d_ff / BK / 8) : 1;
  g2.tail_slab = tail_slab;
  g2.slab_floats = L.slab_floats;
  if (y)
    return launch_gemm<MODE_DOWN>(wq, rows_avg, g2, st);
  return launch_gemm<MODE_DOWN_PERM>(wq, rows_avg, g2, st);
}

hipError_t launch_combine(const moe_shape& s, int64_t P_max, const float* y_perm,
                          const int32_t* slot_pos, const float* topk_w, float* y,
                          hipStream_t st) {
  const float* y_shared = s.has_shared ? y_perm + P_max * (int64_t)s.d : nullptr;
  const int sh_ovf = (s.has_shared && s.overflow == MOE_OVERFLOW_SHARED) ? 1 : 0;
  const int V = (s.d % 4 == 0) ? 4 : 1;
  const int64_t n = s.T * (int64_t)(s.d / V);
  const unsigned blocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 16384));
  if (V == 4)
    combine_kernel<4><<<blocks, 256, 0, st>>>(y_perm, y_shared, slot_pos, topk_w, y, s.T, s.top_k, s.d,
                                              sh_ovf);
  else
    combine_kernel<1><<<blocks, 256, 0, st>>>(y_perm, y_shared, slot_pos, topk_w, y, s.T, s.top_k, s.d,
                                              sh_ovf);
  return hipGetLastError();
}

}  // namespace moe
