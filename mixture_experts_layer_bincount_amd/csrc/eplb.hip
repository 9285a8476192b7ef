// Expert placement with hot-expert replication, computed on the device from
// the step's per-expert counts (no host round trip).
//
// fde-learning "MoE 并行" (通信瓶颈的缓解策略, Expert 复制: a popular expert
// gets a copy on several GPUs) and the adv12 MoE + EPLB tutorial (§3.3 /
// §4.3: LPT packing, heaviest expert first onto the lightest device; §5: the
// online EPLB runs from measured loads):
//   1. every expert has one replica; each of `extra` more goes to the expert
//      with the largest load per replica (compared exactly through
//      fixed-point keys, see rep_key; equal: the lower expert), at most D
//      per expert;
//   2. an expert's tokens split evenly over its replicas (the first
//      load % r replicas take one more); slots are numbered expert by expert;
//   3. LPT over the slots: heaviest first (equal: lower expert, then lower
//      replica), each to the lightest device not yet holding a copy of the
//      same expert (equal: lower device).
// One workgroup of 1024 threads: phase 1 is a block arg-max per extra
// replica, phase 3 ranks the slots by counting (every slot compares itself
// with all others), phase 4 is a sequential walk of the ranked slots by one
// wave whose lanes hold the device loads.  The wave reductions use DPP, so
// each sequential step costs a few dozen cycles rather than LDS round trips.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kEplbMaxE = 1024;
constexpr int kEplbMaxSlots = 2048;

// Wave-wide max / min of a 64-bit key with DPP row shifts and row
// broadcasts (no LDS round trips): after row_shr 1, 2, 4, 8 lane 15 of each
// row of 16 holds the row's extreme, row_bcast 15 and 31 fold the rows, and
// lane 63 ends with the wave's.  Lanes whose DPP source is out of range keep
// the identity.  Returns the result in every lane.
template <bool MAX>
__device__ __forceinline__ uint64_t dpp_step(uint64_t v, int lo_in, int hi_in) {
  const uint64_t o = ((uint64_t)(uint32_t)hi_in << 32) | (uint32_t)lo_in;
  return MAX ? (o > v ? o : v) : (o < v ? o : v);
}

template <bool MAX>
__device__ __forceinline__ uint64_t wave_reduce_u64(uint64_t v) {
  const int idl = MAX ? 0 : -1;  // identity halves: 0 for max, all ones for min
#define MOE_DPP(CTRL, ROWMASK)                                                              \
  v = dpp_step<MAX>(v, __builtin_amdgcn_update_dpp(idl, (int)(uint32_t)v, CTRL, ROWMASK, 0xF, false), \
                    __builtin_amdgcn_update_dpp(idl, (int)(uint32_t)(v >> 32), CTRL, ROWMASK, 0xF, false))
  MOE_DPP(0x111, 0xF);  // row_shr:1
  MOE_DPP(0x112, 0xF);  // row_shr:2
  MOE_DPP(0x114, 0xF);  // row_shr:4
  MOE_DPP(0x118, 0xF);  // row_shr:8
  MOE_DPP(0x142, 0xA);  // row_bcast:15 into rows 1 and 3
  MOE_DPP(0x143, 0xC);  // row_bcast:31 into rows 2 and 3
#undef MOE_DPP
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Wave-wide minimum of a 32-bit key over the first 16, 32 or 64 lanes
// (n_lanes rounded up to one of them; the others are not read), returned
// in every lane.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v, int n_lanes) {
#define MOE_DPP_MIN(CTRL, ROWMASK) \
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, CTRL, ROWMASK, 0xF, false))
  MOE_DPP_MIN(0x111, 0xF);  // row_shr:1
  MOE_DPP_MIN(0x112, 0xF);  // row_shr:2
  MOE_DPP_MIN(0x114, 0xF);  // row_shr:4
  MOE_DPP_MIN(0x118, 0xF);  // row_shr:8
  if (n_lanes <= 16) return __builtin_amdgcn_readlane((int)v, 15);
  MOE_DPP_MIN(0x142, 0xA);  // row_bcast:15 into rows 1 and 3
  if (n_lanes <= 32) return __builtin_amdgcn_readlane((int)v, 31);
  MOE_DPP_MIN(0x143, 0xC);  // row_bcast:31 into rows 2 and 3
#undef MOE_DPP_MIN
  return __builtin_amdgcn_readlane((int)v, 63);
}

// Replication key of expert e with load l and r replicas: larger = more
// deserving.  floor(l * 4096 / r) orders the loads per replica exactly
// (r <= 64, so two different quotients differ by at least 1/4096, and equal
// quotients give equal floors); the low 10 bits put the lower expert first
// among equals.  0 = not a candidate.
__device__ __forceinline__ uint64_t rep_key(int64_t l, int r, int e) {
  return (((uint64_t)((l << 12) / r) + 1) << 10) | (uint64_t)(1023 - e);
}

// The LPT walk, run by one wave: lane d holds device d's load.  The slot
// keys come 64 at a time into the lanes and are read out uniformly
// (readlane), so the only LDS round trip left per slot is the used-device
// mask of an expert's second and later copies (an expert's copies come in
// replica order: their loads differ by at most one, the heavier first, so
// copy 0 never meets a used device).  The arg-min over the devices without
// a copy of the slot's expert is the minimum of (load << 6 | device), so
// equal loads go to the lower device.  NARROW: every device load < 2^26,
// 32-bit keys.
template <bool NARROW>
__device__ __forceinline__ void lpt_walk(const uint64_t* s_sorted, int S, int D, int lane,
                                         uint64_t* s_used, uint8_t* s_bd,
                                         int64_t* __restrict__ device_load) {
  uint64_t dl = 0;
  for (int p0 = 0; p0 < S; p0 += 64) {
    const uint64_t kb = p0 + lane < S ? s_sorted[p0 + lane] : 0;
    const int n = min(64, S - p0);
    for (int j = 0; j < n; ++j) {
      const uint64_t k = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(kb >> 32), j) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)kb, j);
      const int se = (int)((k >> 6) & 1023);
      const int si = (int)(k & 63);
      const uint64_t sl = 0x7FFFFFFFull - (k >> 16);
      const uint64_t used = si > 0 ? s_used[se] : 0ull;
      const bool ok = lane < D && !((used >> lane) & 1);
      int bd;
      if (NARROW)
        bd = (int)(wave_min_u32(ok ? ((uint32_t)dl << 6) | (uint32_t)lane : ~0u, D) & 63);
      else
        bd = (int)(wave_reduce_u64<false>(ok ? (dl << 6) | (uint64_t)lane : ~0ull) & 63);
      if (lane == bd) dl += sl;
      if (lane == 0) {
        s_used[se] = used | (1ull << bd);
        s_bd[p0 + j] = (uint8_t)bd;
      }
    }
  }
  if (lane < D) device_load[lane] = (int64_t)dl;
}

__global__ __launch_bounds__(1024) void eplb_plan_kernel(
    const int32_t* __restrict__ counts, int E, int D, int extra, int32_t* __restrict__ replicas,
    int32_t* __restrict__ slot_device, int32_t* __restrict__ slot_load,
    int64_t* __restrict__ device_load) {
  __shared__ uint64_t s_wbest[2][16];
  __shared__ int32_t s_off[kEplbMaxE + 1];
  __shared__ int32_t s_scan[16];
  __shared__ int64_t s_lsum[16];
  // slot keys in LPT order: (2^31 - 1 - load) << 16 | expert << 6 | replica,
  // so a smaller key comes first (heavier, then lower expert, then lower replica)
  __shared__ uint64_t s_key[kEplbMaxSlots];
  __shared__ uint64_t s_sorted[kEplbMaxSlots];
  __shared__ uint64_t s_used[kEplbMaxE];  // devices holding a copy, per expert
  __shared__ uint8_t s_bd[kEplbMaxSlots];  // device of the slot of LPT rank p
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int e = tid;
  const int64_t load = e < E ? (int64_t)counts[e] : 0;
  int32_t r = 1;

  // 1. replication: one block arg-max per extra replica (the wave results go
  //    to a double-buffered table that every thread reduces itself); only
  //    the winner's key changes between rounds
  const int nw = (E + 63) >> 6;  // waves holding experts
  uint64_t key = (e < E && r < D) ? rep_key(load, r, e) : 0;
  for (int it = 0; it < extra; ++it) {
    if (wave < nw) {
      const uint64_t c = wave_reduce_u64<true>(key);
      if (lane == 0) s_wbest[it & 1][wave] = c;
    }
    __syncthreads();
    uint64_t b = s_wbest[it & 1][0];
    for (int w = 1; w < nw; ++w) b = s_wbest[it & 1][w] > b ? s_wbest[it & 1][w] : b;
    if (b == 0) break;  // every expert is on every device: uniform exit
    if (1023 - (int)(b & 1023) == e) {
      ++r;
      key = r < D ? rep_key(load, r, e) : 0;
    }
  }

  // 2. slots: exclusive scan of the replica counts, then each expert's slots
  const int32_t rv = e < E ? r : 0;
  int32_t incl = rv;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  int64_t lsum = load;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)
    lsum += ((int64_t)__shfl_xor((int)(lsum >> 32), o, 64) << 32) |
            (uint32_t)__shfl_xor((int)(uint32_t)lsum, o, 64);
  if (lane == 63) s_scan[wave] = incl;
  if (lane == 0) s_lsum[wave] = lsum;
  __syncthreads();
  int32_t wpre = 0;
  for (int w = 0; w < wave; ++w) wpre += s_scan[w];
  int32_t S = 0;
  for (int w = 0; w < 16; ++w) S += s_scan[w];
  const int32_t off = wpre + incl - rv;
  if (e < E) {
    s_off[e] = off;
    s_used[e] = 0;
    replicas[e] = r;
    for (int i = 0; i < r; ++i) {
      const int64_t li = load / r + (i < load % r ? 1 : 0);
      s_key[off + i] = ((uint64_t)(0x7FFFFFFF - li) << 16) | ((uint64_t)e << 6) | (uint64_t)i;
      slot_load[off + i] = (int32_t)li;
    }
  }
  __syncthreads();

  // 3. rank of every slot in LPT order (the keys are distinct)
  for (int s = tid; s < S; s += 1024) {
    const uint64_t ks = s_key[s];
    int32_t rank = 0;
#pragma unroll 8
    for (int u = 0; u < S; ++u) rank += s_key[u] < ks;
    s_sorted[rank] = ks;
  }
  __syncthreads();

  // 4. LPT walk by wave 0 (device loads below 2^26, every practical batch,
  //    take 32-bit keys)
  int64_t total = 0;
  for (int w = 0; w < 16; ++w) total += s_lsum[w];
  if (wave == 0) {
    if (total < (1ll << 26)) lpt_walk<true>(s_sorted, S, D, lane, s_used, s_bd, device_load);
    else lpt_walk<false>(s_sorted, S, D, lane, s_used, s_bd, device_load);
  }
  __syncthreads();
  for (int p = tid; p < S; p += 1024) {
    const uint64_t k = s_sorted[p];
    slot_device[s_off[(int)((k >> 6) & 1023)] + (int)(k & 63)] = s_bd[p];
  }
  for (int s = S + tid; s < E + extra; s += 1024) {
    slot_load[s] = 0;
    slot_device[s] = -1;
  }
}

}  // namespace

hipError_t launch_eplb_plan(const int32_t* counts, int E, int D, int extra, int32_t* replicas,
                            int32_t* slot_device, int32_t* slot_load, int64_t* device_load,
                            hipStream_t st) {
  eplb_plan_kernel<<<1, 1024, 0, st>>>(counts, E, D, extra, replicas, slot_device, slot_load,
                                       device_load);
  return hipGetLastError();
}

}  // namespace moe
