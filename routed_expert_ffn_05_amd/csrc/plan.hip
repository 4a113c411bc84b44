// Hot-set placement of the resident expert slots.  The recipes wiki (Home page, the expert
// balance) keeps the experts that the traffic routes to most resident on the GPU, chosen from
// routing histograms by a greedy pick of the largest routing share per byte of weights.  Every
// expert here has the same storage size, so the share per byte orders as the accumulated count.
//   accumulate: hist[e] += counts[e] (int64, one thread per expert)
//   plan:       rank[e] = number of experts ahead of e in (count descending, id ascending);
//               slot_map[e] = rank[e] if rank[e] < S, else -1
// One work-group ranks all E <= 1024 experts: each thread counts the experts ahead of its own by
// reading the whole histogram from LDS (every thread reads the same word: a broadcast).
#include <algorithm>
#include <climits>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(256) void accumulate_counts_kernel(const int32_t* __restrict__ counts, int E,
                                                                int64_t* __restrict__ hist) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e < E) hist[e] += counts[e];
}

__global__ __launch_bounds__(kPlanThreads) void plan_slots_kernel(const int64_t* __restrict__ hist, int E, int S,
                                                                  int32_t* __restrict__ slot_map) {
  __shared__ int64_t h[kPlanThreads];
  const int e = threadIdx.x;
  if (e < E) h[e] = hist[e];
  __syncthreads();
  if (e >= E) return;
  const int64_t mine = h[e];
  int ahead = 0;
  for (int f = 0; f < E; ++f) {
    const int64_t o = h[f];
    ahead += (o > mine) || (o == mine && f < e);
  }
  slot_map[e] = ahead < S ? ahead : -1;
}

hipError_t launch_accumulate_counts(const int32_t* counts, int E, int64_t* hist, hipStream_t st) {
  accumulate_counts_kernel<<<(E + 255) / 256, 256, 0, st>>>(counts, E, hist);
  return hipGetLastError();
}

hipError_t launch_plan_slots(const int64_t* hist, int E, int S, int32_t* slot_map, hipStream_t st) {
  plan_slots_kernel<<<1, kPlanThreads, 0, st>>>(hist, E, S, slot_map);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

// ---------------------------------------------------------------------------------------------
// LRU slot refill (the pages' "full LRU": every resident slot is a spare that the most recently
// used experts occupy -- vLLM-Moet README, the MoET hybrid measurement matrix, 4x 5090 row).  After
// a call, each expert that missed moves into a slot for the next call:
//   1. every slot whose expert took rows in this call gets last_use = step;
//   2. the missed experts (rows > 0, no slot) are ranked by (rows descending, id ascending), the
//      slots not used in this call by (last_use ascending, slot ascending; empty slots hold
//      last_use -1); the i-th missed expert takes the i-th such slot, for i < min of the counts;
//   3. the maps and last_use are updated, and the pairs (slot, expert) listed for the copy.
// One work-group; E, S <= 1024.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kPlanThreads) void refill_plan_kernel(const int32_t* __restrict__ counts, int E, int S,
                                                                   long long step, int32_t* __restrict__ slot_map,
                                                                   int32_t* __restrict__ slot_expert,
                                                                   int64_t* __restrict__ last_use,
                                                                   int2* __restrict__ plan, int32_t* __restrict__ nplan) {
  __shared__ int32_t cnt[kPlanThreads];    // rows per expert, -1 unless the expert missed
  __shared__ int64_t lu[kPlanThreads];     // last use per slot, INT64_MAX if used in this call
  __shared__ int32_t victim[kPlanThreads]; // slot of victim rank r
  __shared__ int32_t nmiss, nvict;
  const int t = threadIdx.x;
  if (t == 0) nmiss = nvict = 0;
  int32_t my_cnt = -1;
  if (t < E) {
    const int c = counts[t];
    my_cnt = (c > 0 && slot_map[t] < 0) ? c : -1;
    cnt[t] = my_cnt;
  }
  int64_t my_lu = INT64_MAX;
  if (t < S) {
    const int e = slot_expert[t];
    const bool used = e >= 0 && e < E && counts[e] > 0;
    my_lu = used ? INT64_MAX : last_use[t];
    if (used) last_use[t] = step;
    lu[t] = my_lu;
  }
  __syncthreads();
  // ranks: missed experts by (rows desc, id asc); free slots by (last_use asc, slot asc)
  int mrank = 0, vrank = 0;
  if (my_cnt > 0) {
    for (int f = 0; f < E; ++f) {
      const int o = cnt[f];
      mrank += (o > my_cnt) || (o == my_cnt && f < t);
    }
    atomicAdd(&nmiss, 1);
  }
  if (t < S && my_lu != INT64_MAX) {
    for (int q = 0; q < S; ++q) {
      const int64_t o = lu[q];
      vrank += (o < my_lu) || (o == my_lu && q < t);
    }
    victim[vrank] = t;
    atomicAdd(&nvict, 1);
  }
  __syncthreads();
  const int n = min(nmiss, nvict);
  int old = -1, slot = -1;
  if (my_cnt > 0 && mrank < n) {
    slot = victim[mrank];
    old = slot_expert[slot];
  }
  __syncthreads();  // every old expert read before any slot_expert write
  if (slot >= 0) {
    if (old >= 0 && old < E) slot_map[old] = -1;
    slot_map[t] = slot;
    slot_expert[slot] = t;
    last_use[slot] = step;
    plan[mrank] = make_int2(slot, t);
  }
  if (t == 0) nplan[0] = n;
}

// Copy the listed experts' weights from the backing store (slot = expert id) into their slots:
// four segments per expert (w_gu, s_gu, w_d, s_d), 16-byte copies where addresses and size allow.
struct RefillSeg {
  const uint8_t* src;
  uint8_t* dst;
  size_t bytes;  // per expert
};

__global__ __launch_bounds__(256) void refill_copy_kernel(const int2* __restrict__ plan,
                                                          const int32_t* __restrict__ nplan, RefillSeg s0,
                                                          RefillSeg s1, RefillSeg s2, RefillSeg s3) {
  const int pair = blockIdx.y;
  if (pair >= nplan[0]) return;
  const int2 pe = plan[pair];
  const RefillSeg segs[4] = {s0, s1, s2, s3};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const RefillSeg g = segs[q];
    if (!g.bytes) continue;
    const uint8_t* src = g.src + size_t(pe.y) * g.bytes;
    uint8_t* dst = g.dst + size_t(pe.x) * g.bytes;
    const bool vec = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) | g.bytes) & 15) == 0;
    const size_t n16 = vec ? g.bytes / 16 : 0;
    for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += size_t(gridDim.x) * 256)
      reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
    if (n16 == 0)
      for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < g.bytes; i += size_t(gridDim.x) * 256) dst[i] = src[i];
  }
}

hipError_t launch_refill(const int32_t* counts, int E, int S, long long step, int32_t* slot_map,
                         int32_t* slot_expert, int64_t* last_use, int2* plan, int32_t* nplan,
                         const uint8_t* const src[4], uint8_t* const dst[4], const size_t bytes[4], hipStream_t st) {
  refill_plan_kernel<<<1, kPlanThreads, 0, st>>>(counts, E, S, step, slot_map, slot_expert, last_use, plan, nplan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  RefillSeg g[4];
  size_t most = 0;
  for (int q = 0; q < 4; ++q) {
    g[q] = RefillSeg{src[q], dst[q], src[q] && dst[q] ? bytes[q] : 0};
    most = g[q].bytes > most ? g[q].bytes : most;
  }
  const unsigned bx = unsigned(std::min<size_t>((most / 16 + 255) / 256, 64));
  refill_copy_kernel<<<dim3(bx > 0 ? bx : 1, S), 256, 0, st>>>(plan, nplan, g[0], g[1], g[2], g[3]);
  return hipGetLastError();
}

}  // namespace moe
