// Hot-set placement of the resident expert slots.  The recipes wiki (Home page, the expert
// balance) keeps the experts that the traffic routes to most resident on the GPU, chosen from
// routing histograms by a greedy pick of the largest routing share per byte of weights.  Every
// expert here has the same storage size, so the share per byte orders as the accumulated count.
//   accumulate: hist[e] += counts[e] (int64, one thread per expert)
//   plan:       rank[e] = number of experts ahead of e in (count descending, id ascending);
//               slot_map[e] = rank[e] if rank[e] < S, else -1
// One work-group ranks all E <= 1024 experts: each thread counts the experts ahead of its own by
// reading the whole histogram from LDS (every thread reads the same word: a broadcast).
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
