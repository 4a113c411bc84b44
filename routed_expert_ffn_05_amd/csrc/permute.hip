// Permutation: expert histogram, per-slot exclusive scan and a stable scatter of the rows into
// slot order, plus the compact miss list.  Deterministic: no global atomics, the position of
// every row is a pure function of the routing.
//
// One work-group of 16 waves.  Wave w owns the contiguous row range [w*L, (w+1)*L).  Keys are
// slots 0..S-1 plus one extra key S for non-resident rows.
//   1. per-wave key counters in LDS (LDS atomics: counting is order-free)
//   2. exclusive scan over keys gives slot_offsets; a running sum over waves gives each wave's
//      base position for every key
//   3. each wave walks its rows in chunks of 64 in order; rows of one chunk that share a key are
//      ranked by lane order (ballot of equal keys, popcount below the lane)
//
// For small batches the top-k of every token runs in the same work-group first (one wave per
// token), its results kept in LDS, so routing and permutation cost one launch.
//
// Batches of at most kSmallPermRows rows skip the counters: every row's composite key
// (key << 16 | r) goes into an LDS table, and after one barrier each output is a count over that
// table, read by LDS broadcast: a row's position is the number of rows with a smaller composite
// key, a slot's offset the number of resident rows in smaller slots, an expert's count the number
// of rows that chose it.
//
// Large batches (more than kPermOneGroupRows rows) spread the same three steps over work-groups
// of 1024 rows each: (1) every group counts its rows per key and per expert into a global table,
// (2) one group sums the table, scans the slot totals and turns each group's counts into its base
// position per key (groups in row order), (3) every group ranks its rows as in the one-group
// version, starting from those bases.  The result is identical to the one-group version.
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;
constexpr int kPermOneGroupRows = 2048;  // larger batches use the multi-group kernels
constexpr int kSmallPermRows = 128;      // batches up to this size rank rows by direct counts

// LDS words used by permute_body
__host__ __device__ inline size_t permute_lds_words(int E, int S) {
  return size_t(kPermWaves) * (S + 1) + E + (S + 2);
}

// LDS words used by permute_small_body
__host__ __device__ inline size_t permute_small_lds_words(int R) { return size_t(2) * ((R + 3) & ~3); }

// key of a row: slot, S for a miss, -1 for an invalid row (expert or slot out of range)
__device__ __forceinline__ int row_key(const int32_t* topk_idx, int E, const int32_t* __restrict__ slot_map,
                                       int S, int r, int& e) {
  e = topk_idx[r];
  if (e < 0 || e >= E) return -1;
  const int s = slot_map ? slot_map[e] : e;
  if (s < -1 || s >= S) return -1;
  return s < 0 ? S : s;
}

// Stable scatter of one wave's 64 rows given its per-key running bases wbase[key] (advanced past
// the rows): rows sharing a key are ranked by lane order.  Lane l places row r = (the wave's first
// row) + l, whose key and expert it holds (key -1 for rows past r1 or invalid rows).
__device__ __forceinline__ void scatter_rows(int key, int e, int r, int r1, const float* topk_w, int k, int S,
                                             int32_t* wbase, int32_t* __restrict__ perm,
                                             int32_t* __restrict__ inv_perm, int32_t* __restrict__ miss_token,
                                             int32_t* __restrict__ miss_expert, float* __restrict__ miss_weight) {
  const int lane = threadIdx.x & 63;
  unsigned long long todo = __ballot(key >= 0);
  int pos = -1;
  while (todo) {
    const int leader = __ffsll((long long)todo) - 1;
    const int lkey = __shfl(key, leader);
    const unsigned long long m = __ballot(key == lkey);
    const int b = wbase[lkey];
    if (key == lkey) pos = b + __popcll(m & ((1ull << lane) - 1ull));
    if (lane == leader) wbase[lkey] = b + __popcll(m);
    todo &= ~m;
  }
  if (r < r1) {
    if (key < 0) {
      inv_perm[r] = -1;
    } else if (key < S) {
      perm[pos] = r;
      inv_perm[r] = pos;
    } else {
      inv_perm[r] = -1;
      miss_token[pos] = r / k;
      miss_expert[pos] = e;
      miss_weight[pos] = topk_w[r];
    }
  }
}

// the same for rows [c0, c0+64), their keys read here
__device__ __forceinline__ void scatter_chunk(const int32_t* topk_idx, const float* topk_w, int k, int E,
                                              const int32_t* __restrict__ slot_map, int S, int c0, int r1,
                                              int32_t* wbase, int32_t* __restrict__ perm,
                                              int32_t* __restrict__ inv_perm, int32_t* __restrict__ miss_token,
                                              int32_t* __restrict__ miss_expert, float* __restrict__ miss_weight) {
  const int r = c0 + (threadIdx.x & 63);
  int e = 0, key = -1;
  if (r < r1) key = row_key(topk_idx, E, slot_map, S, r, e);
  scatter_rows(key, e, r, r1, topk_w, k, S, wbase, perm, inv_perm, miss_token, miss_expert, miss_weight);
}

__device__ void permute_body(const int32_t* topk_idx, const float* topk_w, int T, int k, int E,
                             const int32_t* __restrict__ slot_map, int S, int32_t* __restrict__ counts,
                             int32_t* __restrict__ slot_offsets, int32_t* __restrict__ perm,
                             int32_t* __restrict__ inv_perm, int32_t* __restrict__ miss_count,
                             int32_t* __restrict__ miss_token, int32_t* __restrict__ miss_expert,
                             float* __restrict__ miss_weight, uint32_t* __restrict__ err, int32_t* lds) {
  const int K1 = S + 1;                     // keys: slots + the miss key
  int32_t* cnt = lds;                       // [kPermWaves][K1] per-wave counts, then bases
  int32_t* ecnt = cnt + kPermWaves * K1;    // [E]
  int32_t* tot = ecnt + E;                  // [K1 + 1] key totals -> exclusive offsets
  __shared__ int32_t wsum[kPermWaves];
  __shared__ uint32_t bad;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int R = T * k;
  const int L = (R + kPermWaves - 1) / kPermWaves;
  const int r0 = wid * L, r1 = min(R, r0 + L);

  for (int i = tid; i < kPermWaves * K1; i += kPermThreads) cnt[i] = 0;
  for (int i = tid; i < E; i += kPermThreads) ecnt[i] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();

  auto key_of = [&](int r, int& e) -> int { return row_key(topk_idx, E, slot_map, S, r, e); };

  // 1. counts
  for (int r = r0 + lane; r < r1; r += 64) {
    int e;
    const int key = key_of(r, e);
    if (key < 0) {
      bad = 1;
      continue;
    }
    atomicAdd(&cnt[wid * K1 + key], 1);
    atomicAdd(&ecnt[e], 1);
  }
  __syncthreads();

  // 2a. key totals
  for (int key = tid; key < K1; key += kPermThreads) {
    int s = 0;
    for (int w = 0; w < kPermWaves; ++w) s += cnt[w * K1 + key];
    tot[key] = s;
  }
  __syncthreads();
  // 2b. exclusive scan of the S slot totals (the miss key scans separately from 0):
  //     thread-sequential chunks, then a scan of the chunk sums.
  {
    const int per = (S + kPermThreads - 1) / kPermThreads;
    const int a = tid * per, b = min(S, a + per);
    int local = 0;
    for (int i = a; i < b; ++i) local += tot[i];
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wid; ++w) wbase += wsum[w];
    int run = wbase + incl - local;
    __syncthreads();
    for (int i = a; i < b; ++i) {
      const int c = tot[i];
      tot[i] = run;
      run += c;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int n_res = 0;
    for (int w = 0; w < kPermWaves; ++w) n_res += wsum[w];
    tot[S + 1] = n_res;
  }
  __syncthreads();
  // 2c. per-wave bases: base[w][key] = offset[key] + sum_{w' < w} cnt[w'][key]
  for (int key = tid; key < K1; key += kPermThreads) {
    int run = (key == S) ? 0 : tot[key];
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = cnt[w * K1 + key];
      cnt[w * K1 + key] = run;
      run += c;
    }
  }
  __syncthreads();

  // 3. stable scatter
  for (int c0 = r0; c0 < r1; c0 += 64)
    scatter_chunk(topk_idx, topk_w, k, E, slot_map, S, c0, r1, cnt + wid * K1, perm, inv_perm, miss_token,
                  miss_expert, miss_weight);

  // outputs of the scan and histogram
  for (int i = tid; i < E; i += kPermThreads) counts[i] = ecnt[i];
  for (int i = tid; i < S; i += kPermThreads) slot_offsets[i] = tot[i];
  if (tid == 0) {
    slot_offsets[S] = tot[S + 1];
    if (miss_count) miss_count[0] = tot[S];
    err[0] = bad ? 1u : 0u;
  }
}

// The permutation of at most kSmallPermRows rows (see the file comment).  Thread roles: row tid
// (tid < R), slot s = tid (and s = tid + 1024 for S = 1024), expert e = tid ^ 512 (E <= 1024), so
// the row, slot and expert counts run in different waves.
__device__ void permute_small_body(const int32_t* topk_idx, const float* topk_w, int T, int k, int E,
                                   const int32_t* __restrict__ slot_map, int S, int32_t* __restrict__ counts,
                                   int32_t* __restrict__ slot_offsets, int32_t* __restrict__ perm,
                                   int32_t* __restrict__ inv_perm, int32_t* __restrict__ miss_count,
                                   int32_t* __restrict__ miss_token, int32_t* __restrict__ miss_expert,
                                   float* __restrict__ miss_weight, uint32_t* __restrict__ err, int32_t* lds) {
  const int R = T * k, R4 = (R + 3) & ~3, n4 = R4 / 4;
  uint32_t* ck = reinterpret_cast<uint32_t*>(lds);  // [R4] composite keys; ~0: invalid row or padding
  int32_t* se = lds + R4;                           // [R4] expert of the row; -1: invalid or padding
  const int tid = threadIdx.x;
  if (tid < R4) {
    uint32_t c = ~0u;
    int e = -1;
    if (tid < R) {
      int ee;
      const int key = row_key(topk_idx, E, slot_map, S, tid, ee);
      if (key >= 0) {
        c = (uint32_t(key) << 16) | uint32_t(tid);
        e = ee;
      }
    }
    ck[tid] = c;
    se[tid] = e;
  }
  __syncthreads();
  const uint4* ck4 = reinterpret_cast<const uint4*>(ck);
  const int4* se4 = reinterpret_cast<const int4*>(se);
  const uint32_t res_end = uint32_t(S) << 16;  // composite keys below this are resident rows
  if (tid < R) {
    const uint32_t c = ck[tid];
    int pos = 0, n_res = 0;
    for (int q = 0; q < n4; ++q) {
      const uint4 v = ck4[q];
      pos += int(v.x < c) + int(v.y < c) + int(v.z < c) + int(v.w < c);
      n_res += int(v.x < res_end) + int(v.y < res_end) + int(v.z < res_end) + int(v.w < res_end);
    }
    if (c == ~0u) {
      inv_perm[tid] = -1;
    } else if (c < res_end) {
      perm[pos] = tid;
      inv_perm[tid] = pos;
    } else {
      const int m = pos - n_res;  // misses follow every resident row in (key, r) order
      inv_perm[tid] = -1;
      miss_token[m] = tid / k;
      miss_expert[m] = se[tid];
      miss_weight[m] = topk_w[tid];
    }
  }
  for (int sl = tid; sl <= S; sl += kPermThreads) {
    const uint32_t lo = uint32_t(sl) << 16;
    int off = 0, below_next = 0, bad = 0;
    for (int q = 0; q < n4; ++q) {
      const uint4 v = ck4[q];
      off += int(v.x < lo) + int(v.y < lo) + int(v.z < lo) + int(v.w < lo);
      if (sl == S) {
        const uint32_t hi = lo + 0x10000u;
        below_next += int(v.x < hi) + int(v.y < hi) + int(v.z < hi) + int(v.w < hi);
        bad += int(v.x == ~0u) + int(v.y == ~0u) + int(v.z == ~0u) + int(v.w == ~0u);
      }
    }
    slot_offsets[sl] = off;
    if (sl == S) {
      if (miss_count) miss_count[0] = below_next - off;
      err[0] = bad > R4 - R ? 1u : 0u;
    }
  }
  const int e = tid ^ (kPermThreads / 2);
  if (e < E) {
    int n = 0;
    for (int q = 0; q < n4; ++q) {
      const int4 v = se4[q];
      n += int(v.x == e) + int(v.y == e) + int(v.z == e) + int(v.w == e);
    }
    counts[e] = n;
  }
}

__global__ __launch_bounds__(kPermThreads) void permute_small_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w, int T, int k, int E,
    const int32_t* __restrict__ slot_map, int S, int32_t* __restrict__ counts,
    int32_t* __restrict__ slot_offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    int32_t* __restrict__ miss_count, int32_t* __restrict__ miss_token,
    int32_t* __restrict__ miss_expert, float* __restrict__ miss_weight, uint32_t* __restrict__ err) {
  extern __shared__ __align__(16) int32_t lds[];
  permute_small_body(topk_idx, topk_w, T, k, E, slot_map, S, counts, slot_offsets, perm, inv_perm,
                     miss_count, miss_token, miss_expert, miss_weight, err, lds);
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w, int T, int k, int E,
    const int32_t* __restrict__ slot_map, int S, int32_t* __restrict__ counts,
    int32_t* __restrict__ slot_offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    int32_t* __restrict__ miss_count, int32_t* __restrict__ miss_token,
    int32_t* __restrict__ miss_expert, float* __restrict__ miss_weight, uint32_t* __restrict__ err) {
  extern __shared__ __align__(16) int32_t lds[];
  permute_body(topk_idx, topk_w, T, k, E, slot_map, S, counts, slot_offsets, perm, inv_perm,
               miss_count, miss_token, miss_expert, miss_weight, err, lds);
}

// top-k of every token (one wave each), then the permutation, in one work-group
template <int VPL>
__global__ __launch_bounds__(kPermThreads) void route_permute_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int k, int E, int score,
    int renorm, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    const int32_t* __restrict__ slot_map, int S, int32_t* __restrict__ counts,
    int32_t* __restrict__ slot_offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    int32_t* __restrict__ miss_count, int32_t* __restrict__ miss_token,
    int32_t* __restrict__ miss_expert, float* __restrict__ miss_weight, uint32_t* __restrict__ err) {
  extern __shared__ __align__(16) int32_t lds[];
  const int R = T * k;
  int32_t* sidx = lds;                                   // [R]
  float* sw = reinterpret_cast<float*>(lds + R);         // [R]
  int32_t* scratch = lds + ((2 * R + 3) & ~3);  // 16-byte aligned: the small path reads it 4 words at a time
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  for (int t = wid; t < T; t += kPermWaves) {
    int my_e;
    float my_w;
    topk_wave<VPL>(logits + size_t(t) * E, bias, E, k, score, renorm, my_e, my_w);
    if (lane < k) {
      sidx[t * k + lane] = my_e;
      sw[t * k + lane] = my_w;
      topk_idx[size_t(t) * k + lane] = my_e;
      topk_w[size_t(t) * k + lane] = my_w;
    }
  }
  __syncthreads();
  if (R <= kSmallPermRows)
    permute_small_body(sidx, sw, T, k, E, slot_map, S, counts, slot_offsets, perm, inv_perm, miss_count,
                       miss_token, miss_expert, miss_weight, err, scratch);
  else
    permute_body(sidx, sw, T, k, E, slot_map, S, counts, slot_offsets, perm, inv_perm, miss_count,
                 miss_token, miss_expert, miss_weight, err, scratch);
}

static hipError_t set_lds(const void* kern, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
}

// ---- multi-group permutation -----------------------------------------------------------------
// table row of group g: [K1 key counts (bases after the scan)][E expert counts][invalid flag]
__host__ __device__ inline int perm_table_stride(int E, int S) { return S + 1 + E + 1; }

// (1) per-group counts
__global__ __launch_bounds__(kPermThreads) void perm_count_kernel(const int32_t* __restrict__ topk_idx, int R,
                                                                  int E, const int32_t* __restrict__ slot_map,
                                                                  int S, int32_t* __restrict__ table) {
  extern __shared__ __align__(16) int32_t lds[];
  const int K1 = S + 1, stride = perm_table_stride(E, S);
  int32_t* cnt = lds;        // [K1]
  int32_t* ecnt = lds + K1;  // [E]
  __shared__ uint32_t bad;
  const int tid = threadIdx.x;
  for (int i = tid; i < K1 + E; i += kPermThreads) lds[i] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  const int r = blockIdx.x * kPermThreads + tid;
  if (r < R) {
    int e;
    const int key = row_key(topk_idx, E, slot_map, S, r, e);
    if (key < 0) {
      bad = 1;
    } else {
      atomicAdd(&cnt[key], 1);
      atomicAdd(&ecnt[e], 1);
    }
  }
  __syncthreads();
  int32_t* row = table + size_t(blockIdx.x) * stride;
  for (int i = tid; i < K1 + E; i += kPermThreads) row[i] = lds[i];
  if (tid == 0) row[K1 + E] = bad ? 1 : 0;
}

// (2) totals, slot offsets, per-group bases (one work-group)
__global__ __launch_bounds__(kPermThreads) void perm_scan_kernel(int32_t* __restrict__ table, int ngroups, int E,
                                                                 int S, int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ slot_offsets,
                                                                 int32_t* __restrict__ miss_count,
                                                                 uint32_t* __restrict__ err) {
  extern __shared__ int32_t tot[];  // [K1 + 1]
  __shared__ int32_t wsum[kPermWaves];
  __shared__ uint32_t bad;
  const int K1 = S + 1, stride = perm_table_stride(E, S);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int key = tid; key < K1 + E + 1; key += kPermThreads) {
    int s = 0;
#pragma unroll 8
    for (int g = 0; g < ngroups; ++g) s += table[size_t(g) * stride + key];
    if (key < K1) tot[key] = s;
    else if (key < K1 + E) counts[key - K1] = s;
    else if (s) bad = 1;
  }
  __syncthreads();
  // exclusive scan of the S slot totals (the miss key scans separately from 0)
  {
    const int per = (S + kPermThreads - 1) / kPermThreads;
    const int a = tid * per, b = min(S, a + per);
    int local = 0;
    for (int i = a; i < b; ++i) local += tot[i];
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wid; ++w) wbase += wsum[w];
    int run = wbase + incl - local;
    __syncthreads();
    for (int i = a; i < b; ++i) {
      const int c = tot[i];
      tot[i] = run;
      run += c;
    }
  }
  __syncthreads();
  // group bases per key, groups in row order; eight groups' counts are read before any of their
  // bases is written (each key's column belongs to one thread), so a column takes ngroups / 8
  // round trips rather than one per group
  for (int key = tid; key < K1; key += kPermThreads) {
    int run = key == S ? 0 : tot[key];
    for (int g0 = 0; g0 < ngroups; g0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = g0 + u < ngroups ? table[size_t(g0 + u) * stride + key] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (g0 + u < ngroups) table[size_t(g0 + u) * stride + key] = run;
        run += v[u];
      }
    }
  }
  for (int i = tid; i < S; i += kPermThreads) slot_offsets[i] = tot[i];
  if (tid == 0) {
    int n_res = 0;
    for (int w = 0; w < kPermWaves; ++w) n_res += wsum[w];
    slot_offsets[S] = n_res;
    if (miss_count) miss_count[0] = tot[S];
    err[0] = bad ? 1u : 0u;
  }
}

// (3) per-group stable scatter from the group's bases
__global__ __launch_bounds__(kPermThreads) void perm_scatter_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w, int R, int k, int E,
    const int32_t* __restrict__ slot_map, int S, const int32_t* __restrict__ table, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv_perm, int32_t* __restrict__ miss_token, int32_t* __restrict__ miss_expert,
    float* __restrict__ miss_weight) {
  extern __shared__ int32_t cnt[];  // [kPermWaves][K1]
  const int K1 = S + 1, stride = perm_table_stride(E, S);
  const int tid = threadIdx.x, wid = tid >> 6;
  for (int i = tid; i < kPermWaves * K1; i += kPermThreads) cnt[i] = 0;
  __syncthreads();
  const int r0 = blockIdx.x * kPermThreads, r1 = min(R, r0 + kPermThreads);
  const int r = r0 + tid;
  int e = 0, key = -1;  // kept for the scatter: this thread's lane places row r there too
  if (r < r1) {
    key = row_key(topk_idx, E, slot_map, S, r, e);
    if (key >= 0) atomicAdd(&cnt[wid * K1 + key], 1);
  }
  __syncthreads();
  const int32_t* base = table + size_t(blockIdx.x) * stride;
  for (int key = tid; key < K1; key += kPermThreads) {
    int run = base[key];
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = cnt[w * K1 + key];
      cnt[w * K1 + key] = run;
      run += c;
    }
  }
  __syncthreads();
  if (r0 + wid * 64 < r1)
    scatter_rows(key, e, r, r1, topk_w, k, S, cnt + wid * K1, perm, inv_perm, miss_token, miss_expert, miss_weight);
}

size_t permute_scratch_bytes(int T, int k, int E, int S) {
  const long long R = (long long)T * k;
  if (R <= kPermOneGroupRows) return 0;
  const long long groups = (R + kPermThreads - 1) / kPermThreads;
  return size_t(groups) * perm_table_stride(E, S) * sizeof(int32_t);
}

size_t permute_lds_bytes(int E, int S) { return sizeof(int32_t) * permute_lds_words(E, S); }

size_t route_permute_lds_bytes(int T, int k, int E, int S) {
  const int R = T * k;
  return sizeof(int32_t) * (size_t((2 * R + 3) & ~3) + (R <= kSmallPermRows ? permute_small_lds_words(R) : permute_lds_words(E, S)));
}

hipError_t launch_permute(const int32_t* topk_idx, const float* topk_w, int T, int k, int E,
                          const int32_t* slot_map, int S, int32_t* counts, int32_t* slot_offsets,
                          int32_t* perm, int32_t* inv_perm, int32_t* miss_count,
                          int32_t* miss_token, int32_t* miss_expert, float* miss_weight,
                          uint32_t* err, int32_t* scratch, hipStream_t st) {
  const int R = T * k;
  if (R > kPermOneGroupRows) {
    const int groups = (R + kPermThreads - 1) / kPermThreads;
    const size_t l1 = sizeof(int32_t) * size_t(S + 1 + E);
    const size_t l2 = sizeof(int32_t) * size_t(S + 2);
    const size_t l3 = sizeof(int32_t) * size_t(kPermWaves) * (S + 1);
    hipError_t e = set_lds((const void*)perm_count_kernel, l1);
    if (e == hipSuccess) e = set_lds((const void*)perm_scan_kernel, l2);
    if (e == hipSuccess) e = set_lds((const void*)perm_scatter_kernel, l3);
    if (e != hipSuccess) return e;
    perm_count_kernel<<<groups, kPermThreads, l1, st>>>(topk_idx, R, E, slot_map, S, scratch);
    perm_scan_kernel<<<1, kPermThreads, l2, st>>>(scratch, groups, E, S, counts, slot_offsets, miss_count, err);
    perm_scatter_kernel<<<groups, kPermThreads, l3, st>>>(topk_idx, topk_w, R, k, E, slot_map, S, scratch, perm,
                                                          inv_perm, miss_token, miss_expert, miss_weight);
    return hipGetLastError();
  }
  if (R <= kSmallPermRows) {
    permute_small_kernel<<<1, kPermThreads, sizeof(int32_t) * permute_small_lds_words(R), st>>>(
        topk_idx, topk_w, T, k, E, slot_map, S, counts, slot_offsets, perm, inv_perm, miss_count, miss_token,
        miss_expert, miss_weight, err);
    return hipGetLastError();
  }
  const size_t lds = permute_lds_bytes(E, S);
  hipError_t e = set_lds((const void*)permute_kernel, lds);
  if (e != hipSuccess) return e;
  permute_kernel<<<1, kPermThreads, lds, st>>>(topk_idx, topk_w, T, k, E, slot_map, S, counts,
                                               slot_offsets, perm, inv_perm, miss_count,
                                               miss_token, miss_expert, miss_weight, err);
  return hipGetLastError();
}

template <int VPL>
static hipError_t launch_rp(const float* logits, const float* bias, int T, int k, int E, int score,
                            int renorm, int32_t* idx, float* w, const int32_t* slot_map, int S,
                            int32_t* counts, int32_t* off, int32_t* perm, int32_t* inv, int32_t* mc,
                            int32_t* mt, int32_t* me, float* mw, uint32_t* err, hipStream_t st) {
  const size_t lds = route_permute_lds_bytes(T, k, E, S);
  hipError_t e = set_lds((const void*)route_permute_kernel<VPL>, lds);
  if (e != hipSuccess) return e;
  route_permute_kernel<VPL><<<1, kPermThreads, lds, st>>>(logits, bias, T, k, E, score, renorm, idx, w,
                                                          slot_map, S, counts, off, perm, inv, mc, mt,
                                                          me, mw, err);
  return hipGetLastError();
}

hipError_t launch_route_permute(const float* logits, const float* bias, int T, int k, int E,
                                int score, int renorm, int32_t* idx, float* w,
                                const int32_t* slot_map, int S, int32_t* counts, int32_t* off,
                                int32_t* perm, int32_t* inv, int32_t* mc, int32_t* mt, int32_t* me,
                                float* mw, uint32_t* err, hipStream_t st) {
  const int vpl = (E + 63) / 64;
  if (vpl <= 2)
    return launch_rp<2>(logits, bias, T, k, E, score, renorm, idx, w, slot_map, S, counts, off, perm, inv, mc, mt, me, mw, err, st);
  if (vpl <= 4)
    return launch_rp<4>(logits, bias, T, k, E, score, renorm, idx, w, slot_map, S, counts, off, perm, inv, mc, mt, me, mw, err, st);
  if (vpl <= 6)
    return launch_rp<6>(logits, bias, T, k, E, score, renorm, idx, w, slot_map, S, counts, off, perm, inv, mc, mt, me, mw, err, st);
  if (vpl <= 8)
    return launch_rp<8>(logits, bias, T, k, E, score, renorm, idx, w, slot_map, S, counts, off, perm, inv, mc, mt, me, mw, err, st);
  return launch_rp<16>(logits, bias, T, k, E, score, renorm, idx, w, slot_map, S, counts, off, perm, inv, mc, mt, me, mw, err, st);
}

}  // namespace moe
