// Weighted combine back to token order: out[t] = sum_j w[t,j] * y[row (t,j)] over the computed
// rows, j ascending, fp32, rounded once to the output format.  A row's output comes from tier a
// (y_a[inv_a[t*k+j]]) when it has a position there, else from tier b (y_b[inv_b[t*k+j]]) when one
// is given and the row has a position in it, else the row adds nothing.  With tier b a second
// weight pool holding the experts tier a lacks, the result is the one-pool layer on the union
// of the pools, summed in the same order.  Each thread owns four consecutive hidden columns of
// one token (16-byte loads of the fp32 rows), so the sum order is fixed and the result
// deterministic.  The rows are read once and the output written once, both with non-temporal
// accesses; a work-group covers a whole 4096-wide token row (1024 threads) where H allows and
// the batch has at least 64 tokens (measured at T = 4096, k = 8, H = 4096: 101 us instead of
// 116 us with 256 threads and cached accesses).  Smaller batches are latency-bound: there each
// 64-thread work-group covers 256 columns of a row (T = 4: the layer step 1.6 us shorter than
// with one 1024-thread work-group per row).
#include "common.h"
#include "kernels.h"

namespace moe {

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#ifndef MOE_COMBINE_WIDE_MIN_T
#define MOE_COMBINE_WIDE_MIN_T 64     // tokens from which a work-group covers a whole row
#endif
#ifndef MOE_COMBINE_SMALL_THREADS
#define MOE_COMBINE_SMALL_THREADS 64  // threads per work-group below that
#endif

template <int ODT, int THREADS>
__global__ __launch_bounds__(THREADS) void combine_kernel(const float* __restrict__ y,
                                                               const int32_t* __restrict__ inv,
                                                               const float* __restrict__ y_b,
                                                               const int32_t* __restrict__ inv_b,
                                                               const float* __restrict__ w, int T,
                                                               int k, int H, int cap,
                                                               void* __restrict__ out) {
  const int t = blockIdx.x;
  const int h = (blockIdx.y * THREADS + threadIdx.x) * 4;
  // lanes past H stay active: the positions and gates are read across the wave (readlane), so every
  // lane loads its own; only their row loads and stores are skipped
  const bool live = h < H;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // the token's positions and gates, one per lane (k <= 64), in one load each; then groups of kJ
  // choices: every row load of a group in flight together, the sums in ascending j
  const int lane = threadIdx.x & 63;
  const int pv = lane < k ? inv[size_t(t) * k + lane] : -1;
  const int qv = (inv_b && lane < k) ? inv_b[size_t(t) * k + lane] : -1;
  const float gv = lane < k ? w[size_t(t) * k + lane] : 0.0f;
  constexpr int kJ = 8;
  for (int j0 = 0; j0 < k; j0 += kJ) {
    const float* src[kJ];  // the row's output in tier a or b, or none
    float g[kJ];
#pragma unroll
    for (int u = 0; u < kJ; ++u) {
      const int p = __builtin_amdgcn_readlane(pv, j0 + u);
      const int q = __builtin_amdgcn_readlane(qv, j0 + u);
      g[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), j0 + u));
      src[u] = nullptr;
      if (live && j0 + u < k) {
        if (p >= 0 && p < cap) src[u] = y + size_t(p) * H + h;
        else if (q >= 0 && q < cap) src[u] = y_b + size_t(q) * H + h;
      }
    }
    float4 v[kJ];
#pragma unroll
    for (int u = 0; u < kJ; ++u) {
      v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (src[u]) {
        const uint4 q = ld_stream16(src[u]);
        v[u] = make_float4(__uint_as_float(q.x), __uint_as_float(q.y), __uint_as_float(q.z), __uint_as_float(q.w));
      }
    }
#pragma unroll
    for (int u = 0; u < kJ; ++u) {
      if (src[u]) {
        acc.x = fmaf(g[u], v[u].x, acc.x);
        acc.y = fmaf(g[u], v[u].y, acc.y);
        acc.z = fmaf(g[u], v[u].z, acc.z);
        acc.w = fmaf(g[u], v[u].w, acc.w);
      }
    }
  }
  if (!live) return;
  if constexpr (ODT == DT_F32) {
    const u32x4_t o = {__float_as_uint(acc.x), __float_as_uint(acc.y), __float_as_uint(acc.z), __float_as_uint(acc.w)};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(static_cast<float*>(out) + size_t(t) * H + h));
  } else {
    const u32x2_t o = {uint32_t(f32_to_bf16(acc.x)) | (uint32_t(f32_to_bf16(acc.y)) << 16),
                       uint32_t(f32_to_bf16(acc.z)) | (uint32_t(f32_to_bf16(acc.w)) << 16)};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(out) + size_t(t) * H + h));
  }
}

hipError_t launch_combine(const float* y, const int32_t* inv, const float* y_b, const int32_t* inv_b,
                          const float* w, int T, int k, int H, void* out, int odt, hipStream_t st) {
  const int cap = T * k;
#define MOE_COMBINE_LAUNCH(N)                                                                  \
  {                                                                                            \
    dim3 grid(T, (H / 4 + (N) - 1) / (N)), block(N);                                           \
    if (odt == DT_F32)                                                                         \
      combine_kernel<DT_F32, N><<<grid, block, 0, st>>>(y, inv, y_b, inv_b, w, T, k, H, cap, out); \
    else                                                                                       \
      combine_kernel<DT_BF16, N><<<grid, block, 0, st>>>(y, inv, y_b, inv_b, w, T, k, H, cap, out); \
  }
  if (H >= 4096 && T >= MOE_COMBINE_WIDE_MIN_T) MOE_COMBINE_LAUNCH(1024)
  else if (T < MOE_COMBINE_WIDE_MIN_T) MOE_COMBINE_LAUNCH(MOE_COMBINE_SMALL_THREADS)
  else MOE_COMBINE_LAUNCH(256)
#undef MOE_COMBINE_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
