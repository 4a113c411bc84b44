// Weighted combine back to token order: out[t] = sum_j w[t,j] * y_perm[inv_perm[t*k+j]] over the
// resident rows, j ascending, fp32, rounded once to the output format.  Each thread owns four
// consecutive hidden columns of one token (16-byte loads of the fp32 rows), so the sum order is
// fixed and the result deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kCombThreads = 256;

template <int ODT>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(const float* __restrict__ y,
                                                               const int32_t* __restrict__ inv,
                                                               const float* __restrict__ w, int T,
                                                               int k, int H, int cap,
                                                               void* __restrict__ out) {
  const int t = blockIdx.x;
  const int h = (blockIdx.y * kCombThreads + threadIdx.x) * 4;
  // lanes past H stay active: the positions and gates are read across the wave (readlane), so every
  // lane loads its own; only their row loads and stores are skipped
  const bool live = h < H;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // the token's positions and gates, one per lane (k <= 64), in one load each; then groups of kJ
  // choices: every row load of a group in flight together, the sums in ascending j
  const int lane = threadIdx.x & 63;
  const int pv = lane < k ? inv[size_t(t) * k + lane] : -1;
  const float gv = lane < k ? w[size_t(t) * k + lane] : 0.0f;
  constexpr int kJ = 8;
  for (int j0 = 0; j0 < k; j0 += kJ) {
    int p[kJ];
    float g[kJ];
#pragma unroll
    for (int u = 0; u < kJ; ++u) {
      p[u] = __builtin_amdgcn_readlane(pv, j0 + u);
      g[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), j0 + u));
      if (j0 + u >= k || p[u] >= cap || !live) p[u] = -1;
    }
    float4 v[kJ];
#pragma unroll
    for (int u = 0; u < kJ; ++u) {
      v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (p[u] >= 0) v[u] = *reinterpret_cast<const float4*>(y + size_t(p[u]) * H + h);
    }
#pragma unroll
    for (int u = 0; u < kJ; ++u) {
      if (p[u] >= 0) {
        acc.x = fmaf(g[u], v[u].x, acc.x);
        acc.y = fmaf(g[u], v[u].y, acc.y);
        acc.z = fmaf(g[u], v[u].z, acc.z);
        acc.w = fmaf(g[u], v[u].w, acc.w);
      }
    }
  }
  if (!live) return;
  if constexpr (ODT == DT_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + size_t(t) * H + h) = acc;
  } else {
    uint2 o;
    o.x = uint32_t(f32_to_bf16(acc.x)) | (uint32_t(f32_to_bf16(acc.y)) << 16);
    o.y = uint32_t(f32_to_bf16(acc.z)) | (uint32_t(f32_to_bf16(acc.w)) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + size_t(t) * H + h) = o;
  }
}

hipError_t launch_combine(const float* y, const int32_t* inv, const float* w, int T, int k, int H,
                          void* out, int odt, hipStream_t st) {
  dim3 grid(T, (H / 4 + kCombThreads - 1) / kCombThreads), block(kCombThreads);
  const int cap = T * k;
  if (odt == DT_F32)
    combine_kernel<DT_F32><<<grid, block, 0, st>>>(y, inv, w, T, k, H, cap, out);
  else
    combine_kernel<DT_BF16><<<grid, block, 0, st>>>(y, inv, w, T, k, H, cap, out);
  return hipGetLastError();
}

}  // namespace moe
