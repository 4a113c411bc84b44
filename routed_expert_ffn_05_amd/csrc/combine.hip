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
  if (h >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int p = inv[size_t(t) * k + j];
    if (p < 0 || p >= cap) continue;
    const float g = w[size_t(t) * k + j];
    const float4 v = *reinterpret_cast<const float4*>(y + size_t(p) * H + h);
    acc.x = fmaf(g, v.x, acc.x);
    acc.y = fmaf(g, v.y, acc.y);
    acc.z = fmaf(g, v.z, acc.z);
    acc.w = fmaf(g, v.w, acc.w);
  }
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
