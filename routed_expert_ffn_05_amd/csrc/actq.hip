// Mode B activation quantisation (OCP MX rule): per row and per 32 consecutive elements, a shared
// power-of-two scale 2^X with X = floor(log2 amax) - 8 (E4M3's largest exponent is 8; an all-zero
// block keeps X = 0), and E4M3 (e4m3fn) codes of v / 2^X rounded to nearest even and saturated at
// +-448.  Dividing by 2^X is exact, so code * 2^X is the quantised value exactly.
//
// Four lanes own one 32-element block (eight consecutive elements each); the block maximum is
// exchanged with two lane swaps inside the group.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kQThreads = 256;

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  const float v = e == 0 ? ldexpf(float(m), -9) : ldexpf(float(8 + m), e - 10);
  return (c & 0x80u) ? -v : v;
}

template <int IN, int DEQ>  // DEQ: DT_BF16, DT_F32, or -1 (no dequantised output)
__global__ __launch_bounds__(kQThreads) void act_quant_kernel(const void* __restrict__ in, int rows, int K,
                                                              const int32_t* __restrict__ nrows,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales, void* deq) {
  const int nb = K >> 5;
  const long long blk = (long long)(blockIdx.x) * (kQThreads / 4) + (threadIdx.x >> 2);
  const int part = threadIdx.x & 3;
  const int rlim = nrows ? min(rows, max(nrows[0], 0)) : rows;
  if (blk >= (long long)rlim * nb) return;  // the four lanes of a block leave together
  const size_t e0 = size_t(blk) * 32 + part * 8;  // first element of this lane (row-major)
  float v[8];
  if constexpr (IN == DT_F32) {
    const float4 p = reinterpret_cast<const float4*>(static_cast<const float*>(in) + e0)[0];
    const float4 q = reinterpret_cast<const float4*>(static_cast<const float*>(in) + e0)[1];
    v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w; v[4] = q.x; v[5] = q.y; v[6] = q.z; v[7] = q.w;
  } else {
    const uint4 p = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(in) + e0);
    v[0] = bf16_lo(p.x); v[1] = bf16_hi(p.x); v[2] = bf16_lo(p.y); v[3] = bf16_hi(p.y);
    v[4] = bf16_lo(p.z); v[5] = bf16_hi(p.z); v[6] = bf16_lo(p.w); v[7] = bf16_hi(p.w);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int X = mx_e4m3_exponent(amax);
  const float inv = ldexpf(1.0f, -X);
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = e4m3_code(v[i] * inv);
  if (codes) {
    uint2 o;
    o.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    o.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    *reinterpret_cast<uint2*>(codes + e0) = o;
  }
  if (scales && part == 0) scales[blk] = uint8_t(X + 127);
  if constexpr (DEQ == DT_F32) {
    float d[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = ldexpf(e4m3_value(c[i]), X);
    reinterpret_cast<float4*>(static_cast<float*>(deq) + e0)[0] = make_float4(d[0], d[1], d[2], d[3]);
    reinterpret_cast<float4*>(static_cast<float*>(deq) + e0)[1] = make_float4(d[4], d[5], d[6], d[7]);
  } else if constexpr (DEQ == DT_BF16) {
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = f32_to_bf16(ldexpf(e4m3_value(c[i]), X));  // exact in bf16
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(deq) + e0) =
        make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
  }
}

hipError_t launch_act_quant(const void* in, int in_dt, int rows, int K, const int32_t* nrows, uint8_t* codes,
                            uint8_t* scales, void* deq, int deq_dt, hipStream_t st) {
  const long long blocks = (long long)rows * (K >> 5);
  if (blocks == 0) return hipSuccess;
  dim3 grid(unsigned((blocks + kQThreads / 4 - 1) / (kQThreads / 4))), block(kQThreads);
#define MOE_AQ(I, D) act_quant_kernel<I, D><<<grid, block, 0, st>>>(in, rows, K, nrows, codes, scales, deq)
  if (in_dt == DT_F32) {
    if (!deq) MOE_AQ(DT_F32, -1);
    else if (deq_dt == DT_F32) MOE_AQ(DT_F32, DT_F32);
    else MOE_AQ(DT_F32, DT_BF16);
  } else {
    if (!deq) MOE_AQ(DT_BF16, -1);
    else if (deq_dt == DT_F32) MOE_AQ(DT_BF16, DT_F32);
    else MOE_AQ(DT_BF16, DT_BF16);
  }
#undef MOE_AQ
  return hipGetLastError();
}

}  // namespace moe
