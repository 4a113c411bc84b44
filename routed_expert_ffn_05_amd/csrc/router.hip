// Router: logits GEMV (x . W_r^T, fp32 accumulation) and a wavefront-per-token top-k with
// score and gate computation.
#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------------------------
// logits[t, e] = sum_h x[t,h] W_r[e,h] (+ bias[e])
// One wave per expert row; the row is read once for up to TCH tokens at a time (the weights are
// the large operand at decode sizes).  Lane l covers the 4-float chunks l, l+64, ...
// ---------------------------------------------------------------------------------------------
template <int XDT, int TCH>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ x_,
                                                            const float* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits, int T,
                                                            int H, int E) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const float4* wrow = reinterpret_cast<const float4*>(wr + size_t(e) * H);
  const int nch = H >> 2;
  const float b = bias ? bias[e] : 0.0f;
  for (int t0 = 0; t0 < T; t0 += TCH) {
    float acc[TCH];
#pragma unroll
    for (int i = 0; i < TCH; ++i) acc[i] = 0.0f;
    for (int c = lane; c < nch; c += 64) {
      const float4 w = wrow[c];
#pragma unroll
      for (int i = 0; i < TCH; ++i) {
        const int t = t0 + i;
        if (t < T) {
          float4 xv;
          if (XDT == DT_F32) {
            xv = reinterpret_cast<const float4*>(static_cast<const float*>(x_) + size_t(t) * H)[c];
          } else {
            const uint2 u = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x_) + size_t(t) * H)[c];
            xv = make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
          }
          acc[i] = fmaf(w.x, xv.x, acc[i]);
          acc[i] = fmaf(w.y, xv.y, acc[i]);
          acc[i] = fmaf(w.z, xv.z, acc[i]);
          acc[i] = fmaf(w.w, xv.w, acc[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < TCH; ++i) {
      const float s = wave_sum(acc[i]);
      if (lane == 0 && t0 + i < T) logits[size_t(t0 + i) * E + e] = s + b;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// top-k: one wave per token.  Lane l holds logits l, l+64, ... (up to 16 values, E <= 1024).
// k rounds of a wave-wide (value desc, id asc) argmax; then scores and gates in fp32.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int VPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   const float* __restrict__ bias, int add_bias,
                                                   int T, int E, int k, int score, int renorm,
                                                   int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float NEG = -__builtin_huge_valf();
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    float l = NEG;
    if (e < E) {
      l = logits[size_t(t) * E + e];
      if (add_bias) l += bias[e];
    }
    v[i] = l;
  }
  // softmax statistics over all E (only used for MOE_SCORE_SOFTMAX)
  float mx = NEG, z = 0.0f;
  if (score == 0) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) mx = fmaxf(mx, v[i]);
    mx = wave_max(mx);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) z += expf(v[i] - mx);
    z = wave_sum(z);
  }
  unsigned taken = 0;  // bit i: v[i] already selected
  float my_s = 0.0f;   // score of the expert this lane selected in round j (lane j keeps it)
  int my_e = 0;
  float ssum = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = NEG;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !(taken >> i & 1u) && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    // the owning lane marks it taken
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    const float s = (score == 0) ? expf(bv - mx) / z : 1.0f / (1.0f + expf(-bv));
    ssum += s;  // ascending j, identical on every lane
    if (lane == j) {
      my_s = s;
      my_e = bi;
    }
  }
  if (lane < k) {
    topk_idx[size_t(t) * k + lane] = my_e;
    topk_w[size_t(t) * k + lane] = renorm ? my_s / ssum : my_s;
  }
}

hipError_t launch_router_logits(const void* x, int xdt, const float* wr, const float* bias,
                                float* logits, int T, int H, int E, hipStream_t st) {
  dim3 grid((E + 3) / 4), block(256);
  if (xdt == DT_F32)
    router_logits_kernel<DT_F32, 8><<<grid, block, 0, st>>>(x, wr, bias, logits, T, H, E);
  else
    router_logits_kernel<DT_BF16, 8><<<grid, block, 0, st>>>(x, wr, bias, logits, T, H, E);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, const float* bias, int add_bias, int T, int E, int k,
                       int score, int renorm, int32_t* idx, float* w, hipStream_t st) {
  dim3 grid((T + 3) / 4), block(256);
  const int vpl = (E + 63) / 64;
  if (vpl <= 2)
    topk_kernel<2><<<grid, block, 0, st>>>(logits, bias, add_bias, T, E, k, score, renorm, idx, w);
  else if (vpl <= 4)
    topk_kernel<4><<<grid, block, 0, st>>>(logits, bias, add_bias, T, E, k, score, renorm, idx, w);
  else if (vpl <= 8)
    topk_kernel<8><<<grid, block, 0, st>>>(logits, bias, add_bias, T, E, k, score, renorm, idx, w);
  else
    topk_kernel<16><<<grid, block, 0, st>>>(logits, bias, add_bias, T, E, k, score, renorm, idx, w);
  return hipGetLastError();
}

}  // namespace moe
