// Router: logits GEMV (x . W_r^T, fp32 accumulation) and the wavefront-per-token top-k with
// score and gate computation.
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

// ---------------------------------------------------------------------------------------------
// logits[t, e] = sum_h x[t,h] W_r[e,h] (+ bias[e])
// A work-group computes kRouterEpw expert rows: thread j owns the rows' 16-byte chunks j, j+256,
// ... (NCH per row, H <= 1024*NCH), all loaded before any arithmetic; the activations of TOK
// tokens (TOK >= T rounded up to 1, 2, 4 or 8; larger batches loop over groups of 8) are loaded
// once per work-group and used for every row it owns, so the activation bytes moved from L2 are
// shared by kRouterEpw rows.  Partial sums are reduced with DPP inside each wave and across the
// four waves through LDS.
// ---------------------------------------------------------------------------------------------
constexpr int kRouterThreads = 256;
constexpr int kRouterEpw = 2;  // one row per work-group measured slower at T = 4

template <int XDT, int NCH, int TOK>
__global__ __launch_bounds__(kRouterThreads) void router_logits_kernel(const void* __restrict__ x_,
                                                                       const float* __restrict__ wr,
                                                                       const float* __restrict__ bias,
                                                                       float* __restrict__ logits,
                                                                       int T, int H, int E) {
  __shared__ float part[kRouterThreads / 64][kRouterEpw][TOK];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int e0 = blockIdx.x * kRouterEpw;
  const int nch = H >> 2;
  // the bias of the (row, token) pair this thread stores, loaded with the weights
  const float bv = (bias && tid < kRouterEpw * TOK) ? bias[min(e0 + tid / TOK, E - 1)] : 0.0f;
  // chunks past the row re-read its last chunk and are weighted by zero; a row past E re-reads
  // the last row and is not stored
  float4 w[kRouterEpw][NCH];
#pragma unroll
  for (int r = 0; r < kRouterEpw; ++r) {
    const float4* wrow = reinterpret_cast<const float4*>(wr + size_t(min(e0 + r, E - 1)) * H);
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = tid + kRouterThreads * j;
      w[r][j] = wrow[min(c, nch - 1)];
      if (c >= nch) w[r][j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  }
  for (int t0 = 0; t0 < T; t0 += TOK) {
    float acc[kRouterEpw][TOK];
#pragma unroll
    for (int i = 0; i < TOK; ++i) {
      const int t = min(t0 + i, T - 1);  // tokens past T repeat the last one (not stored)
      float4 xv[NCH];
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = min(tid + kRouterThreads * j, nch - 1);
        if constexpr (XDT == DT_F32) {
          xv[j] = reinterpret_cast<const float4*>(static_cast<const float*>(x_) + size_t(t) * H)[c];
        } else {
          const uint2 u = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x_) + size_t(t) * H)[c];
          xv[j] = make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
        }
      }
#pragma unroll
      for (int r = 0; r < kRouterEpw; ++r) {
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          a = fmaf(w[r][j].x, xv[j].x, a);
          a = fmaf(w[r][j].y, xv[j].y, a);
          a = fmaf(w[r][j].z, xv[j].z, a);
          a = fmaf(w[r][j].w, xv[j].w, a);
        }
        acc[r][i] = a;
      }
    }
#pragma unroll
    for (int r = 0; r < kRouterEpw; ++r)
#pragma unroll
      for (int i = 0; i < TOK; ++i) {
        const float s = seg_sum<64>(acc[r][i]);
        if (lane == 63) part[wid][r][i] = s;
      }
    __syncthreads();
    if (tid < kRouterEpw * TOK) {
      const int r = tid / TOK, i = tid - r * TOK;
      const int e = e0 + r;
      if (e < E && t0 + i < T) {
        float s = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < kRouterThreads / 64; ++w2) s += part[w2][r][i];
        logits[size_t(t0 + i) * E + e] = s + bv;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// top-k: one wave per token
// ---------------------------------------------------------------------------------------------
template <int VPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   const float* __restrict__ bias, int add_bias,
                                                   int T, int E, int k, int score, int renorm,
                                                   int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_e;
  float my_w;
  topk_wave<VPL>(logits + size_t(t) * E, add_bias ? bias : nullptr, E, k, score, renorm, my_e, my_w);
  if (lane < k) {
    topk_idx[size_t(t) * k + lane] = my_e;
    topk_w[size_t(t) * k + lane] = my_w;
  }
}

hipError_t launch_router_logits(const void* x, int xdt, const float* wr, const float* bias,
                                float* logits, int T, int H, int E, hipStream_t st) {
  dim3 grid((E + kRouterEpw - 1) / kRouterEpw), block(kRouterThreads);
  const int nch = (H / 4 + kRouterThreads - 1) / kRouterThreads;  // chunks per thread and row
  const int tok = T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8;
#define MOE_ROUTER_LAUNCH_T(N, TK)                                                                  \
  {                                                                                                 \
    if (xdt == DT_F32)                                                                              \
      router_logits_kernel<DT_F32, N, TK><<<grid, block, 0, st>>>(x, wr, bias, logits, T, H, E);    \
    else                                                                                            \
      router_logits_kernel<DT_BF16, N, TK><<<grid, block, 0, st>>>(x, wr, bias, logits, T, H, E);   \
  }
#define MOE_ROUTER_LAUNCH(N)                         \
  {                                                  \
    if (tok == 1) MOE_ROUTER_LAUNCH_T(N, 1)          \
    else if (tok == 2) MOE_ROUTER_LAUNCH_T(N, 2)     \
    else if (tok == 4) MOE_ROUTER_LAUNCH_T(N, 4)     \
    else MOE_ROUTER_LAUNCH_T(N, 8)                   \
  }
  if (nch <= 1) MOE_ROUTER_LAUNCH(1)
  else if (nch <= 2) MOE_ROUTER_LAUNCH(2)
  else if (nch <= 4) MOE_ROUTER_LAUNCH(4)
  else MOE_ROUTER_LAUNCH(8)
#undef MOE_ROUTER_LAUNCH
#undef MOE_ROUTER_LAUNCH_T
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
  else if (vpl <= 6)
    topk_kernel<6><<<grid, block, 0, st>>>(logits, bias, add_bias, T, E, k, score, renorm, idx, w);
  else if (vpl <= 8)
    topk_kernel<8><<<grid, block, 0, st>>>(logits, bias, add_bias, T, E, k, score, renorm, idx, w);
  else
    topk_kernel<16><<<grid, block, 0, st>>>(logits, bias, add_bias, T, E, k, score, renorm, idx, w);
  return hipGetLastError();
}

}  // namespace moe
