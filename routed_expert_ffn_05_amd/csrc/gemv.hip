// Decode path: dequantising GEMVs over the touched expert slots.
//
//   gate/up:  a[p, i] = silu(W_g[s,i,:] . x_p) * (W_u[s,i,:] . x_p)   (W_gu rows i and I+i)
//   down:     y[p, h] = W_d[s,h,:] . a_p
//
// The weights are the large operand (a decode step touches each slot's bytes once for the few
// rows routed to it), so each kernel streams weight rows from HBM with 16-byte loads per lane
// and keeps the activations of up to kTok rows of the slot in LDS.  A 16-byte weight chunk
// holds 4 (fp32), 8 (bf16), 16 (fp8) or 32 (fp4) elements; lanes of a wave take consecutive
// chunks of a row (a row shorter than 64 chunks is shared by several lane groups), decode them
// in registers and reduce each row's partial sums across the lanes.  FP8 block scales multiply
// the per-chunk partial sums (a chunk never straddles a 128-wide K block); MXFP4 scales enter
// the e2m1 -> fp32 conversion directly (exact: powers of two).
//
// Grid: x = row blocks of the output, y = ordinal of the active (non-empty) slot; work-groups
// whose ordinal exceeds the number of active slots exit at once.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / 64;
constexpr int kTok = 4;           // rows of one slot whose inputs are staged together
constexpr int kGateUpPairs = 16;  // (gate, up) row pairs per work-group
constexpr int kDownRows = 64;     // output rows per work-group

template <int WD> struct WFmt;
template <> struct WFmt<DT_F32> { static constexpr int EPC = 4; };
template <> struct WFmt<DT_BF16> { static constexpr int EPC = 8; };
template <> struct WFmt<DT_FP8> { static constexpr int EPC = 16; };
template <> struct WFmt<DT_MXFP4> { static constexpr int EPC = 32; };

template <int WD>
__host__ __device__ constexpr size_t row_bytes(int K) {
  return WD == DT_F32 ? size_t(K) * 4 : WD == DT_BF16 ? size_t(K) * 2 : WD == DT_FP8 ? size_t(K) : size_t(K) / 2;
}

// decode one 16-byte chunk into EPC floats; MXFP4 applies `scale` (a power of two) exactly
template <int WD>
__device__ __forceinline__ void decode(const uint4 q, float scale, float* w) {
  const uint32_t u[4] = {q.x, q.y, q.z, q.w};
  if constexpr (WD == DT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __uint_as_float(u[i]);
  } else if constexpr (WD == DT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[2 * i] = bf16_lo(u[i]);
      w[2 * i + 1] = bf16_hi(u[i]);
    }
  } else if constexpr (WD == DT_FP8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float2 a = fp8x2_lo(u[i]), b = fp8x2_hi(u[i]);
      w[4 * i] = a.x;
      w[4 * i + 1] = a.y;
      w[4 * i + 2] = b.x;
      w[4 * i + 3] = b.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float2 a = fp4x2<0>(u[i], scale), b = fp4x2<1>(u[i], scale);
      const float2 c = fp4x2<2>(u[i], scale), d = fp4x2<3>(u[i], scale);
      w[8 * i + 0] = a.x;
      w[8 * i + 1] = a.y;
      w[8 * i + 2] = b.x;
      w[8 * i + 3] = b.y;
      w[8 * i + 4] = c.x;
      w[8 * i + 5] = c.y;
      w[8 * i + 6] = d.x;
      w[8 * i + 7] = d.y;
    }
  }
}

// EPC input values of chunk c from an LDS row (bf16 or fp32 storage)
template <int XT, int EPC>
__device__ __forceinline__ void load_in(const uint8_t* row, int c, float* xv) {
  if constexpr (XT == DT_BF16) {
    if constexpr (EPC == 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(row + size_t(c) * 8);
      xv[0] = bf16_lo(u.x);
      xv[1] = bf16_hi(u.x);
      xv[2] = bf16_lo(u.y);
      xv[3] = bf16_hi(u.y);
    } else {
#pragma unroll
      for (int j = 0; j < EPC / 8; ++j) {
        const uint4 u = *reinterpret_cast<const uint4*>(row + size_t(c) * EPC * 2 + 16 * j);
        xv[8 * j + 0] = bf16_lo(u.x);
        xv[8 * j + 1] = bf16_hi(u.x);
        xv[8 * j + 2] = bf16_lo(u.y);
        xv[8 * j + 3] = bf16_hi(u.y);
        xv[8 * j + 4] = bf16_lo(u.z);
        xv[8 * j + 5] = bf16_hi(u.z);
        xv[8 * j + 6] = bf16_lo(u.w);
        xv[8 * j + 7] = bf16_hi(u.w);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPC / 4; ++j) {
      const float4 f = *reinterpret_cast<const float4*>(row + size_t(c) * EPC * 4 + 16 * j);
      xv[4 * j + 0] = f.x;
      xv[4 * j + 1] = f.y;
      xv[4 * j + 2] = f.z;
      xv[4 * j + 3] = f.w;
    }
  }
}

// per-chunk scale of row n, chunk c: FP8 block scale (applied to the partial sum), MXFP4 E8M0
template <int WD>
__device__ __forceinline__ float chunk_scale(const void* s, int n, int c, int K) {
  if constexpr (WD == DT_FP8) {
    const int KB = (K + 127) >> 7;
    return static_cast<const float*>(s)[size_t(n >> 7) * KB + (c >> 3)];
  } else if constexpr (WD == DT_MXFP4) {
    return e8m0_to_f32(static_cast<const uint8_t*>(s)[size_t(n) * (K >> 5) + c]);
  } else {
    return 1.0f;
  }
}

// Two weight rows (n0, n1) of one slot against `ntok` staged input rows.  Lane `sl` of an
// LPR-lane group takes chunks sl, sl+LPR, ...; partial sums are left per lane.
template <int WD, int XT>
__device__ __forceinline__ void dot2(const uint8_t* __restrict__ w, const void* __restrict__ s,
                                     int n0, int n1, bool v0, bool v1, int K,
                                     const uint8_t* in, size_t in_stride, int ntok, int sl,
                                     int LPR, float (&acc0)[kTok], float (&acc1)[kTok]) {
  constexpr int EPC = WFmt<WD>::EPC;
  const int CPR = K / EPC;
  const size_t rb = row_bytes<WD>(K);
  const uint4* p0 = reinterpret_cast<const uint4*>(w + size_t(n0) * rb);
  const uint4* p1 = reinterpret_cast<const uint4*>(w + size_t(n1) * rb);
#pragma unroll 2
  for (int c = sl; c < CPR; c += LPR) {
    uint4 q0 = make_uint4(0, 0, 0, 0), q1 = make_uint4(0, 0, 0, 0);
    if (v0) q0 = ld_stream16(p0 + c);
    if (v1) q1 = ld_stream16(p1 + c);
    const float s0 = v0 ? chunk_scale<WD>(s, n0, c, K) : 0.0f;
    const float s1 = v1 ? chunk_scale<WD>(s, n1, c, K) : 0.0f;
    float w0[EPC], w1[EPC];
    decode<WD>(q0, s0, w0);
    decode<WD>(q1, s1, w1);
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
      if (t < ntok) {
        float xv[EPC];
        load_in<XT, EPC>(in + t * in_stride, c, xv);
        float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          d0 = fmaf(w0[e], xv[e], d0);
          d1 = fmaf(w1[e], xv[e], d1);
        }
        if constexpr (WD == DT_FP8) {
          acc0[t] = fmaf(s0, d0, acc0[t]);
          acc1[t] = fmaf(s1, d1, acc1[t]);
        } else {
          acc0[t] += d0;
          acc1[t] += d1;
        }
      }
    }
  }
}

__device__ __forceinline__ float group_sum(float v, int LPR) {
  for (int o = LPR >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int lanes_per_row(int CPR) {
  if (CPR >= 64) return 64;
  int l = 1;
  while (l < CPR) l <<= 1;
  return l;
}

// stage rows [p0, p0+ntok) of the slot: input row r = src row of position p (token perm[p]/k
// for x, position p itself for a), `bytes` per row, 16-byte granules
__device__ __forceinline__ void stage_rows(uint8_t* lds, const uint8_t* __restrict__ src,
                                           size_t src_stride, const int32_t* __restrict__ perm,
                                           int k, int T, int p0, int ntok, size_t bytes) {
  const int g = int(bytes >> 4);
  for (int i = threadIdx.x; i < ntok * g; i += kGemvThreads) {
    const int t = i / g, j = i - t * g;
    int row = p0 + t;
    bool ok = true;
    if (perm) {
      const int r = perm[row];
      row = r / k;
      ok = r >= 0 && row < T;
    }
    uint4 v = make_uint4(0, 0, 0, 0);
    if (ok) v = reinterpret_cast<const uint4*>(src + size_t(row) * src_stride)[j];
    reinterpret_cast<uint4*>(lds + size_t(t) * bytes)[j] = v;
  }
}

// ---------------------------------------------------------------------------------------------
template <int WD, int XT>
__global__ __launch_bounds__(kGemvThreads) void gemv_gate_up_kernel(
    const uint8_t* __restrict__ w_gu, const void* __restrict__ s_gu, const void* __restrict__ x,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ off, int S, int T, int k, int H,
    int I, float* __restrict__ a_out) {
  extern __shared__ __align__(16) uint8_t xs[];
  __shared__ int tmp[kGemvWaves + 1];
  const int s = find_active_slot<kGemvThreads>(off, S, blockIdx.y, tmp);
  if (s < 0) return;
  const int cap = T * k;
  const int lo = min(max(off[s], 0), cap), hi = min(max(off[s + 1], lo), cap);
  constexpr int EPC = WFmt<WD>::EPC;
  const int CPR = H / EPC;
  const int LPR = lanes_per_row(CPR);
  const int GPW = 64 / LPR;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int sub = lane / LPR, sl = lane - sub * LPR;
  const size_t xbytes = size_t(H) * (XT == DT_F32 ? 4 : 2);
  const uint8_t* wslot = w_gu + size_t(s) * 2 * I * row_bytes<WD>(H);
  const void* sslot = nullptr;
  if constexpr (WD == DT_FP8)
    sslot = static_cast<const float*>(s_gu) + size_t(s) * ((2 * I + 127) >> 7) * ((H + 127) >> 7);
  if constexpr (WD == DT_MXFP4) sslot = static_cast<const uint8_t*>(s_gu) + size_t(s) * 2 * I * (H >> 5);
  const int i0 = blockIdx.x * kGateUpPairs;
  const int i1 = min(I, i0 + kGateUpPairs);

  for (int p0 = lo; p0 < hi; p0 += kTok) {
    const int ntok = min(kTok, hi - p0);
    __syncthreads();
    stage_rows(xs, static_cast<const uint8_t*>(x), xbytes, perm, k, T, p0, ntok, xbytes);
    __syncthreads();
    for (int ib = i0 + wid * GPW; ib < i1; ib += kGemvWaves * GPW) {
      const int i = ib + sub;
      const bool v = i < i1;
      float ag[kTok], au[kTok];
#pragma unroll
      for (int t = 0; t < kTok; ++t) ag[t] = au[t] = 0.0f;
      dot2<WD, XT>(wslot, sslot, v ? i : 0, v ? I + i : 0, v, v, H, xs, xbytes, ntok, sl, LPR, ag, au);
#pragma unroll
      for (int t = 0; t < kTok; ++t) {
        if (t < ntok) {
          const float g = group_sum(ag[t], LPR), u = group_sum(au[t], LPR);
          if (v && sl == 0) a_out[size_t(p0 + t) * I + i] = silu(g) * u;
        }
      }
    }
  }
}

template <int WD>
__global__ __launch_bounds__(kGemvThreads) void gemv_down_kernel(
    const uint8_t* __restrict__ w_d, const void* __restrict__ s_d, const float* __restrict__ a,
    const int32_t* __restrict__ off, int S, int T, int k, int H, int I, float* __restrict__ y) {
  extern __shared__ __align__(16) uint8_t as[];
  __shared__ int tmp[kGemvWaves + 1];
  const int s = find_active_slot<kGemvThreads>(off, S, blockIdx.y, tmp);
  if (s < 0) return;
  const int cap = T * k;
  const int lo = min(max(off[s], 0), cap), hi = min(max(off[s + 1], lo), cap);
  constexpr int EPC = WFmt<WD>::EPC;
  const int CPR = I / EPC;
  const int LPR = lanes_per_row(CPR);
  const int GPW = 64 / LPR;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int sub = lane / LPR, sl = lane - sub * LPR;
  const size_t abytes = size_t(I) * 4;
  const uint8_t* wslot = w_d + size_t(s) * H * row_bytes<WD>(I);
  const void* sslot = nullptr;
  if constexpr (WD == DT_FP8)
    sslot = static_cast<const float*>(s_d) + size_t(s) * ((H + 127) >> 7) * ((I + 127) >> 7);
  if constexpr (WD == DT_MXFP4) sslot = static_cast<const uint8_t*>(s_d) + size_t(s) * H * (I >> 5);
  const int h0 = blockIdx.x * kDownRows;
  const int h1 = min(H, h0 + kDownRows);

  for (int p0 = lo; p0 < hi; p0 += kTok) {
    const int ntok = min(kTok, hi - p0);
    __syncthreads();
    stage_rows(as, reinterpret_cast<const uint8_t*>(a), abytes, nullptr, k, T, p0, ntok, abytes);
    __syncthreads();
    // two rows per group per step: hb + sub and hb + sub + GPW*kGemvWaves
    const int step = kGemvWaves * GPW;
    for (int hb = h0 + wid * GPW; hb < h1; hb += 2 * step) {
      const int ha = hb + sub, hc = hb + sub + step;
      const bool va = ha < h1, vc = hc < h1;
      float ya[kTok], yc[kTok];
#pragma unroll
      for (int t = 0; t < kTok; ++t) ya[t] = yc[t] = 0.0f;
      dot2<WD, DT_F32>(wslot, sslot, va ? ha : 0, vc ? hc : 0, va, vc, I, as, abytes, ntok, sl, LPR, ya, yc);
#pragma unroll
      for (int t = 0; t < kTok; ++t) {
        if (t < ntok) {
          const float r0 = group_sum(ya[t], LPR), r1 = group_sum(yc[t], LPR);
          if (sl == 0) {
            if (va) y[size_t(p0 + t) * H + ha] = r0;
            if (vc) y[size_t(p0 + t) * H + hc] = r1;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
template <int WD, int XT>
static hipError_t gate_up_t(const GemvArgs& g, hipStream_t st) {
  const size_t lds = size_t(kTok) * g.H * (XT == DT_F32 ? 4 : 2);
  auto kern = gemv_gate_up_kernel<WD, XT>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  dim3 grid((g.I + kGateUpPairs - 1) / kGateUpPairs, g.n_ord), block(kGemvThreads);
  kern<<<grid, block, lds, st>>>(static_cast<const uint8_t*>(g.w_gu), g.s_gu, g.x, g.perm, g.off,
                                 g.S, g.T, g.k, g.H, g.I, g.a);
  return hipGetLastError();
}

template <int WD>
static hipError_t down_t(const GemvArgs& g, hipStream_t st) {
  const size_t lds = size_t(kTok) * g.I * 4;
  auto kern = gemv_down_kernel<WD>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  dim3 grid((g.H + kDownRows - 1) / kDownRows, g.n_ord), block(kGemvThreads);
  kern<<<grid, block, lds, st>>>(static_cast<const uint8_t*>(g.w_d), g.s_d, g.a, g.off, g.S, g.T,
                                 g.k, g.H, g.I, g.y);
  return hipGetLastError();
}

hipError_t launch_gemv_gate_up(const GemvArgs& g, hipStream_t st) {
  const bool xf = g.xdt == DT_F32;
  switch (g.wdt) {
    case DT_F32: return xf ? gate_up_t<DT_F32, DT_F32>(g, st) : gate_up_t<DT_F32, DT_BF16>(g, st);
    case DT_BF16: return xf ? gate_up_t<DT_BF16, DT_F32>(g, st) : gate_up_t<DT_BF16, DT_BF16>(g, st);
    case DT_FP8: return xf ? gate_up_t<DT_FP8, DT_F32>(g, st) : gate_up_t<DT_FP8, DT_BF16>(g, st);
    case DT_MXFP4: return xf ? gate_up_t<DT_MXFP4, DT_F32>(g, st) : gate_up_t<DT_MXFP4, DT_BF16>(g, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_down(const GemvArgs& g, hipStream_t st) {
  switch (g.wdt) {
    case DT_F32: return down_t<DT_F32>(g, st);
    case DT_BF16: return down_t<DT_BF16>(g, st);
    case DT_FP8: return down_t<DT_FP8>(g, st);
    case DT_MXFP4: return down_t<DT_MXFP4>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
