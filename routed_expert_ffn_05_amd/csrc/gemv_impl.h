// Decode path: dequantising GEMVs over the touched expert slots (included once per weight format
// by gemv_<fmt>.hip).
//
//   gate/up:  a[p, i] = silu(W_g[s,i,:] . x_p) * (W_u[s,i,:] . x_p)   (W_gu rows i and I+i)
//   down:     y[p, h] = W_d[s,h,:] . a_p
//
// At decode sizes the weights are the only large operand: a call touches each routed slot's bytes
// once for the one or two rows routed to it.  The kernels therefore stream weight rows from HBM
// with 16-byte loads and keep everything else in registers:
//   * a row of K elements is cut into 16-byte chunks of EPC elements (4 fp32, 8 bf16, 16 fp8,
//     32 fp4); a group of LPR lanes shares a row, lane l of the group owning chunks l, l+LPR, ...
//     (CPL chunks per lane), so consecutive lanes read consecutive 16 bytes;
//   * the activations of the row's tokens at exactly those positions are loaded once per
//     work-group into registers (they are the same for every row the lane visits);
//   * ROWS rows are loaded per step (ROWS*CPL 16-byte loads in flight per lane), decoded in
//     registers (FP8 partial sums times the 128x128 block scale; MXFP4 through the scaled e2m1
//     conversion, exact for power-of-two scales) and accumulated in fp32;
//   * per-row sums are reduced across the LPR lanes with DPP row shifts and row broadcasts.
// Grid: x = row blocks of the output, y = ordinal of the active (non-empty) slot.
#pragma once
#include "common.h"
#include "kernels.h"

#ifndef MOE_GEMV_WD
#error "define MOE_GEMV_WD before including gemv_impl.h"
#endif

namespace moe {
namespace gemv {

// Tuning constants (compile-time; the defaults were chosen by timing on MI355X).
#ifndef MOE_GEMV_ITERS
#define MOE_GEMV_ITERS 4          // most row steps per wave and work-group
#endif
#ifndef MOE_GEMV_LOADS
#define MOE_GEMV_LOADS 8          // gate/up: 16-byte weight loads in flight per lane and row step
#endif
#ifndef MOE_GEMV_LOADS_DOWN
#define MOE_GEMV_LOADS_DOWN 4     // down (short rows of I elements): the same, per row step
#endif
#ifndef MOE_GEMV_TARGET_BLOCKS
#define MOE_GEMV_TARGET_BLOCKS 4096  // fewer row steps per work-group until the grid has this many
#endif
#ifndef MOE_GEMV_NT
#define MOE_GEMV_NT 1             // non-temporal (streaming) weight loads
#endif

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTok = 1;           // token rows of one slot handled per pass (weights re-read from L2 for more)
constexpr int kIters = MOE_GEMV_ITERS;

__device__ __forceinline__ uint4 ld_weight16(const uint4* p) {
#if MOE_GEMV_NT
  return ld_stream16(p);
#else
  return *p;
#endif
}

template <int WD> struct WFmt;
template <> struct WFmt<DT_F32> { static constexpr int EPC = 4; };
template <> struct WFmt<DT_BF16> { static constexpr int EPC = 8; };
template <> struct WFmt<DT_FP8> { static constexpr int EPC = 16; };
template <> struct WFmt<DT_MXFP4> { static constexpr int EPC = 32; };

template <int WD>
__host__ __device__ constexpr size_t row_bytes(int K) {
  return WD == DT_F32 ? size_t(K) * 4 : WD == DT_BF16 ? size_t(K) * 2 : WD == DT_FP8 ? size_t(K) : size_t(K) / 2;
}

// ---------------------------------------------------------------------------------------------
// chunk decode
// ---------------------------------------------------------------------------------------------
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

// per-chunk scale of row n, chunk c: FP8 block scale (multiplies the chunk's partial sum) or the
// MXFP4 E8M0 block scale (enters the conversion)
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

// ---------------------------------------------------------------------------------------------
// Inputs of the dot products.  A provider hands out, for token t and the lane's j-th chunk
// (chunk index c), the EPC input values at that chunk's K positions.
//   RegIn: one token, the lane's whole slice held in registers (loaded once per work-group);
//   LdsIn: up to kTokL tokens staged in LDS, read with 16-byte LDS loads.
// ---------------------------------------------------------------------------------------------
template <int XT, int EPC, int CPL>
struct RegIn {
  static constexpr int PK = XT == DT_BF16 ? 2 : 1;
  static constexpr int WPC = EPC / PK;  // 32-bit words per chunk
  uint32_t w[CPL * WPC];

  __device__ __forceinline__ void load(const void* row, int sl, int LPR, int CPR, bool ok) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = sl + LPR * j;
      const bool v = ok && c < CPR;
      const uint32_t* src = static_cast<const uint32_t*>(row) + size_t(c) * WPC;
      if constexpr (WPC % 4 == 0) {
#pragma unroll
        for (int q = 0; q < WPC / 4; ++q) {
          uint4 t = make_uint4(0, 0, 0, 0);
          if (v) t = reinterpret_cast<const uint4*>(src)[q];
          w[j * WPC + 4 * q + 0] = t.x;
          w[j * WPC + 4 * q + 1] = t.y;
          w[j * WPC + 4 * q + 2] = t.z;
          w[j * WPC + 4 * q + 3] = t.w;
        }
      } else {  // WPC == 2 (fp32 weights, bf16 inputs)
        uint2 t = make_uint2(0, 0);
        if (v) t = *reinterpret_cast<const uint2*>(src);
        w[j * WPC + 0] = t.x;
        w[j * WPC + 1] = t.y;
      }
    }
  }
  __device__ __forceinline__ void chunk(int /*t*/, int j, int /*c*/, float* xv) const {
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      if constexpr (PK == 2) {
        const uint32_t u = w[j * WPC + (e >> 1)];
        xv[e] = (e & 1) ? bf16_hi(u) : bf16_lo(u);
      } else {
        xv[e] = __uint_as_float(w[j * WPC + e]);
      }
    }
  }
};

template <int XT, int EPC>
struct LdsIn {
  const uint8_t* base;  // token t's row at base + t * stride
  size_t stride;
  __device__ __forceinline__ void chunk(int t, int /*j*/, int c, float* xv) const {
    const uint8_t* row = base + size_t(t) * stride;
    if constexpr (XT == DT_BF16) {
      if constexpr (EPC == 4) {
        const uint2 u = *reinterpret_cast<const uint2*>(row + size_t(c) * 8);
        xv[0] = bf16_lo(u.x);
        xv[1] = bf16_hi(u.x);
        xv[2] = bf16_lo(u.y);
        xv[3] = bf16_hi(u.y);
      } else {
#pragma unroll
        for (int q = 0; q < EPC / 8; ++q) {
          const uint4 u = *reinterpret_cast<const uint4*>(row + size_t(c) * EPC * 2 + 16 * q);
          xv[8 * q + 0] = bf16_lo(u.x);
          xv[8 * q + 1] = bf16_hi(u.x);
          xv[8 * q + 2] = bf16_lo(u.y);
          xv[8 * q + 3] = bf16_hi(u.y);
          xv[8 * q + 4] = bf16_lo(u.z);
          xv[8 * q + 5] = bf16_hi(u.z);
          xv[8 * q + 6] = bf16_lo(u.w);
          xv[8 * q + 7] = bf16_hi(u.w);
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < EPC / 4; ++q) {
        const float4 f = *reinterpret_cast<const float4*>(row + size_t(c) * EPC * 4 + 16 * q);
        xv[4 * q + 0] = f.x;
        xv[4 * q + 1] = f.y;
        xv[4 * q + 2] = f.z;
        xv[4 * q + 3] = f.w;
      }
    }
  }
};

constexpr int kTokL = 4;  // tokens staged together in LDS when a slot has several rows

// ROWS weight rows of one slot (row ids n[r], validity v[r]) against `nt` (<= NT) input rows:
// all ROWS*CPL 16-byte weight loads are issued first, then decoded and accumulated.
template <int WD, int CPL, int ROWS, int NT, typename In>
__device__ __forceinline__ void dot_rows(const uint8_t* __restrict__ w, const void* __restrict__ s,
                                         const int (&n)[ROWS], const bool (&v)[ROWS], int K, int sl,
                                         int LPR, const In& x, int nt, float (&acc)[ROWS][NT]) {
  constexpr int EPC = WFmt<WD>::EPC;
  const int CPR = K / EPC;
  const size_t rb = row_bytes<WD>(K);
  uint4 q[ROWS][CPL];
  float sc[ROWS][CPL];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const uint4* p = reinterpret_cast<const uint4*>(w + size_t(n[r]) * rb);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = sl + LPR * j;
      const bool ok = v[r] && c < CPR;
      q[r][j] = ok ? ld_weight16(p + c) : make_uint4(0, 0, 0, 0);
      sc[r][j] = ok ? chunk_scale<WD>(s, n[r], c, K) : 0.0f;
    }
  }
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = sl + LPR * j;
    if (c >= CPR) continue;
    if constexpr (NT == 1) {  // one input row: decode and consume row by row
      float xv[EPC];
      x.chunk(0, j, c, xv);
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        float wv[EPC];
        decode<WD>(q[r][j], sc[r][j], wv);
        float d = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) d = fmaf(wv[e], xv[e], d);
        if constexpr (WD == DT_FP8)
          acc[r][0] = fmaf(sc[r][j], d, acc[r][0]);
        else
          acc[r][0] += d;
      }
    } else {  // several input rows: decode each weight chunk once, use it for every row
      float wv[ROWS][EPC];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) decode<WD>(q[r][j], sc[r][j], wv[r]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < nt) {
          float xv[EPC];
          x.chunk(t, j, c, xv);
#pragma unroll
          for (int r = 0; r < ROWS; ++r) {
            float d = 0.0f;
#pragma unroll
            for (int e = 0; e < EPC; ++e) d = fmaf(wv[r][e], xv[e], d);
            if constexpr (WD == DT_FP8)
              acc[r][t] = fmaf(sc[r][j], d, acc[r][t]);
            else
              acc[r][t] += d;
          }
        }
      }
    }
  }
}

template <int CPL, int LOADS = MOE_GEMV_LOADS>
__host__ __device__ constexpr int rows_per_step() {
  return CPL >= LOADS ? 1 : LOADS / CPL;
}

// stage the input rows of positions [p0, p0+nt) into LDS: x rows of tokens perm[p]/k, or the
// rows p of `a` (perm == nullptr); 16-byte granules; rows of invalid tokens become zeros
__device__ __forceinline__ void stage_rows(uint8_t* lds, const uint8_t* __restrict__ src,
                                           size_t bytes, const int32_t* __restrict__ perm, int k,
                                           int T, int p0, int nt) {
  const int g = int(bytes >> 4);
  for (int i = threadIdx.x; i < nt * g; i += kThreads) {
    const int t = i / g, j = i - t * g;
    int row = p0 + t;
    bool ok = true;
    if (perm) {
      const int r = perm[row];
      row = r / k;
      ok = r >= 0 && row < T;
    }
    uint4 val = make_uint4(0, 0, 0, 0);
    if (ok) val = reinterpret_cast<const uint4*>(src + size_t(row) * bytes)[j];
    reinterpret_cast<uint4*>(lds + size_t(t) * bytes)[j] = val;
  }
}

// ---------------------------------------------------------------------------------------------
// gate/up + SiLU*mul
// ---------------------------------------------------------------------------------------------
template <int WD, int XT, int LPR, int CPL>
__global__ __launch_bounds__(kThreads) void gate_up_kernel(
    const uint8_t* __restrict__ w_gu, const void* __restrict__ s_gu, const void* __restrict__ x,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ off, int S, int T, int k, int H,
    int I, int iters, float* __restrict__ a_out) {
  constexpr int EPC = WFmt<WD>::EPC;
  constexpr int GPW = 64 / LPR;
  constexpr int PAIRS = rows_per_step<CPL>() / 2 > 0 ? rows_per_step<CPL>() / 2 : 1;  // pairs per group-step
  constexpr int ROWS = 2 * PAIRS;
  extern __shared__ __align__(16) uint8_t xs_lds[];
  __shared__ int tmp[kWaves + 1];
  const int s = find_active_slot<kThreads>(off, S, blockIdx.y, tmp);
  if (s < 0) return;
  const int cap = T * k;
  const int lo = min(max(off[s], 0), cap), hi = min(max(off[s + 1], lo), cap);
  const int CPR = H / EPC;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int grp = lane / LPR, sl = lane - grp * LPR;
  const size_t xrow = size_t(H) * (XT == DT_F32 ? 4 : 2);
  const uint8_t* wslot = w_gu + size_t(s) * 2 * I * row_bytes<WD>(H);
  const void* sslot = nullptr;
  if constexpr (WD == DT_FP8)
    sslot = static_cast<const float*>(s_gu) + size_t(s) * ((2 * I + 127) >> 7) * ((H + 127) >> 7);
  if constexpr (WD == DT_MXFP4) sslot = static_cast<const uint8_t*>(s_gu) + size_t(s) * 2 * I * (H >> 5);
  // pair indices: block b covers [b*span, (b+1)*span); step m of wave w, group g, pair q:
  //   i = base + ((m*kWaves + w)*GPW + g)*PAIRS + q
  const int span = iters * kWaves * GPW * PAIRS;
  const int i0 = blockIdx.x * span;

  auto pair_rows = [&](int m, int (&n)[ROWS], bool (&v)[ROWS]) {
    const int ib = i0 + ((m * kWaves + wid) * GPW + grp) * PAIRS;
#pragma unroll
    for (int q = 0; q < PAIRS; ++q) {
      const int i = ib + q;
      v[2 * q] = v[2 * q + 1] = i < I;
      n[2 * q] = i < I ? i : 0;
      n[2 * q + 1] = i < I ? I + i : 0;
    }
    return ib;
  };

  if (hi - lo == 1) {  // one row: the token's slice of x lives in registers
    RegIn<XT, EPC, CPL> xr;
    const int r = perm[lo];
    const int tok = (r >= 0 && r / k < T) ? r / k : -1;
    xr.load(static_cast<const uint8_t*>(x) + size_t(tok < 0 ? 0 : tok) * xrow, sl, LPR, CPR, tok >= 0);
    for (int m = 0; m < iters; ++m) {
      int n[ROWS];
      bool v[ROWS];
      const int ib = pair_rows(m, n, v);
      float acc[ROWS][1];
#pragma unroll
      for (int rr = 0; rr < ROWS; ++rr) acc[rr][0] = 0.0f;
      dot_rows<WD, CPL, ROWS, 1>(wslot, sslot, n, v, H, sl, LPR, xr, 1, acc);
#pragma unroll
      for (int q = 0; q < PAIRS; ++q) {
        const float g = seg_sum<LPR>(acc[2 * q][0]);
        const float u = seg_sum<LPR>(acc[2 * q + 1][0]);
        if (sl == LPR - 1 && v[2 * q]) a_out[size_t(lo) * I + ib + q] = silu(g) * u;
      }
    }
    return;
  }
  // several rows: up to kTokL tokens' x rows staged in LDS, each weight chunk used for all of
  // them; one (gate, up) pair per group step
  const LdsIn<XT, EPC> xl{xs_lds, xrow};
  for (int p0 = lo; p0 < hi; p0 += kTokL) {
    const int nt = min(kTokL, hi - p0);
    __syncthreads();
    stage_rows(xs_lds, static_cast<const uint8_t*>(x), xrow, perm, k, T, p0, nt);
    __syncthreads();
    for (int m = 0; m < iters; ++m) {
      int nn[ROWS];
      bool vv[ROWS];
      const int ib = pair_rows(m, nn, vv);
      for (int q = 0; q < PAIRS; ++q) {
        const int n[2] = {nn[2 * q], nn[2 * q + 1]};
        const bool v[2] = {vv[2 * q], vv[2 * q + 1]};
        float acc[2][kTokL];
#pragma unroll
        for (int t = 0; t < kTokL; ++t) acc[0][t] = acc[1][t] = 0.0f;
        dot_rows<WD, CPL, 2, kTokL>(wslot, sslot, n, v, H, sl, LPR, xl, nt, acc);
#pragma unroll
        for (int t = 0; t < kTokL; ++t) {
          if (t < nt) {
            const float g = seg_sum<LPR>(acc[0][t]);
            const float u = seg_sum<LPR>(acc[1][t]);
            if (sl == LPR - 1 && v[0]) a_out[size_t(p0 + t) * I + ib + q] = silu(g) * u;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// down projection
// ---------------------------------------------------------------------------------------------
template <int WD, int LPR, int CPL, int LOADS = MOE_GEMV_LOADS_DOWN>
__global__ __launch_bounds__(kThreads) void down_kernel(
    const uint8_t* __restrict__ w_d, const void* __restrict__ s_d, const float* __restrict__ a,
    const int32_t* __restrict__ off, int S, int T, int k, int H, int I, int iters,
    float* __restrict__ y) {
  constexpr int EPC = WFmt<WD>::EPC;
  constexpr int GPW = 64 / LPR;
  constexpr int ROWS = rows_per_step<CPL, LOADS>();
  extern __shared__ __align__(16) uint8_t as_lds[];
  __shared__ int tmp[kWaves + 1];
  const int s = find_active_slot<kThreads>(off, S, blockIdx.y, tmp);
  if (s < 0) return;
  const int cap = T * k;
  const int lo = min(max(off[s], 0), cap), hi = min(max(off[s + 1], lo), cap);
  const int CPR = I / EPC;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int grp = lane / LPR, sl = lane - grp * LPR;
  const uint8_t* wslot = w_d + size_t(s) * H * row_bytes<WD>(I);
  const void* sslot = nullptr;
  if constexpr (WD == DT_FP8)
    sslot = static_cast<const float*>(s_d) + size_t(s) * ((H + 127) >> 7) * ((I + 127) >> 7);
  if constexpr (WD == DT_MXFP4) sslot = static_cast<const uint8_t*>(s_d) + size_t(s) * H * (I >> 5);
  const int span = iters * kWaves * GPW * ROWS;
  const int h0 = blockIdx.x * span;
  const size_t arow = size_t(I) * 4;

  auto out_rows = [&](int m, int (&n)[ROWS], bool (&v)[ROWS]) {
    const int hb = h0 + ((m * kWaves + wid) * GPW + grp) * ROWS;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      v[r] = hb + r < H;
      n[r] = v[r] ? hb + r : 0;
    }
    return hb;
  };

  if (hi - lo == 1) {
    RegIn<DT_F32, EPC, CPL> ar;
    ar.load(a + size_t(lo) * I, sl, LPR, CPR, true);
    for (int m = 0; m < iters; ++m) {
      int n[ROWS];
      bool v[ROWS];
      const int hb = out_rows(m, n, v);
      float acc[ROWS][1];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) acc[r][0] = 0.0f;
      dot_rows<WD, CPL, ROWS, 1>(wslot, sslot, n, v, I, sl, LPR, ar, 1, acc);
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const float sum = seg_sum<LPR>(acc[r][0]);
        if (sl == LPR - 1 && v[r]) y[size_t(lo) * H + hb + r] = sum;
      }
    }
    return;
  }
  // several rows: up to kTokL rows of `a` staged in LDS; two output rows per group step
  const LdsIn<DT_F32, EPC> al{as_lds, arow};
  constexpr int RL = ROWS < 2 ? ROWS : 2;
  for (int p0 = lo; p0 < hi; p0 += kTokL) {
    const int nt = min(kTokL, hi - p0);
    __syncthreads();
    stage_rows(as_lds, reinterpret_cast<const uint8_t*>(a), arow, nullptr, k, T, p0, nt);
    __syncthreads();
    for (int m = 0; m < iters; ++m) {
      int nn[ROWS];
      bool vv[ROWS];
      const int hb = out_rows(m, nn, vv);
      for (int r0 = 0; r0 < ROWS; r0 += RL) {
        int n[RL];
        bool v[RL];
#pragma unroll
        for (int r = 0; r < RL; ++r) {
          n[r] = nn[r0 + r];
          v[r] = vv[r0 + r];
        }
        float acc[RL][kTokL];
#pragma unroll
        for (int r = 0; r < RL; ++r)
#pragma unroll
          for (int t = 0; t < kTokL; ++t) acc[r][t] = 0.0f;
        dot_rows<WD, CPL, RL, kTokL>(wslot, sslot, n, v, I, sl, LPR, al, nt, acc);
#pragma unroll
        for (int r = 0; r < RL; ++r) {
#pragma unroll
          for (int t = 0; t < kTokL; ++t) {
            if (t < nt) {
              const float sum = seg_sum<LPR>(acc[r][t]);
              if (sl == LPR - 1 && v[r]) y[size_t(p0 + t) * H + hb + r0 + r] = sum;
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// host dispatch
// ---------------------------------------------------------------------------------------------
// lanes per row and chunks per lane for a row of CPR chunks
inline void pick_lpr_cpl(int CPR, int& lpr, int& cpl) {
  if (CPR <= 16) {
    lpr = 16;
    cpl = 1;
  } else if (CPR <= 32) {
    lpr = 32;
    cpl = 1;
  } else {
    lpr = 64;
    const int need = (CPR + 63) / 64;
    cpl = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 16;
  }
}

// row steps per wave: enough work-groups to fill the chip when few slots are active
inline int pick_iters(int rows_total, int rows_per_block_step, int n_ord) {
  int iters = kIters;
  while (iters > 1) {
    const int blocks = (rows_total + rows_per_block_step * iters - 1) / (rows_per_block_step * iters);
    if ((long long)blocks * n_ord >= MOE_GEMV_TARGET_BLOCKS) break;
    iters >>= 1;
  }
  return iters;
}

template <int WD, int XT, int LPR, int CPL>
hipError_t launch_gate_up_t(const GemvArgs& g, hipStream_t st) {
  constexpr int ROWS = rows_per_step<CPL>();
  constexpr int PAIRS = ROWS / 2 > 0 ? ROWS / 2 : 1;
  const int step = kWaves * (64 / LPR) * PAIRS;
  const int iters = pick_iters(g.I, step, g.n_ord);
  dim3 grid((g.I + step * iters - 1) / (step * iters), g.n_ord), block(kThreads);
  const size_t lds = size_t(kTokL) * g.H * (XT == DT_F32 ? 4 : 2);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)gate_up_kernel<WD, XT, LPR, CPL>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  gate_up_kernel<WD, XT, LPR, CPL><<<grid, block, lds, st>>>(
      static_cast<const uint8_t*>(g.w_gu), g.s_gu, g.x, g.perm, g.off, g.S, g.T, g.k, g.H, g.I, iters, g.a);
  return hipGetLastError();
}

template <int WD, int LPR, int CPL, int LOADS = MOE_GEMV_LOADS_DOWN>
hipError_t launch_down_t(const GemvArgs& g, hipStream_t st) {
  constexpr int ROWS = rows_per_step<CPL, LOADS>();
  const int step = kWaves * (64 / LPR) * ROWS;
  const int iters = pick_iters(g.H, step, g.n_ord);
  dim3 grid((g.H + step * iters - 1) / (step * iters), g.n_ord), block(kThreads);
  const size_t lds = size_t(kTokL) * g.I * 4;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)down_kernel<WD, LPR, CPL, LOADS>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  down_kernel<WD, LPR, CPL, LOADS><<<grid, block, lds, st>>>(static_cast<const uint8_t*>(g.w_d), g.s_d, g.a, g.off,
                                                            g.S, g.T, g.k, g.H, g.I, iters, g.y);
  return hipGetLastError();
}

template <int WD, int XT>
hipError_t gate_up_dispatch(const GemvArgs& g, hipStream_t st) {
  int lpr, cpl;
  pick_lpr_cpl(g.H / WFmt<WD>::EPC, lpr, cpl);
  if (lpr == 16) return launch_gate_up_t<WD, XT, 16, 1>(g, st);
  if (lpr == 32) return launch_gate_up_t<WD, XT, 32, 1>(g, st);
  switch (cpl) {
    case 1: return launch_gate_up_t<WD, XT, 64, 1>(g, st);
    case 2: return launch_gate_up_t<WD, XT, 64, 2>(g, st);
    case 4: return launch_gate_up_t<WD, XT, 64, 4>(g, st);
    case 8: return launch_gate_up_t<WD, XT, 64, 8>(g, st);
    default: return launch_gate_up_t<WD, XT, 64, 16>(g, st);
  }
}

template <int WD>
hipError_t down_dispatch(const GemvArgs& g, hipStream_t st) {
  int lpr, cpl;
  pick_lpr_cpl(g.I / WFmt<WD>::EPC, lpr, cpl);
  // rows of exactly 64 chunks (e.g. I = 1024 FP8): 16 lanes of 4 chunks per row and two rows per
  // step (measured: 13 % less time than 64 lanes of one chunk at the FP8 decode shape)
  if (g.I / WFmt<WD>::EPC == 64) return launch_down_t<WD, 16, 4, 8>(g, st);
  if (lpr == 16) return launch_down_t<WD, 16, 1>(g, st);
  if (lpr == 32) return launch_down_t<WD, 32, 1>(g, st);
  switch (cpl) {
    case 1: return launch_down_t<WD, 64, 1>(g, st);
    case 2: return launch_down_t<WD, 64, 2>(g, st);
    case 4: return launch_down_t<WD, 64, 4>(g, st);
    case 8: return launch_down_t<WD, 64, 8>(g, st);
    default: return launch_down_t<WD, 64, 16>(g, st);
  }
}

}  // namespace gemv
}  // namespace moe
