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
#include "topk.h"

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
#define MOE_GEMV_TARGET_BLOCKS 4096  // fewer row steps per work-group until the grid has this many,
#endif
#ifndef MOE_GEMV_TARGET_BLOCKS_MAX
#define MOE_GEMV_TARGET_BLOCKS_MAX 8192  // and on to this many while the byte floors below hold
#endif
#ifndef MOE_GEMV_WG_BYTES_GU
#define MOE_GEMV_WG_BYTES_GU 65536   // gate/up: weight bytes a work-group streams, at least
#endif
#ifndef MOE_GEMV_WG_BYTES_DN
#define MOE_GEMV_WG_BYTES_DN 32768   // down: the same
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

// The chunk's weights as bf16 pairs (pair p holds elements 2p, 2p+1): exact for bf16, e4m3 and
// e2m1 times a power-of-two scale (the conversion applies the MXFP4 scale; the FP8 block scale
// multiplies the chunk's partial sum later).
template <int WD>
__device__ __forceinline__ void decode_pairs(const uint4 q, float scale, uint32_t* wp) {
  const uint32_t u[4] = {q.x, q.y, q.z, q.w};
  if constexpr (WD == DT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) wp[i] = u[i];
  } else if constexpr (WD == DT_FP8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wp[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u[i], 1.0f, false));
      wp[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u[i], 1.0f, true));
    }
  } else if constexpr (WD == DT_MXFP4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wp[4 * i + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u[i], scale, 0));
      wp[4 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u[i], scale, 1));
      wp[4 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u[i], scale, 2));
      wp[4 * i + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u[i], scale, 3));
    }
  }
}

// A chunk's partial dot product in a fixed association: element e (pair p) goes to partial sum
// e % 4 (p % 4), and the result is (s0 + s1) + (s2 + s3).  Four independent chains instead of
// one keep the FMA pipeline busy; every GEMV launch forms its sums this way, so the decode flows
// give the same bits.  dot_pairs multiplies bf16 pairs with v_dot2 (both products exact in fp32).
template <int EPC>
__device__ __forceinline__ float dot_f32(const float* w, const float* x) {
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
  for (int e = 0; e < EPC; e += 4) {
    s0 = fmaf(w[e], x[e], s0);
    s1 = fmaf(w[e + 1], x[e + 1], s1);
    s2 = fmaf(w[e + 2], x[e + 2], s2);
    s3 = fmaf(w[e + 3], x[e + 3], s3);
  }
  return (s0 + s1) + (s2 + s3);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <int NP>
__device__ __forceinline__ float dot_pairs(const uint32_t* w, const uint32_t* x) {
  static_assert(NP % 4 == 0, "pairs");
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
  for (int p = 0; p < NP; p += 4) {
    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[p]), __builtin_bit_cast(bf16x2_t, x[p]), s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[p + 1]), __builtin_bit_cast(bf16x2_t, x[p + 1]), s1, false);
    s2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[p + 2]), __builtin_bit_cast(bf16x2_t, x[p + 2]), s2, false);
    s3 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[p + 3]), __builtin_bit_cast(bf16x2_t, x[p + 3]), s3, false);
  }
  return (s0 + s1) + (s2 + s3);
}
// bf16 inputs meet bf16-convertible weights (bf16, FP8, MXFP4) on v_dot2; anything with an fp32
// operand on fmaf
template <int WD, int XT>
__host__ __device__ constexpr bool packed_dot() { return XT == DT_BF16 && WD != DT_F32; }

// Per-chunk scale of row n, chunk c, in two halves: chunk_scale_bits loads the stored bits (the
// FP8 block scale's fp32 bits, or the MXFP4 E8M0 byte), scale_of turns them into the value (the
// factor of the chunk's FP8 partial sum, or the MXFP4 scale the conversion applies).  Keeping the
// conversion out of the load phase lets every load of a row step be in flight before the first
// is consumed.
template <int WD>
__device__ __forceinline__ uint32_t chunk_scale_bits(const void* s, int n, int c, int K) {
  if constexpr (WD == DT_FP8) {
    const int KB = (K + 127) >> 7;
    return static_cast<const uint32_t*>(s)[size_t(n >> 7) * KB + (c >> 3)];
  } else if constexpr (WD == DT_MXFP4) {
    return static_cast<const uint8_t*>(s)[size_t(n) * (K >> 5) + c];
  } else {
    return 0u;
  }
}
template <int WD>
__device__ __forceinline__ float scale_of(uint32_t bits) {
  if constexpr (WD == DT_FP8) return __uint_as_float(bits);
  else if constexpr (WD == DT_MXFP4) return e8m0_to_f32(bits);
  else return 1.0f;
}

// ---------------------------------------------------------------------------------------------
// Inputs of the dot products.  A provider hands out, for token t and the lane's j-th chunk
// (chunk index c), the EPC input values at that chunk's K positions.
//   RegIn: one token, the lane's whole slice held in registers (loaded once per work-group);
//   LdsIn: up to kTokL tokens staged in LDS, read with 16-byte LDS loads.
// ---------------------------------------------------------------------------------------------
template <int XT, int EPC, int CPL>
struct RegIn {
  static constexpr int kXT = XT;
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
  // bf16 inputs as packed pairs (EPC / 2 words)
  __device__ __forceinline__ void words(int /*t*/, int j, int /*c*/, uint32_t* xw) const {
#pragma unroll
    for (int e = 0; e < EPC / 2; ++e) xw[e] = w[j * WPC + e];
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
  static constexpr int kXT = XT;
  const uint8_t* base;  // token t's row at base + t * stride
  size_t stride;
  // bf16 inputs as packed pairs (EPC / 2 words; EPC >= 8)
  __device__ __forceinline__ void words(int t, int /*j*/, int c, uint32_t* xw) const {
    const uint8_t* row = base + size_t(t) * stride;
#pragma unroll
    for (int q = 0; q < EPC / 8; ++q) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + size_t(c) * EPC * 2 + 16 * q);
      xw[4 * q + 0] = u.x;
      xw[4 * q + 1] = u.y;
      xw[4 * q + 2] = u.z;
      xw[4 * q + 3] = u.w;
    }
  }
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
  uint32_t sb[ROWS][CPL];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const uint4* p = reinterpret_cast<const uint4*>(w + size_t(n[r]) * rb);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = sl + LPR * j;
      const bool ok = v[r] && c < CPR;
      q[r][j] = ok ? ld_weight16(p + c) : make_uint4(0, 0, 0, 0);
      sb[r][j] = ok ? chunk_scale_bits<WD>(s, n[r], c, K) : 0u;
    }
  }
  // scale values only now (an invalid chunk has zero codes and a zero FP8 scale: adds nothing)
  float sc[ROWS][CPL];
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
#pragma unroll
    for (int j = 0; j < CPL; ++j) sc[r][j] = scale_of<WD>(sb[r][j]);
  constexpr bool kPacked = packed_dot<WD, In::kXT>();
  auto add = [&](float& a, float d, float scale) {
    if constexpr (WD == DT_FP8)
      a = fmaf(scale, d, a);
    else
      a += d;
  };
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = sl + LPR * j;
    if (c >= CPR) continue;
    if constexpr (NT == 1) {  // one input row: decode and consume row by row
      if constexpr (kPacked) {
        uint32_t xw[EPC / 2];
        x.words(0, j, c, xw);
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          uint32_t wp[EPC / 2];
          decode_pairs<WD>(q[r][j], sc[r][j], wp);
          add(acc[r][0], dot_pairs<EPC / 2>(wp, xw), sc[r][j]);
        }
      } else {
        float xv[EPC];
        x.chunk(0, j, c, xv);
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          float wv[EPC];
          decode<WD>(q[r][j], sc[r][j], wv);
          add(acc[r][0], dot_f32<EPC>(wv, xv), sc[r][j]);
        }
      }
    } else {  // several input rows: decode each weight chunk once, use it for every row
      if constexpr (kPacked) {
        uint32_t wp[ROWS][EPC / 2];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) decode_pairs<WD>(q[r][j], sc[r][j], wp[r]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t < nt) {
            uint32_t xw[EPC / 2];
            x.words(t, j, c, xw);
#pragma unroll
            for (int r = 0; r < ROWS; ++r) add(acc[r][t], dot_pairs<EPC / 2>(wp[r], xw), sc[r][j]);
          }
        }
      } else {
        float wv[ROWS][EPC];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) decode<WD>(q[r][j], sc[r][j], wv[r]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t < nt) {
            float xv[EPC];
            x.chunk(t, j, c, xv);
#pragma unroll
            for (int r = 0; r < ROWS; ++r) add(acc[r][t], dot_f32<EPC>(wv[r], xv), sc[r][j]);
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
// Fused decode layer: T <= kDecMaxT tokens, T*k <= kDecMaxR rows, two launches.
//
// decode_gate_up_kernel: every work-group selects the top-k of all T tokens itself (wave t takes
//   token t, from the logits) and maps the experts to slots; it owns one (gate, up) row pair per
//   lane group and computes a = silu(g) * u of those pairs for every resident slot's rows (stored
//   by row index r = t*k + j), NSL slots' weight loads in flight together.  The token rows (direct
//   LDS loads) and the slot map are loaded while the logits are, so the weights follow after one
//   round trip.  Work-group 0 also writes the routing outputs: top-k ids and gates, the slot of
//   each row (-1 when the row has none) for the second launch, the compact miss list (rows in
//   ascending r), the miss count and the error word.
// decode_down_combine_kernel: a work-group owns RB consecutive output columns for every row: it
//   loads all rows of a into LDS (direct LDS loads, in flight with the row slots, or with MXFP4
//   weights with the first slots' weights), computes y for each resident slot's rows, NSL slots'
//   weight loads in flight together, keeps y in LDS and sums out[t] = sum_j w[t,j] * y[t*k+j] over
//   the computed rows in ascending j.
//
// Every element is formed as on the GEMV path (same lanes per row and chunks per lane, so the
// same partial sums in the same order and the same segmented reduction; the same combine order),
// so a token's output is the same bits whichever flow computed it.
// ---------------------------------------------------------------------------------------------
// The decode layer's slots are dealt to kDecGroups groups of waves (work-groups of the gate/up
// launch, wave halves of a down + combine work-group), so each wave forms fewer slots' sums.
constexpr int kDecGroups = 2;
constexpr int kDecThreads2 = kThreads * kDecGroups;  // down + combine work-group

// the leaders (first rows of their slots) whose index among all leaders is g mod kDecGroups
__device__ __forceinline__ unsigned long long leaders_of_group(unsigned long long all, int g) {
  unsigned long long mine = 0;
  int idx = 0;
  for (unsigned long long m = all; m; m &= m - 1, ++idx)
    if (idx % kDecGroups == g) mine |= m & (~m + 1ull);
  return mine;
}

// gate/up of the decode layer: one (gate, up) row pair per lane group and work-group column
// block, NSL slots' weight loads in flight together
template <int LPR>
__host__ __device__ constexpr int dec_gu_pairs() { return kWaves * (64 / LPR); }
template <int CPL>
__host__ __device__ constexpr int dec_gu_slots() { return 16 / (2 * CPL) > 0 ? 16 / (2 * CPL) : 1; }

template <int WD, int XT, int LPR, int CPL, int VPL>
__global__ __launch_bounds__(kThreads) void decode_gate_up_kernel(const DecodeArgs d) {
  constexpr int EPC = WFmt<WD>::EPC;
  constexpr int GPW = 64 / LPR;
  constexpr int NSL = dec_gu_slots<CPL>();
  extern __shared__ __align__(16) uint8_t dl[];
  __shared__ int s_e[kDecMaxR];
  __shared__ float s_w[kDecMaxR];
  const int T = d.T, k = d.k, R = T * k, H = d.H, I = d.I, S = d.S, E = d.E;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const size_t xrow = size_t(H) * (XT == DT_F32 ? 4 : 2);
  const int ngx = T * int(xrow >> 4);                                  // 16-byte granules of the T token rows
  uint8_t* xl = dl;                                                    // [T][xrow]
  int32_t* smap = reinterpret_cast<int32_t*>(dl + size_t(T) * xrow);  // [E]
  const bool first = blockIdx.x == 0 && blockIdx.y == 0;
  const uint8_t* xg = static_cast<const uint8_t*>(d.x);

  // 1. loads that do not depend on the routing, in flight with the logits: the T token rows go
  //    straight into LDS (direct loads, 1 KB per wave instruction), the slot map into registers
  const uint32_t xbase = lds_addr(xl);
  for (int g = wid * 64; g < ngx; g += kThreads)
    if (g + lane < ngx) dma16(xg + size_t(g + lane) * 16, xbase + uint32_t(g) * 16);
  constexpr int kMapPre = (1024 + kThreads - 1) / kThreads;  // E <= 1024
  int mr[kMapPre];
  if (d.slot_map) {
#pragma unroll
    for (int u = 0; u < kMapPre; ++u) {
      const int i = tid + u * kThreads;
      mr[u] = i < E ? d.slot_map[i] : 0;
    }
  }
  // 2. token t's experts and gates in wave t
  if (wid < T) {
    int my_e;
    float my_w;
    topk_wave<VPL>(d.logits + size_t(wid) * E, d.bias, E, k, d.score, d.renorm, my_e, my_w);
    if (lane < k) {
      s_e[wid * k + lane] = my_e;
      s_w[wid * k + lane] = my_w;
      if (first) {
        d.topk_idx[wid * k + lane] = my_e;
        d.topk_w[wid * k + lane] = my_w;
      }
    }
  }
  if (d.slot_map) {
#pragma unroll
    for (int u = 0; u < kMapPre; ++u) {
      const int i = tid + u * kThreads;
      if (i < E) smap[i] = mr[u];
    }
  }
  wait_vmcnt<0>();  // the direct loads of the token rows
  __syncthreads();

  // 3. the slot of every row: key = slot, S for an absent expert, -1 for an out-of-range map
  //    entry, -2 on lanes past R (each wave derives the same from LDS)
  int key = -2, e = 0;
  if (lane < R) {
    e = s_e[lane];
    const int s = d.slot_map ? smap[e] : e;
    key = (s < -1 || s >= S) ? -1 : s < 0 ? S : s;
  }
  bool lead = key >= 0 && key < S;  // the first row of its slot
  for (int q = 0; q < R; ++q) {
    const int kq = __builtin_amdgcn_readlane(key, q);
    if (q < lane && kq == key) lead = false;
  }
  const unsigned long long leaders = __ballot(lead);
  if (first && wid == 0) {
    const unsigned long long miss = __ballot(key == S);
    const unsigned long long bad = __ballot(key == -1);
    if (lane < R) d.rkey[lane] = (key >= 0 && key < S) ? key : -1;
    if (key == S && d.miss_token) {
      const int m = __popcll(miss & ((1ull << lane) - 1ull));
      d.miss_token[m] = lane / k;
      d.miss_expert[m] = e;
      d.miss_weight[m] = s_w[lane];
    }
    if (lane == 0) {
      d.miss_count[0] = __popcll(miss);
      d.err[0] = bad ? 1u : 0u;
    }
  }
  // 4. gate/up: this lane group's pair (gate row i, up row I + i) for every resident slot's rows,
  //    each element as gate_up_kernel forms it
  const int CPR = H / EPC;
  const size_t rb = row_bytes<WD>(H);
  const int grp = lane / LPR, sl = lane - grp * LPR;
  const int i = blockIdx.x * dec_gu_pairs<LPR>() + wid * GPW + grp;
  const bool iv = i < I;
  const int nrow[2] = {iv ? i : 0, iv ? I + i : 0};
  unsigned long long rest = leaders_of_group(leaders, blockIdx.y);
  while (rest) {
    int sv[NSL];
    unsigned long long rm[NSL];
#pragma unroll
    for (int u = 0; u < NSL; ++u) {
      sv[u] = -1;
      rm[u] = 0;
      if (rest) {
        sv[u] = __builtin_amdgcn_readlane(key, __ffsll((long long)rest) - 1);
        rest &= rest - 1;
        rm[u] = __ballot(key == sv[u]);
      }
    }
    uint4 q[NSL][2][CPL];
    uint32_t sb[NSL][2][CPL];
#pragma unroll
    for (int u = 0; u < NSL; ++u) {
      const int su = sv[u] < 0 ? 0 : sv[u];
      const uint8_t* wslot = static_cast<const uint8_t*>(d.w_gu) + size_t(su) * 2 * I * rb;
      const void* sslot = nullptr;
      if constexpr (WD == DT_FP8)
        sslot = static_cast<const float*>(d.s_gu) + size_t(su) * ((2 * I + 127) >> 7) * ((H + 127) >> 7);
      if constexpr (WD == DT_MXFP4) sslot = static_cast<const uint8_t*>(d.s_gu) + size_t(su) * 2 * I * (H >> 5);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const uint4* p = reinterpret_cast<const uint4*>(wslot + size_t(nrow[r]) * rb);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const int c = sl + LPR * j;
          const bool ok = sv[u] >= 0 && iv && c < CPR;
          q[u][r][j] = ok ? ld_weight16(p + c) : make_uint4(0, 0, 0, 0);
          sb[u][r][j] = ok ? chunk_scale_bits<WD>(sslot, nrow[r], c, H) : 0u;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < NSL; ++u) {
      unsigned long long mm = rm[u];
      while (mm) {  // the slot's rows in passes of kDecMaxT
        int rr[kDecMaxT];
        int ntp = 0;
#pragma unroll
        for (int t = 0; t < kDecMaxT; ++t) {
          rr[t] = mm ? __ffsll((long long)mm) - 1 : 0;
          if (mm) {
            mm &= mm - 1;
            ++ntp;
          }
        }
        float acc[2][kDecMaxT];
#pragma unroll
        for (int t = 0; t < kDecMaxT; ++t) acc[0][t] = acc[1][t] = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const int c = sl + LPR * j;
          if (c >= CPR) continue;
#pragma unroll
          for (int r = 0; r < 2; ++r) {  // one weight row decoded at a time
            const float sc = scale_of<WD>(sb[u][r][j]);
            float dd[kDecMaxT];
            if constexpr (packed_dot<WD, XT>()) {
              uint32_t wp[EPC / 2];
              decode_pairs<WD>(q[u][r][j], sc, wp);
#pragma unroll
              for (int t = 0; t < kDecMaxT; ++t) {
                if (t < ntp) {
                  uint32_t xw[EPC / 2];
                  LdsIn<XT, EPC>{xl + size_t(rr[t] / k) * xrow, 0}.words(0, 0, c, xw);
                  dd[t] = dot_pairs<EPC / 2>(wp, xw);
                }
              }
            } else {
              float wv[EPC];
              decode<WD>(q[u][r][j], sc, wv);
#pragma unroll
              for (int t = 0; t < kDecMaxT; ++t) {
                if (t < ntp) {
                  float xv[EPC];
                  LdsIn<XT, EPC>{xl + size_t(rr[t] / k) * xrow, 0}.chunk(0, 0, c, xv);
                  dd[t] = dot_f32<EPC>(wv, xv);
                }
              }
            }
#pragma unroll
            for (int t = 0; t < kDecMaxT; ++t) {
              if (t < ntp) {
                if constexpr (WD == DT_FP8)
                  acc[r][t] = fmaf(sc, dd[t], acc[r][t]);
                else
                  acc[r][t] += dd[t];
              }
            }
          }
        }
#pragma unroll
        for (int t = 0; t < kDecMaxT; ++t) {
          if (t < ntp) {
            const float g = seg_sum<LPR>(acc[0][t]);
            const float uu = seg_sum<LPR>(acc[1][t]);
            if (sl == LPR - 1 && iv) d.a[size_t(rr[t]) * I + i] = silu(g) * uu;
          }
        }
      }
    }
  }
}

// output rows per lane group and slot in the down + combine launch; the work-group's columns
// RB = kWaves * (64 / LPR) * rows
template <int LPR, int CPL, int EPC>
__host__ __device__ constexpr int dec_rows() {
  return LPR == 64 ? (CPL >= 16 ? 1 : (CPL >= 8 || EPC >= 32) ? 2 : 4) : LPR == 32 ? 2 : 1;
}
template <int LPR, int CPL, int EPC>
__host__ __device__ constexpr int dec_cols() {
  return kWaves * (64 / LPR) * dec_rows<LPR, CPL, EPC>();
}

template <int WD, int LPR, int CPL, int ODT>
__global__ __launch_bounds__(kDecThreads2) void decode_down_combine_kernel(const DecodeArgs d) {
  constexpr int EPC = WFmt<WD>::EPC;
  constexpr int GPW = 64 / LPR;
  constexpr int ROWS = dec_rows<LPR, CPL, EPC>();
  constexpr int RB = dec_cols<LPR, CPL, EPC>();
  static_assert(RB <= kDecRB, "column block");
  constexpr int NSL = 8 / (ROWS * CPL) > 0 ? 8 / (ROWS * CPL) : 1;  // slots whose loads fly together
  extern __shared__ __align__(16) uint8_t dl[];
  __shared__ int s_key[kDecMaxR];
  __shared__ float s_w[kDecMaxR];
  const int T = d.T, k = d.k, R = T * k, H = d.H, I = d.I, S = d.S;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int grp = lane / LPR, sl = lane - grp * LPR;
  const size_t arow = size_t(I) * 4;
  const uint8_t* al = dl;                                           // [R][I] fp32 rows of a
  float* yl = reinterpret_cast<float*>(dl + size_t(R) * arow);      // [R][RB]
  const int h0 = blockIdx.x * RB;

  // every row of a (direct LDS loads, 1 KB per wave instruction)
  auto load_a = [&]() {
    const int ng = R * (I >> 2);
    const uint32_t abase = lds_addr(al);
    for (int c0 = wid * 64; c0 < ng; c0 += kDecThreads2)
      if (c0 + lane < ng) dma16(reinterpret_cast<const uint8_t*>(d.a) + size_t(c0 + lane) * 16, abase + uint32_t(c0) * 16);
  };
  // MXFP4 weights (small slot slices): the first slots' weight loads are issued before the rows of
  // a, which they do not depend on, so both fly together; bf16 and FP8 slices measured faster with
  // a first
  constexpr bool kEarlyW = WD == DT_MXFP4;
  if constexpr (!kEarlyW) load_a();

  // 1. the rows' slots and gates
  int key = -1;
  float gw = 0.0f;
  if (lane < R) {
    key = d.rkey[lane];
    gw = d.topk_w[lane];
  }
  if (key < 0 || key >= S) key = -1;
  if (wid == 0 && lane < R) {
    s_key[lane] = key;
    s_w[lane] = gw;
  }
  bool lead = key >= 0;  // the first row of its slot
  for (int q = 0; q < R; ++q) {
    const int kq = __builtin_amdgcn_readlane(key, q);
    if (q < lane && kq == key) lead = false;
  }
  // wave half g = wid / kWaves takes every kDecGroups-th slot; both halves cover the same columns
  unsigned long long rest = leaders_of_group(__ballot(lead), wid / kWaves);
  const int CPR = I / EPC;
  const size_t rb = row_bytes<WD>(I);
  const int hb = h0 + ((wid % kWaves) * GPW + grp) * ROWS;  // this lane group's first output row

  // 2. y of every resident slot's rows for this work-group's columns, NSL slots' weights in flight
  // at a time
  int sv[NSL];
  unsigned long long rm[NSL];
  uint4 q[NSL][ROWS][CPL];
  uint32_t sb[NSL][ROWS][CPL];
  auto load_batch = [&]() {
#pragma unroll
    for (int u = 0; u < NSL; ++u) {
      sv[u] = -1;
      rm[u] = 0;
      if (rest) {
        sv[u] = __builtin_amdgcn_readlane(key, __ffsll((long long)rest) - 1);
        rest &= rest - 1;
        rm[u] = __ballot(key == sv[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < NSL; ++u) {
      const int su = sv[u] < 0 ? 0 : sv[u];
      const uint8_t* wslot = static_cast<const uint8_t*>(d.w_d) + size_t(su) * H * rb;
      const void* sslot = nullptr;
      if constexpr (WD == DT_FP8)
        sslot = static_cast<const float*>(d.s_d) + size_t(su) * ((H + 127) >> 7) * ((I + 127) >> 7);
      if constexpr (WD == DT_MXFP4) sslot = static_cast<const uint8_t*>(d.s_d) + size_t(su) * H * (I >> 5);
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const int n = hb + r;
        const uint4* p = reinterpret_cast<const uint4*>(wslot + size_t(n < H ? n : 0) * rb);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const int c = sl + LPR * j;
          const bool ok = sv[u] >= 0 && n < H && c < CPR;
          q[u][r][j] = ok ? ld_weight16(p + c) : make_uint4(0, 0, 0, 0);
          sb[u][r][j] = ok ? chunk_scale_bits<WD>(sslot, n, c, I) : 0u;
        }
      }
    }
  };
  auto compute_batch = [&]() {
#pragma unroll
    for (int u = 0; u < NSL; ++u) {
      unsigned long long mm = rm[u];
      while (mm) {  // the slot's rows in passes of kDecMaxT
        int rr[kDecMaxT];
        int ntp = 0;
#pragma unroll
        for (int t = 0; t < kDecMaxT; ++t) {
          rr[t] = mm ? __ffsll((long long)mm) - 1 : 0;
          if (mm) {
            mm &= mm - 1;
            ++ntp;
          }
        }
        float acc[ROWS][kDecMaxT];
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
#pragma unroll
          for (int t = 0; t < kDecMaxT; ++t) acc[r][t] = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const int c = sl + LPR * j;
          if (c >= CPR) continue;
#pragma unroll
          for (int r = 0; r < ROWS; ++r) {  // one weight row decoded at a time
            float wv[EPC];
            const float sc = scale_of<WD>(sb[u][r][j]);
            decode<WD>(q[u][r][j], sc, wv);
#pragma unroll
            for (int t = 0; t < kDecMaxT; ++t) {
              if (t < ntp) {
                float xv[EPC];
                LdsIn<DT_F32, EPC>{al + size_t(rr[t]) * arow, 0}.chunk(0, 0, c, xv);
                const float dd = dot_f32<EPC>(wv, xv);
                if constexpr (WD == DT_FP8)
                  acc[r][t] = fmaf(sc, dd, acc[r][t]);
                else
                  acc[r][t] += dd;
              }
            }
          }
        }
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
#pragma unroll
          for (int t = 0; t < kDecMaxT; ++t) {
            if (t < ntp) {
              const float sum = seg_sum<LPR>(acc[r][t]);
              if (sl == LPR - 1 && hb + r < H) yl[rr[t] * RB + (hb - h0) + r] = sum;
            }
          }
      }
    }
  };
  if constexpr (kEarlyW) {
    load_batch();
    load_a();
  }
  wait_vmcnt<0>();
  __syncthreads();
  if constexpr (kEarlyW) compute_batch();
  while (rest) {
    load_batch();
    compute_batch();
  }
  __syncthreads();

  // 3. combine: out[t, h] = sum over the computed rows t*k+j, j ascending, of w * y
  for (int i = tid; i < T * RB; i += kDecThreads2) {
    const int t = i / RB, hl = i - t * RB, h = h0 + hl;
    if (h >= H) continue;
    float acc = 0.0f;
    for (int j0 = 0; j0 < k; j0 += 8) {  // eight choices' operands read before their sums
      int kk[8];
      float ww[8], yy[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = t * k + j0 + u;
        const bool in = j0 + u < k;
        kk[u] = in ? s_key[r] : -1;
        ww[u] = in ? s_w[r] : 0.0f;
        yy[u] = in ? yl[r * RB + hl] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (kk[u] >= 0) acc = fmaf(ww[u], yy[u], acc);
    }
    if constexpr (ODT == DT_F32)
      static_cast<float*>(d.out)[size_t(t) * H + h] = acc;
    else
      static_cast<uint16_t*>(d.out)[size_t(t) * H + h] = f32_to_bf16(acc);
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

// row steps per wave: enough work-groups to fill the chip when few slots are active, and more (up
// to the larger target) while each still streams floor_bytes of weights (timed together: decode
// bf16 T=4 gate/up 80.0 -> 75.7 us with one row step, while FP8 rows, half as long, and the down
// projection's short rows measured slower below the floors)
inline int pick_iters(int rows_total, int rows_per_block_step, int n_ord, size_t bytes_per_block_step,
                      size_t floor_bytes) {
  int iters = kIters;
  while (iters > 1) {
    const int blocks = (rows_total + rows_per_block_step * iters - 1) / (rows_per_block_step * iters);
    const long long grid = (long long)blocks * n_ord;
    if (grid >= MOE_GEMV_TARGET_BLOCKS_MAX) break;
    if (grid >= MOE_GEMV_TARGET_BLOCKS && bytes_per_block_step * size_t(iters / 2) < floor_bytes) break;
    iters >>= 1;
  }
  return iters;
}

template <int WD, int XT, int LPR, int CPL>
hipError_t launch_gate_up_t(const GemvArgs& g, hipStream_t st) {
  constexpr int ROWS = rows_per_step<CPL>();
  constexpr int PAIRS = ROWS / 2 > 0 ? ROWS / 2 : 1;
  const int step = kWaves * (64 / LPR) * PAIRS;
  const int iters = pick_iters(g.I, step, g.n_ord, size_t(step) * 2 * row_bytes<WD>(g.H), MOE_GEMV_WG_BYTES_GU);
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
  const int iters = pick_iters(g.H, step, g.n_ord, size_t(step) * row_bytes<WD>(g.I), MOE_GEMV_WG_BYTES_DN);
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

template <int WD, int XT, int LPR, int CPL>
hipError_t launch_decode_gate_up_t(const DecodeArgs& d, hipStream_t st) {
  constexpr int PB = dec_gu_pairs<LPR>();
  dim3 grid((d.I + PB - 1) / PB, kDecGroups), block(kThreads);
  const size_t lds = size_t(d.T) * d.H * (XT == DT_F32 ? 4 : 2) + size_t(d.E) * 4;
  // logits per lane of the top-k: the fewest that hold E (the selection does not depend on it)
  const void* kern = d.E <= 384 ? (const void*)decode_gate_up_kernel<WD, XT, LPR, CPL, 6>
                     : d.E <= 512 ? (const void*)decode_gate_up_kernel<WD, XT, LPR, CPL, 8>
                                  : (const void*)decode_gate_up_kernel<WD, XT, LPR, CPL, 16>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  if (d.E <= 384)
    decode_gate_up_kernel<WD, XT, LPR, CPL, 6><<<grid, block, lds, st>>>(d);
  else if (d.E <= 512)
    decode_gate_up_kernel<WD, XT, LPR, CPL, 8><<<grid, block, lds, st>>>(d);
  else
    decode_gate_up_kernel<WD, XT, LPR, CPL, 16><<<grid, block, lds, st>>>(d);
  return hipGetLastError();
}

template <int WD, int XT>
hipError_t decode_gate_up_dispatch(const DecodeArgs& d, hipStream_t st) {
  int lpr, cpl;
  pick_lpr_cpl(d.H / WFmt<WD>::EPC, lpr, cpl);  // as gate_up_dispatch: the same lanes per row
  if (lpr == 16) return launch_decode_gate_up_t<WD, XT, 16, 1>(d, st);
  if (lpr == 32) return launch_decode_gate_up_t<WD, XT, 32, 1>(d, st);
  switch (cpl) {
    case 1: return launch_decode_gate_up_t<WD, XT, 64, 1>(d, st);
    case 2: return launch_decode_gate_up_t<WD, XT, 64, 2>(d, st);
    case 4: return launch_decode_gate_up_t<WD, XT, 64, 4>(d, st);
    case 8: return launch_decode_gate_up_t<WD, XT, 64, 8>(d, st);
    default: return launch_decode_gate_up_t<WD, XT, 64, 16>(d, st);
  }
}

template <int WD, int LPR, int CPL>
hipError_t launch_decode_down_t(const DecodeArgs& d, hipStream_t st) {
  constexpr int RB = dec_cols<LPR, CPL, WFmt<WD>::EPC>();
  dim3 grid((d.H + RB - 1) / RB), block(kDecThreads2);
  const size_t R = size_t(d.T) * d.k;
  const size_t lds = R * d.I * 4 + R * RB * 4;
  const void* kern = d.odt == DT_F32 ? (const void*)decode_down_combine_kernel<WD, LPR, CPL, DT_F32>
                                     : (const void*)decode_down_combine_kernel<WD, LPR, CPL, DT_BF16>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  if (d.odt == DT_F32)
    decode_down_combine_kernel<WD, LPR, CPL, DT_F32><<<grid, block, lds, st>>>(d);
  else
    decode_down_combine_kernel<WD, LPR, CPL, DT_BF16><<<grid, block, lds, st>>>(d);
  return hipGetLastError();
}

template <int WD>
hipError_t decode_down_dispatch(const DecodeArgs& d, hipStream_t st) {
  int lpr, cpl;
  pick_lpr_cpl(d.I / WFmt<WD>::EPC, lpr, cpl);
  // the same lanes per row and chunks per lane as down_dispatch
  if (d.I / WFmt<WD>::EPC == 64) return launch_decode_down_t<WD, 16, 4>(d, st);
  if (lpr == 16) return launch_decode_down_t<WD, 16, 1>(d, st);
  if (lpr == 32) return launch_decode_down_t<WD, 32, 1>(d, st);
  switch (cpl) {
    case 1: return launch_decode_down_t<WD, 64, 1>(d, st);
    case 2: return launch_decode_down_t<WD, 64, 2>(d, st);
    case 4: return launch_decode_down_t<WD, 64, 4>(d, st);
    case 8: return launch_decode_down_t<WD, 64, 8>(d, st);
    default: return launch_decode_down_t<WD, 64, 16>(d, st);
  }
}

}  // namespace gemv
}  // namespace moe
