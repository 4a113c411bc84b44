// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// element formats (same values as the public moe_dtype)
enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_MXFP4 = 3 };

// ---------------------------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// E8M0 scale code -> fp32 value 2^(c-127) (c = 0 gives the subnormal 2^-127, 255 NaN)
__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
  c &= 0xFFu;
  return __uint_as_float(c == 0 ? 0x00400000u : c == 255 ? 0x7FC00000u : (c << 23));
}

// two OCP e4m3fn codes (bytes 0,1 or 2,3 of w) -> fp32 (gfx950 converts the OCP format)
__device__ __forceinline__ float2 fp8x2_lo(uint32_t w) {
  auto v = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  return make_float2(v[0], v[1]);
}
__device__ __forceinline__ float2 fp8x2_hi(uint32_t w) {
  auto v = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  return make_float2(v[0], v[1]);
}

// two e2m1 codes (byte `sel` of w; low nibble first) -> fp32, each multiplied by `scale`
template <int SEL>
__device__ __forceinline__ float2 fp4x2(uint32_t w, float scale) {
  auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, SEL);
  return make_float2(v[0], v[1]);
}

// 16-byte streaming load (non-temporal hint: weights are read once per call)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// ---------------------------------------------------------------------------------------------
// direct LDS loads
// ---------------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) const void lds_void;

// 16 bytes per lane from `src` into LDS at byte address lds + 16*lane (lds wave-uniform).
// Written as inline assembly so that the compiler's wait insertion does not treat it as aliasing
// every LDS read: the kernel orders these loads itself (explicit vmcnt waits and barriers), and no
// other vector memory load is in flight while they are.  The memory clobber keeps LDS reads from
// moving across it.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(m), "v"(src) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(uint32_t(size_t((lds_void*)p)));
}

// s_waitcnt vmcnt(n) lgkmcnt(0), expcnt unconstrained (gfx9 encoding).  lgkmcnt(0) makes this
// wave's LDS reads of earlier steps complete before the barrier that lets a stage be reloaded.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
// silu on the hardware exp2 and reciprocal (each about 1 ulp): z * 1 / (1 + 2^(-z log2 e)); the
// matrix-core epilogues round the result to bf16 (or quantise it), far coarser than the
// difference from silu() above.  Limits: z -> -inf gives -0 (2^+inf = inf, 1/inf = 0),
// z -> +inf gives z.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

// Mode B activation quantisation (OCP MX rule with E4M3 elements), shared by the quantisation
// kernel and the gate/up GEMM's epilogue so both give the same bits.
// Nearest-even E4M3 (e4m3fn) code of a finite y, saturating at +-448.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (!(a < 448.0f)) return sign | 0x7Eu;
  if (a == 0.0f) return sign;
  int e;
  (void)frexpf(a, &e);
  e -= 1;  // a in [2^e, 2^(e+1))
  if (e < -6) return sign | uint32_t(rintf(a * 512.0f));  // multiples of 2^-9 (8 -> 2^-6, code 0x08)
  int m = int(rintf(ldexpf(a, 3 - e)));                   // 8 .. 16
  if (m == 16) {
    m = 8;
    ++e;
  }
  const uint32_t code = (uint32_t(e + 7) << 3) | uint32_t(m - 8);
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

// Shared exponent X of a 32-element block with largest magnitude amax: floor(log2 amax) - 8
// (E4M3's largest exponent is 8), 0 for an all-zero block, kept within E8M0 (>= -127).
__device__ __forceinline__ int mx_e4m3_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int ex;
  (void)frexpf(amax, &ex);
  return max(ex - 9, -127);
}

// ---------------------------------------------------------------------------------------------
// wave-level reductions (64 lanes)
// ---------------------------------------------------------------------------------------------
template <int WIDTH = kWave>
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WIDTH);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---------------------------------------------------------------------------------------------
// DPP reductions (GFX9 row shifts and row broadcasts; all 64 lanes must be active)
// ---------------------------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_src(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_src_or(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}

// Segmented sum: the total of each LPR-lane group (LPR = 16, 32 or 64) lands in its last lane.
template <int LPR>
__device__ __forceinline__ float seg_sum(float v) {
  v += dpp_src<0x111>(v);  // row_shr:1
  v += dpp_src<0x112>(v);  // row_shr:2
  v += dpp_src<0x114>(v);  // row_shr:4
  v += dpp_src<0x118>(v);  // row_shr:8   -> lane 15 of each 16-lane row holds the row sum
  if constexpr (LPR >= 32) v += dpp_src<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  if constexpr (LPR >= 64) v += dpp_src<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Sum over the wave, returned to every lane.
__device__ __forceinline__ float wave_total(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(seg_sum<64>(v)), 63));
}

// Max over the wave, returned to every lane.
__device__ __forceinline__ float wave_max_all(float v) {
  const float NEG = -__builtin_huge_valf();
  auto step = [&](float o) { v = fmaxf(v, o); };
  step(__int_as_float(dpp_src_or<0x111>(__float_as_int(NEG), __float_as_int(v))));
  step(__int_as_float(dpp_src_or<0x112>(__float_as_int(NEG), __float_as_int(v))));
  step(__int_as_float(dpp_src_or<0x114>(__float_as_int(NEG), __float_as_int(v))));
  step(__int_as_float(dpp_src_or<0x118>(__float_as_int(NEG), __float_as_int(v))));
  step(__int_as_float(dpp_src_or<0x142, 0xA>(__float_as_int(NEG), __float_as_int(v))));
  step(__int_as_float(dpp_src_or<0x143, 0xC>(__float_as_int(NEG), __float_as_int(v))));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Unsigned 32-bit maximum over the wave, returned to every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, uint32_t(dpp_src_or<0x111>(0, int(v))));
  v = max(v, uint32_t(dpp_src_or<0x112>(0, int(v))));
  v = max(v, uint32_t(dpp_src_or<0x114>(0, int(v))));
  v = max(v, uint32_t(dpp_src_or<0x118>(0, int(v))));
  v = max(v, uint32_t(dpp_src_or<0x142, 0xA>(0, int(v))));
  v = max(v, uint32_t(dpp_src_or<0x143, 0xC>(0, int(v))));
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}

// Unsigned 64-bit maximum over the wave, returned to every lane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#define MOE_MAXU64_STEP(CTRL, RM)                                                        \
  {                                                                                      \
    const uint32_t oh = uint32_t(dpp_src_or<CTRL, RM>(0, int(uint32_t(v >> 32))));      \
    const uint32_t ol = uint32_t(dpp_src_or<CTRL, RM>(0, int(uint32_t(v))));             \
    const uint64_t o = (uint64_t(oh) << 32) | ol;                                        \
    v = o > v ? o : v;                                                                   \
  }
  MOE_MAXU64_STEP(0x111, 0xF)
  MOE_MAXU64_STEP(0x112, 0xF)
  MOE_MAXU64_STEP(0x114, 0xF)
  MOE_MAXU64_STEP(0x118, 0xF)
  MOE_MAXU64_STEP(0x142, 0xA)
  MOE_MAXU64_STEP(0x143, 0xC)
#undef MOE_MAXU64_STEP
  const uint32_t h = __builtin_amdgcn_readlane(int(uint32_t(v >> 32)), 63);
  const uint32_t l = __builtin_amdgcn_readlane(int(uint32_t(v)), 63);
  return (uint64_t(h) << 32) | l;
}


// ---------------------------------------------------------------------------------------------
// active-slot lookup: the ord-th slot with a non-empty row range in off[0..S]
// (block-cooperative; every thread of the block gets the same answer, -1 if none)
// ---------------------------------------------------------------------------------------------
template <int BLOCK>
__device__ int find_active_slot(const int32_t* __restrict__ off, int S, int ord, int* lds /*[BLOCK/64+1]*/) {
  constexpr int NW = BLOCK / kWave;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int before = 0;  // active slots in earlier chunks
  for (int base = 0; base < S; base += BLOCK) {
    int s = base + tid;
    bool act = false;
    if (s < S) act = off[s + 1] > off[s];
    unsigned long long m = __ballot(act);
    if (lane == 0) lds[wid] = __popcll(m);
    __syncthreads();
    int wbase = before;
    int total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      int c = lds[w];
      if (w < wid) wbase += c;
      total += c;
    }
    int rank = wbase + __popcll(m & ((1ull << lane) - 1ull));
    __syncthreads();
    if (act && rank == ord) lds[NW] = s;
    if (ord < before + total) {
      __syncthreads();
      int r = lds[NW];
      __syncthreads();
      return r;
    }
    before += total;
  }
  return -1;
}

}  // namespace moe
