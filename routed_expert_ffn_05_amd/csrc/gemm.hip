// Prefill path: grouped GEMMs on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16), mode A.
//
//   gate/up:  a[p, i] = silu(x_p . W_g[s,i,:]) * (x_p . W_u[s,i,:])  for the rows p of slot s
//   down:     y[p, h] = a_p . W_d[s,h,:]
//
// Tiles.  A work-group computes a BM x BN output tile of one slot with 4 waves side by side along
// N (32 columns each) and up to 4 MFMA row blocks of 32 rows; a tile whose slot has fewer rows
// skips the empty row blocks, so a slot of n rows costs ceil(n/32) row blocks of matrix work while
// its weights are streamed once per 128-row M-tile.  K advances in steps of BK = 64 through two
// LDS stages (global loads of step k+1 are in flight while step k runs on the matrix cores).
//   * activations (bf16) are gathered row by row through the permutation and copied to LDS;
//   * weights are decoded exactly into bf16 while being staged: e4m3fn values are bf16-exact,
//     e2m1 times a power-of-two E8M0 scale is bf16-exact (the conversion applies the scale);
//   * an FP8 128x128 block scale is constant over a wave's 32 columns and a 128-wide K block, so
//     each wave accumulates a K block in a temporary and adds scale * temporary to the result;
//   * gate/up: the N tile holds 64 gate rows then the 64 matching up rows; wave w reads its 32
//     MFMA columns as gate rows 16w..16w+15 followed by up rows 16w..16w+15, so each lane pair
//     (l, l+16) holds gate and up of the same (row, i) and SiLU(g)*u is formed in registers.
// Scheduling.  A one-work-group kernel lists the tiles in (slot, N tile, M tile) order; tile
// blocks are mapped XCD-major (block b runs on XCD b % 8), so the M tiles that share a weight tile
// run back to back on one XCD and find it in that XCD's L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace gemm {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kStride = BK + 8;  // bf16 per LDS row: 16-byte pad against bank conflicts

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int x = b & 7, j = b >> 3;
  int base = 0;
  for (int xx = 0; xx < x; ++xx) base += (n - xx + 7) >> 3;
  return base + j;
}

// 16 e4m3fn codes -> 16 bf16 (exact), written as two 16-byte words
__device__ __forceinline__ void fp8x16_to_bf16(const uint4 q, uint4& lo, uint4& hi) {
  const uint32_t u[4] = {q.x, q.y, q.z, q.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u[i], 1.0f, false);
    auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u[i], 1.0f, true);
    o[2 * i] = __builtin_bit_cast(uint32_t, a);
    o[2 * i + 1] = __builtin_bit_cast(uint32_t, b);
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// 32 e2m1 codes times `scale` (power of two) -> 32 bf16 (exact), four 16-byte words
__device__ __forceinline__ void fp4x32_to_bf16(const uint4 q, float scale, uint4 (&o)[4]) {
  const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u[i], scale, 0));
    const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u[i], scale, 1));
    const uint32_t c = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u[i], scale, 2));
    const uint32_t d = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u[i], scale, 3));
    o[i] = make_uint4(a, b, c, d);
  }
}

template <int WD>
__host__ __device__ constexpr size_t row_bytes(int K) {
  return WD == DT_BF16 ? size_t(K) * 2 : WD == DT_FP8 ? size_t(K) : size_t(K) / 2;
}

// ---------------------------------------------------------------------------------------------
// GATEUP = true:  A = x rows (through perm), B = W_gu[s] (gate/up interleaved), out a (bf16)
// GATEUP = false: A = a rows (positions),    B = W_d[s],                        out y (fp32)
// ---------------------------------------------------------------------------------------------
template <int WD, bool GATEUP, int XT = DT_BF16>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(
    const uint8_t* __restrict__ w, const void* __restrict__ wscale, const void* __restrict__ act,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ off, const int2* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, int T, int k, int K, int N, int I, void* __restrict__ out) {
  __shared__ __align__(16) uint16_t As[2][BM * kStride];
  __shared__ __align__(16) uint16_t Bs[2][BN * kStride];
  const int n_act = ntiles[0];
  if (int(blockIdx.x) >= n_act) return;
  const int2 ent = tiles[xcd_remap(blockIdx.x, n_act)];
  const int s = ent.x, nt = ent.y & 0xFF, mt = ent.y >> 8;
  const int cap = T * k;
  const int lo = min(max(off[s], 0), cap), hi = min(max(off[s + 1], lo), cap);
  const int m0 = lo + mt * BM;
  const int rows = min(BM, hi - m0);
  if (rows <= 0) return;
  const int nsub = (rows + 31) >> 5;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ln = lane & 31, kh = lane >> 5;
  // output columns of this tile: gate/up -> i in [n0, n0+64); down -> h in [n0, n0+128)
  const int n0 = GATEUP ? nt * (BN / 2) : nt * BN;
  const size_t rb = row_bytes<WD>(K);
  const uint8_t* wslot = w + size_t(s) * N * rb;

  // ---- global -> register assignments --------------------------------------------------------
  // A: 128 rows x 64 bf16 = 1024 16-byte granules, 4 per thread: row (tid>>3) + 32*i, granule tid&7
  // (fp32 activations are rounded to bf16, nearest even, as they are staged)
  const uint8_t* arow[4];
  bool aok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    aok[i] = r < rows;
    int src = 0;
    if (aok[i]) {
      if constexpr (GATEUP) {
        const int rr = perm[m0 + r];
        src = rr / k;
        aok[i] = rr >= 0 && src < T;
      } else {
        src = m0 + r;
      }
    }
    constexpr int XB = XT == DT_F32 ? 4 : 2;
    arow[i] = static_cast<const uint8_t*>(act) + (size_t(aok[i] ? src : 0) * K + (tid & 7) * 8) * XB;
  }
  // B rows of the tile in LDS order
  auto brow_global = [&](int r) -> int {
    if constexpr (GATEUP) return r < 64 ? n0 + r : I + n0 + (r - 64);
    return n0 + r;
  };
  // B granules per thread: bf16 4 (row (tid>>3)+32i, 8 elements), fp8 2 (row (tid>>2)+64i,
  // 16 elements), fp4 1 (row tid>>1, 32 elements)
  constexpr int NBG = WD == DT_BF16 ? 4 : WD == DT_FP8 ? 2 : 1;
  int brow[NBG], bcol[NBG];
  bool bok[NBG];
#pragma unroll
  for (int i = 0; i < NBG; ++i) {
    int r, c;
    if constexpr (WD == DT_BF16) {
      r = (tid >> 3) + 32 * i;
      c = (tid & 7) * 8;
    } else if constexpr (WD == DT_FP8) {
      r = (tid >> 2) + 64 * i;
      c = (tid & 3) * 16;
    } else {
      r = tid >> 1;
      c = (tid & 1) * 32;
    }
    const int g = brow_global(r);
    bok[i] = g < N;
    brow[i] = r;
    bcol[i] = c;
  }
  const uint8_t* bsrc[NBG];
#pragma unroll
  for (int i = 0; i < NBG; ++i) {
    const int g = bok[i] ? brow_global(brow[i]) : 0;
    bsrc[i] = wslot + size_t(g) * rb;
  }
  const uint8_t* s_fp4 = nullptr;  // MXFP4: this thread's row of E8M0 scales
  if constexpr (WD == DT_MXFP4)
    s_fp4 = static_cast<const uint8_t*>(wscale) + (size_t(s) * N + (bok[0] ? brow_global(brow[0]) : 0)) * (K >> 5);

  // one K step of operands in registers: A granules, B granules, and the per-step scales
  struct Stage {
    uint4 a[4];
    uint4 b[NBG];
    float bsc;  // MXFP4: E8M0 scale of this thread's B granule
  };
  const int bl = GATEUP ? (ln < 16 ? 16 * wv + ln : 64 + 16 * wv + (ln - 16)) : 32 * wv + ln;
  constexpr bool kBlockScaled = WD == DT_FP8;
  // FP8: the tile's B rows lie in at most three 128-row scale blocks (gate rows in one, up rows
  // in one or two; down rows in one).  Their K-block scales are staged in LDS once per tile;
  // lane column bl reads the row of its own weight row's block.
  __shared__ float Ssc[3][64];
  int srow = 0;
  if constexpr (kBlockScaled) {
    const int KB = (K + 127) >> 7;
    const int NBk = (N + 127) >> 7;
    int blk[3];
    blk[0] = brow_global(0) >> 7;
    blk[1] = GATEUP ? (brow_global(64) >> 7) : blk[0];
    blk[2] = GATEUP ? min(brow_global(127) >> 7, NBk - 1) : blk[0];
    const float* sbase = static_cast<const float*>(wscale) + size_t(s) * NBk * KB;
    for (int t = tid; t < 3 * KB; t += kThreads) {
      const int r = t / KB, kb = t - r * KB;
      Ssc[r][kb] = sbase[size_t(min(blk[r], NBk - 1)) * KB + kb];
    }
    const int gb = min(brow_global(bl), N - 1) >> 7;
    srow = gb == blk[0] ? 0 : gb == blk[1] ? 1 : 2;
  }
  // Loads are unconditional (rows outside the tile read a valid row and are zeroed or ignored
  // later) so that the number of loads in flight is static and the waits stay precise.
  auto load = [&](int kk, Stage& st) {
    const int k0 = kk * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (XT == DT_F32) {
        const float4 f0 = reinterpret_cast<const float4*>(arow[i] + size_t(k0) * 4)[0];
        const float4 f1 = reinterpret_cast<const float4*>(arow[i] + size_t(k0) * 4)[1];
        uint4 v;
        v.x = uint32_t(f32_to_bf16(f0.x)) | (uint32_t(f32_to_bf16(f0.y)) << 16);
        v.y = uint32_t(f32_to_bf16(f0.z)) | (uint32_t(f32_to_bf16(f0.w)) << 16);
        v.z = uint32_t(f32_to_bf16(f1.x)) | (uint32_t(f32_to_bf16(f1.y)) << 16);
        v.w = uint32_t(f32_to_bf16(f1.z)) | (uint32_t(f32_to_bf16(f1.w)) << 16);
        st.a[i] = v;
      } else {
        st.a[i] = *reinterpret_cast<const uint4*>(arow[i] + size_t(k0) * 2);
      }
    }
#pragma unroll
    for (int i = 0; i < NBG; ++i) {
      const size_t byte = WD == DT_BF16 ? size_t(k0 + bcol[i]) * 2 : WD == DT_FP8 ? size_t(k0 + bcol[i]) : size_t(k0 + bcol[i]) / 2;
      st.b[i] = ld_stream16(bsrc[i] + byte);
    }
    if constexpr (WD == DT_MXFP4) st.bsc = e8m0_to_f32(s_fp4[(k0 + bcol[0]) >> 5]);
  };
  auto store = [&](int buf, const Stage& st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t m = aok[i] ? 0xFFFFFFFFu : 0u;
      *reinterpret_cast<uint4*>(&As[buf][((tid >> 3) + 32 * i) * kStride + (tid & 7) * 8]) =
          make_uint4(st.a[i].x & m, st.a[i].y & m, st.a[i].z & m, st.a[i].w & m);
    }
#pragma unroll
    for (int i = 0; i < NBG; ++i) {
      uint16_t* dst = &Bs[buf][brow[i] * kStride + bcol[i]];
      if constexpr (WD == DT_BF16) {
        *reinterpret_cast<uint4*>(dst) = st.b[i];
      } else if constexpr (WD == DT_FP8) {
        uint4 a, b;
        fp8x16_to_bf16(st.b[i], a, b);
        reinterpret_cast<uint4*>(dst)[0] = a;
        reinterpret_cast<uint4*>(dst)[1] = b;
      } else {
        uint4 o[4];
        fp4x32_to_bf16(st.b[i], st.bsc, o);
#pragma unroll
        for (int q = 0; q < 4; ++q) reinterpret_cast<uint4*>(dst)[q] = o[q];
      }
    }
  };

  const int nk_total = K / BK;
  // The K loop for NS = ceil(rows / 32) row blocks (a compile-time count: straight-line MFMAs).
  // Operands of step k+2 are loaded while step k runs; step k+1 is written to the other LDS
  // stage after step k's MFMAs.
  auto run = [&](auto ns_c) {
    constexpr int NS = decltype(ns_c)::value;
    f32x16_t acc[NS], tmp[NS];
#pragma unroll
    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ms][r] = tmp[ms][r] = 0.0f;
    auto compute = [&](int buf) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const bf16x8_t bfrag = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][bl * kStride + ks * 16 + kh * 8]);
        bf16x8_t afrag[NS];
#pragma unroll
        for (int ms = 0; ms < NS; ++ms)
          afrag[ms] = *reinterpret_cast<const bf16x8_t*>(&As[buf][(ms * 32 + ln) * kStride + ks * 16 + kh * 8]);
#pragma unroll
        for (int ms = 0; ms < NS; ++ms) {
          if constexpr (kBlockScaled)
            tmp[ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[ms], bfrag, tmp[ms], 0, 0, 0);
          else
            acc[ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[ms], bfrag, acc[ms], 0, 0, 0);
        }
      }
    };
    // end of a 128-wide K block (or of K): fold the block's partial sums in with their scale
    auto fold = [&](int kk) {
      if constexpr (kBlockScaled) {
        if (((kk + 1) * BK) % 128 == 0 || kk + 1 == nk_total) {
          const float sc = Ssc[srow][(kk * BK) >> 7];
#pragma unroll
          for (int ms = 0; ms < NS; ++ms)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              acc[ms][r] = fmaf(sc, tmp[ms][r], acc[ms][r]);
              tmp[ms][r] = 0.0f;
            }
        }
      }
    };
    const int nk = nk_total;
    Stage s0, s1;
    // prefetches past the last step reload the last step (and are ignored): the number of
    // loads in flight is the same on every path, which keeps the compiler's waits exact
    load(0, s0);
    load(min(1, nk - 1), s1);
    store(0, s0);
    __syncthreads();
    for (int kk = 0; kk < nk; kk += 2) {
      // step kk from LDS stage 0; s1 holds step kk+1
      load(min(kk + 2, nk - 1), s0);
      compute(0);
      fold(kk);
      if (kk + 1 < nk) store(1, s1);
      __syncthreads();
      if (kk + 1 >= nk) break;
      // step kk+1 from LDS stage 1; s0 holds step kk+2
      load(min(kk + 3, nk - 1), s1);
      compute(1);
      fold(kk + 1);
      if (kk + 2 < nk) store(0, s0);
      __syncthreads();
    }

    // ---- epilogue: accumulator r of lane l is row 8*(r/4) + 4*(l/32) + r%4 of its row block,
    // column l%32
#pragma unroll
    for (int ms = 0; ms < NS; ++ms) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = ms * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        const float v = acc[ms][r];
        if constexpr (GATEUP) {
          const float o = __shfl_xor(v, 16);
          if (ln < 16 && m < rows) {
            const int i = n0 + 16 * wv + ln;
            if (i < I) static_cast<uint16_t*>(out)[size_t(m0 + m) * I + i] = f32_to_bf16(silu(v) * o);
          }
        } else {
          const int h = n0 + 32 * wv + ln;
          if (m < rows && h < N) static_cast<float*>(out)[size_t(m0 + m) * N + h] = v;
        }
      }
    }
  };
  switch (nsub) {
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 3: run(std::integral_constant<int, 3>{}); break;
    default: run(std::integral_constant<int, 4>{}); break;
  }
}

// ---------------------------------------------------------------------------------------------
// tile scheduler: M tiles per slot, exclusive scan, then one entry per (slot, N tile, M tile)
// for both GEMMs.  Entry = {slot, (m_tile << 8) | n_tile}.
// ---------------------------------------------------------------------------------------------
constexpr int kSchedThreads = 1024;

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const int32_t* __restrict__ off, int S,
                                                                 int cap, int nt_gu, int nt_dn, int max_gu,
                                                                 int max_dn, int2* __restrict__ tiles_gu,
                                                                 int2* __restrict__ tiles_dn,
                                                                 int32_t* __restrict__ counts) {
  extern __shared__ int32_t mbase[];  // [S + 1]
  __shared__ int32_t wsum[kSchedThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int per = (S + kSchedThreads - 1) / kSchedThreads;
  const int a = tid * per, b = min(S, a + per);
  int local = 0;
  for (int s = a; s < b; ++s) {
    const int lo = min(max(off[s], 0), cap), hi = min(max(off[s + 1], lo), cap);
    const int mt = (hi - lo + BM - 1) / BM;
    mbase[s] = mt;
    local += mt;
  }
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  int run = incl - local;
  for (int w = 0; w < wid; ++w) run += wsum[w];
  for (int s = a; s < b; ++s) {
    const int c = mbase[s];
    mbase[s] = run;
    run += c;
  }
  __syncthreads();
  int MT = 0;
  for (int w = 0; w < kSchedThreads / 64; ++w) MT += wsum[w];
  if (tid == 0) mbase[S] = MT;
  __syncthreads();
  // entries: tile L of a GEMM with NT column tiles belongs to the last slot s with
  // mbase[s] * NT <= L; within the slot, L - mbase[s]*NT = n_tile * mt_s + m_tile
  for (int g = 0; g < 2; ++g) {
    const int NT = g ? nt_dn : nt_gu;
    int2* tl = g ? tiles_dn : tiles_gu;
    // the host sized the lists for consistent offsets (sum of rows <= T*k); never write past them
    const int total = min(MT * NT, g ? max_dn : max_gu);
    for (int L = tid; L < total; L += kSchedThreads) {
      const int q = L / NT;
      int lo = 0, hi = S - 1;  // last s in [0, S) with mbase[s] <= q
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (mbase[mid] <= q) lo = mid;
        else hi = mid - 1;
      }
      const int s = lo;
      const int mt = mbase[s + 1] - mbase[s];
      const int local2 = L - mbase[s] * NT;
      const int n = local2 / mt, m = local2 - n * mt;
      tl[L] = make_int2(s, (m << 8) | n);
    }
  }
  if (tid == 0) {
    counts[0] = min(MT * nt_gu, max_gu);
    counts[1] = min(MT * nt_dn, max_dn);
  }
}

}  // namespace gemm

size_t gemm_tiles_max(int T, int k, int S, int nt) {
  const long long R = (long long)T * k;
  const long long mt = R / gemm::BM + (R < S ? R : S);
  return size_t(mt) * nt;
}

int gemm_nt_gate_up(int I) { return (I + gemm::BN / 2 - 1) / (gemm::BN / 2); }
int gemm_nt_down(int H) { return (H + gemm::BN - 1) / gemm::BN; }

hipError_t launch_gemm_schedule(const GemmArgs& g, hipStream_t st) {
  const size_t lds = sizeof(int32_t) * size_t(g.S + 1);
  const int ngu = gemm_nt_gate_up(g.I), ndn = gemm_nt_down(g.H);
  gemm::schedule_kernel<<<1, gemm::kSchedThreads, lds, st>>>(
      g.off, g.S, g.T * g.k, ngu, ndn, int(gemm_tiles_max(g.T, g.k, g.S, ngu)), int(gemm_tiles_max(g.T, g.k, g.S, ndn)),
      g.tiles_gu, g.tiles_dn, g.counts);
  return hipGetLastError();
}

template <int WD>
static hipError_t gate_up_t(const GemmArgs& g, hipStream_t st) {
  const size_t grid = gemm_tiles_max(g.T, g.k, g.S, gemm_nt_gate_up(g.I));
  if (grid == 0) return hipSuccess;
  if (g.xdt == DT_F32)
    gemm::gemm_kernel<WD, true, DT_F32><<<dim3(unsigned(grid)), dim3(gemm::kThreads), 0, st>>>(
        static_cast<const uint8_t*>(g.w_gu), g.s_gu, g.x, g.perm, g.off, g.tiles_gu, g.counts, g.T, g.k, g.H,
        2 * g.I, g.I, g.a);
  else
    gemm::gemm_kernel<WD, true, DT_BF16><<<dim3(unsigned(grid)), dim3(gemm::kThreads), 0, st>>>(
        static_cast<const uint8_t*>(g.w_gu), g.s_gu, g.x, g.perm, g.off, g.tiles_gu, g.counts, g.T, g.k, g.H,
        2 * g.I, g.I, g.a);
  return hipGetLastError();
}

template <int WD>
static hipError_t down_t(const GemmArgs& g, hipStream_t st) {
  const size_t grid = gemm_tiles_max(g.T, g.k, g.S, gemm_nt_down(g.H));
  if (grid == 0) return hipSuccess;
  gemm::gemm_kernel<WD, false><<<dim3(unsigned(grid)), dim3(gemm::kThreads), 0, st>>>(
      static_cast<const uint8_t*>(g.w_d), g.s_d, g.a, nullptr, g.off, g.tiles_dn,
      g.counts + 1, g.T, g.k, g.I, g.H, g.I, g.y);
  return hipGetLastError();
}

hipError_t launch_gemm_gate_up(const GemmArgs& g, hipStream_t st) {
  switch (g.wdt) {
    case DT_BF16: return gate_up_t<DT_BF16>(g, st);
    case DT_FP8: return gate_up_t<DT_FP8>(g, st);
    case DT_MXFP4: return gate_up_t<DT_MXFP4>(g, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_down(const GemmArgs& g, hipStream_t st) {
  switch (g.wdt) {
    case DT_BF16: return down_t<DT_BF16>(g, st);
    case DT_FP8: return down_t<DT_FP8>(g, st);
    case DT_MXFP4: return down_t<DT_MXFP4>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
