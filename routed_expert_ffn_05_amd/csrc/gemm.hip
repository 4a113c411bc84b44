// Prefill path: grouped GEMMs on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16), mode A.
//
//   gate/up:  a[p, i] = silu(x_p . W_g[s,i,:]) * (x_p . W_u[s,i,:])  for the rows p of slot s
//   down:     y[p, h] = a_p . W_d[s,h,:]
//
// Tiles.  A work-group (8 waves) computes a BM x BN output tile of one slot.  A tile whose slot
// has fewer than 128 rows runs only ceil(rows/32) MFMA row blocks of 32 rows (each wave: 32 of the
// BN = 256 columns, all row blocks), so a slot of n rows costs that much matrix work while its
// weights are streamed once per 128-row M tile; a full tile of bf16 or FP8 weights runs on a 2 x 4
// grid of waves of 64 x 64 (2 x 2 MFMA blocks, so each LDS fragment feeds two instructions).  The wide N tile halves how often each activation
// row is moved from L2 into LDS (the on-chip traffic that bounds these GEMMs).
// Staging.  Operand tiles of each K step (BK = 128 for FP8 and MXFP4 weights, 64 for bf16: a
// weight row segment per step is a whole 128-byte line where LDS allows) move from HBM to LDS by
// direct LDS loads (global_load_lds_dwordx4: each lane's 16 bytes land at LDS base + 16*lane)
// with no register staging; one explicit vmcnt wait and one barrier per step, the loads of a step
// spread over its MFMA sub-steps.  One work-group per CU owns most of the LDS: a stage holds the
// A rows the tile uses plus the B tile, and tiles with fewer row blocks keep more K steps in
// flight (2 for a full FP8 tile, up to 8).
// Within a row, the 16-byte granule g of row r is stored at slot g ^ f(r) (f spreads consecutive
// rows over distinct bank groups for the MFMA fragment reads).  Weights stay in their stored
// format in LDS and are decoded when a B fragment is read: e4m3fn -> bf16 is exact; e2m1 times a
// power-of-two E8M0 scale -> bf16 is exact (the conversion applies the scale).
// FP8 block scales.  A 128x128 block scale is constant over a lane's column and a 128-wide K
// block: each lane accumulates a K block in a temporary and adds scale * temporary to the result.
// Gate/up fusion.  The N tile holds 128 gate rows then the 128 matching up rows; wave w reads its
// 32 MFMA columns as gate rows 16w..16w+15 followed by up rows 16w..16w+15, so lanes l and l+16
// hold gate and up of the same (row, i) and SiLU(g)*u is formed in registers, then staged in LDS
// to leave in whole 16-byte pieces (mode B: quantised to E4M3 + E8M0 on the way out).
// Down: y is written with non-temporal stores (read once, by the combine).
// Scheduling.  A one-work-group kernel deals the tiles to the eight XCDs (block b runs on XCD
// b % 8) in units of up to four M tiles of one slot with all their N tiles, so the tiles
// co-resident on one XCD are the N tiles of a few M tiles of one slot: each activation slice is
// read from L2 by all N tiles, each weight slice by the M tiles in flight.  Units go out largest
// first and serpentine over the XCDs, which evens out their work on skewed routing (see
// schedule_kernel).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace gemm {

constexpr int BM = 128, BN = 256;
constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kMaxFp4Kb = 128;  // MXFP4: E8M0 scales per row staged in LDS (K <= 4096)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// K step, operand bytes per row and step, direct loads per wave and step, LDS for the stages.
// The K step makes every weight row segment a whole 128-byte line where LDS allows (bf16: 64,
// FP8: 128 elements; MXFP4: 128 elements = 64 bytes), since each direct load of a line segment
// occupies one of the CU's outstanding-request slots whatever its length.
template <int WD> struct BFmt {
  static constexpr int BK = WD == DT_BF16 ? 64 : 128;
  static constexpr int ROW = WD == DT_BF16 ? 128 : WD == DT_FP8 ? 128 : 64;  // B bytes per row
  static constexpr int AROW = BK * 2;                                         // A (bf16) bytes per row
  static constexpr int STAGE = BN * ROW;
  static constexpr int INSTR = STAGE / (1024 * kWaves);
  static constexpr int KS = BK / 16;  // MFMA sub-steps per step
  // the MXFP4 tile keeps its E8M0 scales (BN x K/32 bytes) in LDS beside the stages
  static constexpr int BUDGET = WD == DT_MXFP4 ? 112 * 1024 : 144 * 1024;
  // a K step of a tile with NS row blocks occupies 32*NS A rows plus the B tile; as many steps
  // are kept in flight as the budget holds (at most 8)
  static constexpr int stage_bytes(int ns) { return ns * 32 * AROW + STAGE; }
  static constexpr int nstage(int ns) { return BUDGET / stage_bytes(ns) < 8 ? BUDGET / stage_bytes(ns) : 8; }
};


// swizzled position of 16-byte granule g in row r of a 256-byte tile row (16 granules)
__device__ __forceinline__ int swz256(int r, int g) { return g ^ (r & 15); }
// 128-byte rows
__device__ __forceinline__ int swz128(int r, int g) { return g ^ ((r >> 1) & 7); }
// 64-byte rows (fp8)
__device__ __forceinline__ int swz64(int r, int g) { return g ^ ((r >> 2) & 3); }
// 32-byte rows (fp4)
__device__ __forceinline__ int swz32(int r, int g) { return g ^ ((r >> 3) & 1); }


template <int WD>
__host__ __device__ constexpr size_t row_bytes(int K) {
  return WD == DT_BF16 ? size_t(K) * 2 : WD == DT_FP8 ? size_t(K) : size_t(K) / 2;
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Down epilogue: the tile's y (rows x 256 columns, fp32; accumulator r of lane l is row
// 8*(r/4) + 4*(l/32) + r%4 of its row block, column l%32 of its column block) leaves through LDS
// in 16-byte pieces, 64 rows at a time (row stride 264 floats: the two lane halves, 4 rows apart,
// write disjoint bank halves).  acc[i][c] is row block i, column block c of the wave: with the
// 2 x 4 wave grid (TD) wave w holds rows 64(w/4) + 32i.., columns 64(w%4) + 32c..; otherwise
// rows 32i.., columns 32w...  y is read once, by the combine, long after: the stores are
// non-temporal.  Needs N % 4 == 0 and 64 * 264 * 4 bytes of `lds`; every wave's stage reads and
// direct loads must be done (the caller waited for its loads).  acc(i, c, r) reads register r of
// accumulator block (i, c).
template <int NR, int NC, bool TD, typename Acc>
__device__ __forceinline__ void store_y_tile(Acc acc, uint8_t* lds, float* __restrict__ y, int m0, int rows,
                                             int n0, int N, int halves) {
  constexpr int YS = 264;
  float* yt = reinterpret_cast<float*>(lds);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, ln = lane & 31, kh = lane >> 5;
  for (int half = 0; half < halves; ++half) {
    __syncthreads();  // the stages (first half) or the previous half's rows are no longer read
    if constexpr (TD) {
      if ((wv >> 2) == half) {
#pragma unroll
        for (int i = 0; i < NR; ++i)
#pragma unroll
          for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              yt[(i * 32 + 8 * (r >> 2) + 4 * kh + (r & 3)) * YS + 64 * (wv & 3) + 32 * c + ln] = acc(i, c, r);
      }
    } else {
#pragma unroll
      for (int mh = 0; mh < 2; ++mh) {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          if (i == 2 * half + mh) {
#pragma unroll
            for (int r = 0; r < 16; ++r) yt[(mh * 32 + 8 * (r >> 2) + 4 * kh + (r & 3)) * YS + 32 * wv + ln] = acc(i, 0, r);
          }
        }
      }
    }
    __syncthreads();
    const int rh = min(64, rows - 64 * half);  // rows of this half
    for (int t = tid; t < rh * 64; t += kThreads) {
      const int m = t >> 6, h = n0 + (t & 63) * 4;
      if (h < N) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(yt + m * YS + (t & 63) * 4);
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(y + size_t(m0 + 64 * half + m) * N + h));
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// GATEUP = true:  A = x rows (through perm), B = W_gu[s] (gate/up interleaved), out a (bf16)
// GATEUP = false: A = a rows (positions),    B = W_d[s],                        out y (fp32)
// ---------------------------------------------------------------------------------------------
template <int WD, bool GATEUP>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(
    const uint8_t* __restrict__ w, const void* __restrict__ wscale, const uint16_t* __restrict__ act,
    const int32_t* __restrict__ perm, const int4* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, int S, int T, int k, int K, int N, int I, int asplit,
    void* __restrict__ out) {
  using F = BFmt<WD>;
  __shared__ __align__(16) uint8_t smem[F::BUDGET];
  __shared__ float Ssc[4][64];                                    // FP8 block scales
  __shared__ __align__(16) uint8_t Sfp4[WD == DT_MXFP4 ? BN * kMaxFp4Kb : 16];  // MXFP4 scales
  __shared__ uint8_t rowok[BM];
  // tile j = b / 8 of XCD x = b % 8 (the scheduler's per-XCD lists of gridDim.x / 8 entries); the
  // count and the entry are loaded together (the entry slot exists for every block), and the entry
  // carries the tile's first row and row count, so no further index load precedes the operands
  const int xcd = blockIdx.x & 7, jt = blockIdx.x >> 3;
  const int ncnt = ntiles[xcd];
  const int4 ent = tiles[size_t(xcd) * (gridDim.x >> 3) + jt];
  if (jt >= ncnt) return;
  const int s = ent.x, m0 = ent.y, rows = ent.z, nt = ent.w;
  const int cap = T * k;
  // never taken for the scheduler's entries
  if (unsigned(s) >= unsigned(S) || rows <= 0 || rows > BM || m0 < 0 || m0 + rows > cap) return;
  const int nsub = (rows + 31) >> 5;
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, kh = lane >> 5;
  // output columns of this tile: gate/up -> i in [n0, n0+128); down -> h in [n0, n0+256)
  const int n0 = GATEUP ? nt * (BN / 2) : nt * BN;
  const size_t rb = row_bytes<WD>(K);
  const uint8_t* wslot = w + size_t(s) * N * rb;
  auto brow_global = [&](int r) -> int {
    if constexpr (GATEUP) return r < BN / 2 ? n0 + r : I + n0 + (r - BN / 2);
    return n0 + r;
  };
  // rows past N read the last row (valid memory; their columns are never stored)
  auto brow_clamped = [&](int r) -> int { return min(brow_global(r), N - 1); };

  constexpr int BK = F::BK;
  // swizzled slot of A granule g in tile row r
  auto swzA = [](int r, int g) -> int {
    if constexpr (F::AROW == 256) return swz256(r, g);
    return swz128(r, g);
  };
  constexpr int AGR = F::AROW / 16;     // A granules per row
  constexpr int ARPC = 1024 / F::AROW;  // A rows per 1 KiB chunk

  // ---- per-lane sources of the direct loads ---------------------------------------------------
  // A (set up per row-block count in run()): with NS row blocks the tile's first 32*NS rows are
  // loaded as 1 KiB chunks of ARPC rows; chunk c is issued by wave c % 8, lane -> row
  // ARPC*c + lane/AGR, slot lane%AGR.  Rows past the tile read a valid row and are never stored.
  auto a_source = [&](int r) -> const uint8_t* {
    int src = GATEUP ? 0 : m0;
    if (r < rows) {
      if constexpr (GATEUP) {
        const int rr = perm[m0 + r];
        src = (rr >= 0 && rr / k < T) ? rr / k : 0;
      } else {
        src = m0 + r;
      }
    }
    // down with a split a: a row holds the hi halves of its I values, then the lo halves
    return reinterpret_cast<const uint8_t*>(act + size_t(src) * K * (GATEUP ? 1 : asplit)) + swzA(r, lane % AGR) * 16;
  };
  // B: chunk c = INSTR*w + j covers 1 KiB of the tile: 128-byte rows, lane -> row 8c + lane/8
  // (bf16, FP8); 64-byte rows: lane -> row 16c + lane/4 (MXFP4)
  const uint8_t* bsrc[F::INSTR];
#pragma unroll
  for (int j = 0; j < F::INSTR; ++j) {
    const int c = F::INSTR * wv + j;
    int r, g;
    if constexpr (F::ROW == 128) {
      r = 8 * c + (lane >> 3);
      g = swz128(r, lane & 7);
    } else {
      r = 16 * c + (lane >> 2);
      g = swz64(r, lane & 3);
    }
    bsrc[j] = wslot + size_t(brow_clamped(r)) * rb + g * 16;
  }

  // ---- per-tile side data in LDS: row validity, FP8 block scales, MXFP4 scales ------------------
  if (tid < BM) {
    bool ok = tid < rows;
    if constexpr (GATEUP) {
      if (ok) {
        const int rr = perm[m0 + tid];
        ok = rr >= 0 && rr / k < T;
      }
    }
    rowok[tid] = ok;
  }
  constexpr bool kBlockScaled = WD == DT_FP8;
  // the tile's B rows lie in at most four 128-row scale blocks: those of tile rows 0, 127, 128
  // and 255 (gate/up: the gate rows start on a block boundary, the up rows may straddle one);
  // srow_of(c) is the one of tile row c
  int blk[4] = {0, 0, 0, 0};
  auto srow_of = [&](int c) -> int {
    const int gb = brow_clamped(c) >> 7;
    return gb == blk[0] ? 0 : gb == blk[1] ? 1 : gb == blk[2] ? 2 : 3;
  };
  if constexpr (kBlockScaled) {
    const int KB = (K + 127) >> 7;
    const int NBk = (N + 127) >> 7;
    blk[0] = brow_clamped(0) >> 7;
    blk[1] = brow_clamped(127) >> 7;
    blk[2] = brow_clamped(128) >> 7;
    blk[3] = brow_clamped(255) >> 7;
    const float* sbase = static_cast<const float*>(wscale) + size_t(s) * NBk * KB;
    for (int t = tid; t < 4 * KB; t += kThreads) {
      const int r = t / KB, kb = t - r * KB;
      Ssc[r][kb] = sbase[size_t(blk[r]) * KB + kb];
    }
  }
  // MXFP4: E8M0 scales of the tile's rows over all of K, [row][K/32] in LDS (K/32 is even).
  // With K % 512 == 0 a row is gpr whole 16-byte granules, stored rotated by a per-row key so that
  // the rows read together by one instruction fall in different LDS banks (granule q of row r at
  // slot (q + key(r)) % gpr); they arrive by direct loads issued with the first stages.  Otherwise
  // the work-group copies them unrotated before the main loop.
  const int KB32 = K >> 5;
  const uint8_t* fp4_src = WD == DT_MXFP4 ? static_cast<const uint8_t*>(wscale) + size_t(s) * N * KB32 : nullptr;
  const bool fp4_async = WD == DT_MXFP4 && KB32 % 16 == 0;
  const int gpr = fp4_async ? KB32 >> 4 : 1;
  // rows r and r + D start in the same bank: D = 64 dwords over the row's dwords, made coprime
  const int fp4_d = fp4_async ? 16 / ((gpr & -gpr) < 16 ? (gpr & -gpr) : 16) : 1;
  auto fp4_key = [&](int r) -> int { return fp4_async ? (r / fp4_d) % gpr : 0; };
  if constexpr (WD == DT_MXFP4) {
    if (!fp4_async) {
      const int per_row = KB32 >> 1;
      for (int t = tid; t < BN * per_row; t += kThreads) {
        const int r = t / per_row, q = t - r * per_row;
        reinterpret_cast<uint16_t*>(Sfp4 + r * KB32)[q] = reinterpret_cast<const uint16_t*>(fp4_src + size_t(brow_clamped(r)) * KB32)[q];
      }
    }
  }

  // K steps: the weights' K once, or (down with a split a) twice, first against the hi halves of
  // a, then against the lo halves; kwof(kk) is the weights' K step of step kk
  const int nkw = K / BK;
  const int nk = GATEUP ? nkw : nkw * asplit;
  auto kwof = [&](int kk) -> int { return kk >= nkw ? kk - nkw : kk; };

  // Wave layouts.  A tile of NS < 4 row blocks (and every MXFP4 tile): wave w owns MFMA column
  // block w (32 B columns) and all NS row blocks, so each B fragment feeds NS matrix instructions.
  // A full tile of bf16 or FP8 weights (4 row blocks): the waves form a 2 x 4 grid, wave w owning row blocks 2(w/4), 2(w/4)+1 and column
  // blocks 2(w%4), 2(w%4)+1, so each A and each B fragment feeds two matrix instructions (the
  // LDS bytes read per instruction fall by a third for FP8 weights; the two waves on a SIMD,
  // w and w+4, share its matrix core evenly).  Column block q holds B rows 16q..16q+15 of the
  // gate half and the same rows of the up half (gate/up), or rows 32q..32q+31 (down), so that
  // lanes l and l+16 of a gate/up block hold gate and up of the same output column.
  auto bcol = [&](int q) -> int {
    return GATEUP ? (ln < 16 ? 16 * q + ln : BN / 2 + 16 * q + (ln - 16)) : 32 * q + ln;
  };
  auto run = [&](auto ns_c) {
    constexpr int NS = decltype(ns_c)::value;
    // 2 x 4 wave grid for full tiles of bf16 and FP8 weights (MXFP4 tiles measured slower with it:
    // each column block adds its own scale reads and conversions)
    constexpr bool TD = NS == 4 && WD != DT_MXFP4;
    constexpr int NR = TD ? 2 : NS, NC = TD ? 2 : 1;  // row and column blocks of a wave
    const int rbase = TD ? 64 * (wv >> 2) : 0;        // first tile row of the wave's row blocks
    int blc[NC], srowc[NC], fp4_row[NC], fp4_keyl[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      blc[c] = bcol(TD ? 2 * (wv & 3) + c : wv);
      srowc[c] = kBlockScaled ? srow_of(blc[c]) : 0;
      fp4_row[c] = blc[c] * KB32;
      fp4_keyl[c] = fp4_key(blc[c]);
    }
    constexpr int AB = NS * 32 * F::AROW;             // A bytes per stage
    constexpr int NA = AB / 1024;                     // A chunks per step
    constexpr int A_HI = (NA + kWaves - 1) / kWaves;  // A chunks of waves 0 .. NA%8-1 (or all)
    constexpr int A_LO = NA / kWaves;                 // A chunks of the other waves
    constexpr int NST = F::nstage(NS);                // K steps in flight
    constexpr int SB = F::stage_bytes(NS);            // bytes per stage: A rows, then the B tile
    constexpr int KS = F::KS;                         // MFMA K sub-steps per step
    constexpr int kReads = NR + NC * (WD == DT_MXFP4 ? 2 : 1);  // LDS reads per sub-step
    static_assert(NST >= 2, "LDS budget");
    const int na = (NA % kWaves == 0 || wv < NA % kWaves) ? A_HI : A_LO;  // this wave's A chunks
    const int nl = na + F::INSTR;                                       // its loads per step
    const uint8_t* asrc[A_HI];
#pragma unroll
    for (int j = 0; j < A_HI; ++j) {
      const int c = j < na ? wv + kWaves * j : wv;  // unused entries point at a valid row
      asrc[j] = a_source(ARPC * c + lane / AGR);
    }
    const uint32_t lds0 = lds_addr(smem);
    // direct load j of this wave for K step kk into the stage at LDS address st: j < na are
    // A chunks, the rest B
    auto issue_one = [&](int j, int kk, uint32_t st) {
      if (j < na) {
#pragma unroll
        for (int q = 0; q < A_HI; ++q)
          if (q == j) dma16(asrc[q] + size_t(kk) * BK * 2, st + (wv + kWaves * q) * 1024);
      } else {
#pragma unroll
        for (int q = 0; q < F::INSTR; ++q)
          if (q == j - na) dma16(bsrc[q] + size_t(kwof(kk)) * (F::ROW), st + AB + (F::INSTR * wv + q) * 1024);
      }
    };
    // the step's loads are spread over the first half of its K sub-steps (KG of them), so that
    // they have the second half to land: group g issues loads [lo(g), lo(g+1))
    constexpr int KG = KS >= 4 ? KS / 2 : KS;
    auto issue_group = [&](int g, int kk, uint32_t st) {
      if (g >= KG) return;
#pragma unroll
      for (int j = 0; j < A_HI + F::INSTR; ++j)
        if (j < nl && j >= (nl * g) / KG && j < (nl * (g + 1)) / KG) issue_one(j, kk, st);
    };

    f32x16_t acc[NR][NC], tmp[NR][NC];
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][c][r] = tmp[i][c][r] = 0.0f;

    // raw LDS fragments of one K sub-step: A rows as bf16, B in its stored format (+ MXFP4 scale)
    struct Raw {
      bf16x8_t a[NR];
      uint32_t b[NC][WD == DT_BF16 ? 4 : WD == DT_FP8 ? 2 : 1];
      uint32_t sc[NC];
    };
    auto load_raw = [&](const uint8_t* st, int kk, int ks, Raw& f) {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int m = rbase + i * 32 + ln;
        f.a[i] = *reinterpret_cast<const bf16x8_t*>(st + m * F::AROW + swzA(m, ks * 2 + kh) * 16);
      }
      const uint8_t* B = st + AB;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int bl = blc[c];
        if constexpr (WD == DT_BF16) {
          const uint4 q = *reinterpret_cast<const uint4*>(B + bl * 128 + swz128(bl, ks * 2 + kh) * 16);
          f.b[c][0] = q.x; f.b[c][1] = q.y; f.b[c][2] = q.z; f.b[c][3] = q.w;
        } else if constexpr (WD == DT_FP8) {  // 128 K per row: granule ks holds K [16ks, 16ks+16)
          const uint2 q = *reinterpret_cast<const uint2*>(B + bl * 128 + swz128(bl, ks) * 16 + kh * 8);
          f.b[c][0] = q.x; f.b[c][1] = q.y;
        } else {  // 64-byte rows of 128 K: granule ks/2 holds K [32(ks/2), +32)
          f.b[c][0] = *reinterpret_cast<const uint32_t*>(B + bl * 64 + swz64(bl, ks >> 1) * 16 + (ks & 1) * 8 + kh * 4);
          const int kb = kwof(kk) * (BK / 32) + (ks >> 1);
          if (fp4_async) {
            int slot = (kb >> 4) + fp4_keyl[c];
            slot -= slot >= gpr ? gpr : 0;
            f.sc[c] = Sfp4[fp4_row[c] + slot * 16 + (kb & 15)];
          } else {
            f.sc[c] = Sfp4[fp4_row[c] + kb];
          }
        }
      }
    };
    // B fragment of column block c as bf16 (e4m3fn -> bf16 exact; e2m1 x power-of-two scale ->
    // bf16 exact)
    auto decode_b = [&](const Raw& f, int c) -> bf16x8_t {
      uint32_t o[4];
      if constexpr (WD == DT_BF16) {
        o[0] = f.b[c][0]; o[1] = f.b[c][1]; o[2] = f.b[c][2]; o[3] = f.b[c][3];
      } else if constexpr (WD == DT_FP8) {
        o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f.b[c][0], 1.0f, false));
        o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f.b[c][0], 1.0f, true));
        o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f.b[c][1], 1.0f, false));
        o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f.b[c][1], 1.0f, true));
      } else {
        const float sc = e8m0_to_f32(f.sc[c]);
        o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f.b[c][0], sc, 0));
        o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f.b[c][0], sc, 1));
        o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f.b[c][0], sc, 2));
        o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f.b[c][0], sc, 3));
      }
      return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
    };

    // prologue: side data visible (LDS writes done, then a barrier: no wait for the direct loads),
    // the MXFP4 scales and the first NST-1 steps in flight (steps past the end re-load the last
    // step, unused, so every wave always has the same number of loads in flight)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if constexpr (WD == DT_MXFP4) {
      if (fp4_async) {
        const int total = BN * gpr;  // granules, a multiple of 256
        const uint32_t sl = lds_addr(Sfp4);
        for (int c = wv; c * 64 < total; c += kWaves) {
          const int L = c * 64 + lane;
          const int r = L / gpr, slot = L - r * gpr;
          int q = slot - fp4_key(r);
          q += q < 0 ? gpr : 0;
          dma16(fp4_src + size_t(brow_clamped(r)) * KB32 + q * 16, sl + c * 1024);
        }
      }
    }
#pragma unroll
    for (int p = 0; p < NST - 1; ++p)
#pragma unroll
      for (int g = 0; g < KG; ++g) issue_group(g, min(p, nk - 1), lds0 + p * SB);
    int sr = 0;             // stage of step kk
    int sw = NST - 1;       // stage that step kk loads into
    for (int kk = 0; kk < nk; ++kk) {
      // this wave's loads of step kk are done once at most the next NST-2 steps' remain;
      // after the barrier every wave's are, and every wave has left step kk-1 (whose stage is sw)
      if (na == A_HI) wait_vmcnt<(A_HI + F::INSTR) * (NST - 2)>();
      else wait_vmcnt<(A_LO + F::INSTR) * (NST - 2)>();
      __builtin_amdgcn_s_barrier();
      const uint8_t* st = smem + sr * SB;
      const uint32_t wst = lds0 + sw * SB;
      const int kn = min(kk + NST - 1, nk - 1);
      sr = sr + 1 == NST ? 0 : sr + 1;
      sw = sw + 1 == NST ? 0 : sw + 1;
      Raw f[2];
      load_raw(st, kk, 0, f[0]);
      __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) load_raw(st, kk, ks + 1, f[(ks + 1) & 1]);
        issue_group(ks, kn, wst);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8_t b = decode_b(f[ks & 1], c);
#pragma unroll
          for (int i = 0; i < NR; ++i) {
            if constexpr (kBlockScaled)
              tmp[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[ks & 1].a[i], b, tmp[i][c], 0, 0, 0);
            else
              acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[ks & 1].a[i], b, acc[i][c], 0, 0, 0);
          }
        }
        // keep the next sub-step's LDS reads ahead of this sub-step's matrix instructions
        if (ks + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NR * NC, 0);
      }
      if constexpr (kBlockScaled) {
        // a step is one 128-wide K block: fold its partial sums in with the blocks' scales
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const float sc = Ssc[srowc[c]][kwof(kk)];
#pragma unroll
          for (int i = 0; i < NR; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              acc[i][c][r] = fmaf(sc, tmp[i][c][r], acc[i][c][r]);
              tmp[i][c][r] = 0.0f;
            }
        }
      }
    }
    wait_vmcnt<0>();  // the trailing re-loads must land before the work-group's LDS is released

    // ---- epilogue: accumulator r of lane l is row 8*(r/4) + 4*(l/32) + r%4 of its row block,
    // column l%32 of its column block
    if constexpr (GATEUP) {
      // a = silu(g) * u in bf16 goes through LDS so that it leaves in whole 16-byte pieces per
      // lane (the accumulator layout gives 2-byte pieces, 16 lanes to a row segment)
      uint16_t* at = reinterpret_cast<uint16_t*>(smem);  // [BM][128] bf16
      __syncthreads();  // every wave's direct loads have landed and its stage reads are done
#pragma unroll
      for (int i = 0; i < NR; ++i) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int col = 16 * (TD ? 2 * (wv & 3) + c : wv) + (ln & 15);  // output column in the tile
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            // registers r, r+1 are rows m, m+1; lane ln < 16 holds gate values, lane ln + 16 the
            // up values of the same columns.  One exchange gives the low lane (gate, up) of row m
            // and the high lane those of row m+1, so each lane forms one silu(g)*u per pair.
            const bool lo = ln < 16;
            const float x0 = acc[i][c][r], x1 = acc[i][c][r + 1];
            const float recv = __shfl_xor(lo ? x1 : x0, 16);
            const float g = lo ? x0 : recv, u = lo ? recv : x1;
            const int m = rbase + i * 32 + 8 * (r >> 2) + 4 * kh + (r & 3) + (lo ? 0 : 1);
            if (m < rows) {
              const float a = rowok[m] ? silu_fast(g) * u : 0.0f;
              const uint16_t hi = f32_to_bf16(a);
              at[m * 128 + col] = hi;
              // split a: the rounding error of the hi half, itself rounded to bf16 (a to ~16 bits)
              if (asplit == 2) at[BM * 128 + m * 128 + col] = f32_to_bf16(a - bf16_to_f32(hi));
            }
          }
        }
      }
      __syncthreads();
      const int ncol = min(128, I - n0);  // columns of this tile (a multiple of 8)
      const size_t ld = size_t(I) * asplit;  // a row: I values, or I hi halves then I lo halves
      for (int t = tid; t < rows * 16 * asplit; t += kThreads) {
        const int half = t / (rows * 16), tt = t - half * rows * 16;
        const int m = tt >> 4, c8 = (tt & 15) * 8;
        if (c8 < ncol)
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + size_t(m0 + m) * ld + size_t(half) * I + n0 + c8) =
              *reinterpret_cast<const uint4*>(at + half * BM * 128 + m * 128 + c8);
      }
    } else {
      store_y_tile<NR, NC, TD>([&](int i, int c, int r) { return acc[i][c][r]; }, smem, static_cast<float*>(out), m0,
                               rows, n0, N, (NS + 1) / 2);
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
// Mode B: block-scaled low-precision matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4).  A = E4M3
// activation codes with one E8M0 scale per row and 32 K (quantised beforehand), B = the stored
// weights: E4M3 (scale operand 1.0, the 128x128 block scale folded in per K block as in mode A)
// or E2M1 with its own E8M0 scales.  One MFMA covers 64 K (a 128-wide K step of the kernel takes
// two); operand lanes: lane (r, h) holds 8-bit K granules h and 2+h (16 elements each) of its 64,
// or 4-bit K [32h, 32h+32);
// lane r+32b supplies the scale of K block b of row (column) r.
// GATEUP = true:  A = quantised x rows (through perm), out a quantised (aq_out, as_out) for down
// GATEUP = false: A = quantised a rows (positions),    out y (fp32)
// ---------------------------------------------------------------------------------------------
template <int WD> struct QFmt {
  static constexpr int BK = 128;                            // K step: 128-byte E4M3 rows
  static constexpr int ROW = WD == DT_FP8 ? 128 : 64;       // B bytes per row and K step
  static constexpr int STAGE = BN * ROW;
  static constexpr int INSTR = STAGE / (1024 * kWaves);
  static constexpr int BUDGET = WD == DT_MXFP4 ? 104 * 1024 : 128 * 1024;
  static constexpr int stage_bytes(int ns) { return ns * 4096 + STAGE; }  // A: 32*NS rows x 128 B
  static constexpr int nstage(int ns) { return BUDGET / stage_bytes(ns) < 8 ? BUDGET / stage_bytes(ns) : 8; }
};

typedef int i32x8_t __attribute__((ext_vector_type(8)));

template <int WD, bool GATEUP>
__global__ __launch_bounds__(kThreads, 1) void gemm_q_kernel(
    const uint8_t* __restrict__ w, const void* __restrict__ wscale, const uint8_t* __restrict__ aq,
    const uint8_t* __restrict__ as, const int32_t* __restrict__ perm,
    const int4* __restrict__ tiles, const int32_t* __restrict__ ntiles, int S, int T, int k, int K, int N, int I,
    float* __restrict__ out, uint8_t* __restrict__ aq_out, uint8_t* __restrict__ as_out) {
  static_assert(WD == DT_FP8 || WD == DT_MXFP4, "mode B weights");
  using F = QFmt<WD>;
  __shared__ __align__(16) uint8_t smem[F::BUDGET];
  __shared__ float Ssc[4][64];                                                    // FP8 block scales
  __shared__ __align__(16) uint8_t Sfp4[WD == DT_MXFP4 ? BN * kMaxFp4Kb : 16];    // weight E8M0
  __shared__ __align__(16) uint8_t Sact[BM * kMaxFp4Kb];                          // activation E8M0
  __shared__ uint8_t rowok[BM];
  // tile j = b / 8 of XCD x = b % 8 (the scheduler's per-XCD lists of gridDim.x / 8 entries); the
  // count and the entry are loaded together (the entry slot exists for every block), and the entry
  // carries the tile's first row and row count, so no further index load precedes the operands
  const int xcd = blockIdx.x & 7, jt = blockIdx.x >> 3;
  const int ncnt = ntiles[xcd];
  const int4 ent = tiles[size_t(xcd) * (gridDim.x >> 3) + jt];
  if (jt >= ncnt) return;
  const int s = ent.x, m0 = ent.y, rows = ent.z, nt = ent.w;
  const int cap = T * k;
  // never taken for the scheduler's entries
  if (unsigned(s) >= unsigned(S) || rows <= 0 || rows > BM || m0 < 0 || m0 + rows > cap) return;
  const int nsub = (rows + 31) >> 5;
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, kh = lane >> 5;
  const int n0 = GATEUP ? nt * (BN / 2) : nt * BN;
  const size_t rb = row_bytes<WD>(K);
  const uint8_t* wslot = w + size_t(s) * N * rb;
  auto brow_global = [&](int r) -> int {
    if constexpr (GATEUP) return r < BN / 2 ? n0 + r : I + n0 + (r - BN / 2);
    return n0 + r;
  };
  auto brow_clamped = [&](int r) -> int { return min(brow_global(r), N - 1); };
  // activation row of tile row r (a valid row for rows past the tile, never stored)
  auto a_row = [&](int r) -> int {
    int src = GATEUP ? 0 : m0;
    if (r < rows) {
      if constexpr (GATEUP) {
        const int rr = perm[m0 + r];
        src = (rr >= 0 && rr / k < T) ? rr / k : 0;
      } else {
        src = m0 + r;
      }
    }
    return src;
  };
  constexpr int BK = F::BK;
  // B sources: 128-byte rows: lane -> row 8c + lane/8 (fp8); 64-byte rows: row 16c + lane/4 (fp4)
  const uint8_t* bsrc[F::INSTR];
#pragma unroll
  for (int j = 0; j < F::INSTR; ++j) {
    const int c = F::INSTR * wv + j;
    int r, g;
    if constexpr (WD == DT_FP8) {
      r = 8 * c + (lane >> 3);
      g = swz128(r, lane & 7);
    } else {
      r = 16 * c + (lane >> 2);
      g = swz64(r, lane & 3);
    }
    bsrc[j] = wslot + size_t(brow_clamped(r)) * rb + g * 16;
  }
  if (tid < BM) {
    bool ok = tid < rows;
    if constexpr (GATEUP) {
      if (ok) {
        const int rr = perm[m0 + tid];
        ok = rr >= 0 && rr / k < T;
      }
    }
    rowok[tid] = ok;
  }
  const int bl = GATEUP ? (ln < 16 ? 16 * wv + ln : BN / 2 + 16 * wv + (ln - 16)) : 32 * wv + ln;
  int srow = 0;
  if constexpr (WD == DT_FP8) {
    const int KB = (K + 127) >> 7;
    const int NBk = (N + 127) >> 7;
    int blk[4];
    blk[0] = brow_clamped(0) >> 7;
    blk[1] = brow_clamped(127) >> 7;
    blk[2] = brow_clamped(128) >> 7;
    blk[3] = brow_clamped(255) >> 7;
    const float* sbase = static_cast<const float*>(wscale) + size_t(s) * NBk * KB;
    for (int t = tid; t < 4 * KB; t += kThreads) {
      const int r = t / KB, kb = t - r * KB;
      Ssc[r][kb] = sbase[size_t(blk[r]) * KB + kb];
    }
    const int gb = brow_clamped(bl) >> 7;
    srow = gb == blk[0] ? 0 : gb == blk[1] ? 1 : gb == blk[2] ? 2 : 3;
  }
  // E8M0 rows (weights of the tile's columns; activations of its rows): [row][K/32] in LDS.  With
  // K % 512 == 0 a row is gpr whole 16-byte granules, rotated by a per-row key so that the rows
  // read together by one instruction fall in different LDS banks, and loaded by direct loads
  // issued with the first stages; otherwise copied unrotated before the main loop.
  const int KB32 = K >> 5;
  const bool sc_async = KB32 % 16 == 0;
  const int gpr = sc_async ? KB32 >> 4 : 1;
  const int sc_d = sc_async ? 16 / ((gpr & -gpr) < 16 ? (gpr & -gpr) : 16) : 1;
  auto sc_key = [&](int r) -> int { return sc_async ? (r / sc_d) % gpr : 0; };
  auto sc_index = [&](int r, int kb) -> int {
    if (!sc_async) return r * KB32 + kb;
    int slot = (kb >> 4) + sc_key(r);
    slot -= slot >= gpr ? gpr : 0;
    return r * KB32 + slot * 16 + (kb & 15);
  };
  const uint8_t* fp4_src = WD == DT_MXFP4 ? static_cast<const uint8_t*>(wscale) + size_t(s) * N * KB32 : nullptr;
  if (!sc_async) {
    for (int t = tid; t < BM * KB32; t += kThreads) {
      const int r = t / KB32, q = t - r * KB32;
      Sact[t] = as[size_t(a_row(r)) * KB32 + q];
    }
    if constexpr (WD == DT_MXFP4) {
      for (int t = tid; t < BN * KB32; t += kThreads) {
        const int r = t / KB32, q = t - r * KB32;
        Sfp4[t] = fp4_src[size_t(brow_clamped(r)) * KB32 + q];
      }
    }
  }

  const int nk = K / BK;

  auto run = [&](auto ns_c) {
    constexpr int NS = decltype(ns_c)::value;
    constexpr int NA = 4 * NS;                        // A chunks (8 rows x 128 B) per step
    constexpr int A_HI = (NA + kWaves - 1) / kWaves;
    constexpr int A_LO = NA / kWaves;
    constexpr int NST = F::nstage(NS);
    constexpr int SB = F::stage_bytes(NS);
    constexpr int AB = NS * 4096;
    static_assert(NST >= 2, "LDS budget");
    const int na = (NA % kWaves == 0 || wv < NA % kWaves) ? A_HI : A_LO;
    const int nl = na + F::INSTR;
    const uint8_t* asrc[A_HI > 0 ? A_HI : 1];
#pragma unroll
    for (int j = 0; j < (A_HI > 0 ? A_HI : 1); ++j) {
      const int c = j < na ? wv + kWaves * j : 0;
      const int r = 8 * c + (lane >> 3);
      asrc[j] = aq + size_t(a_row(r)) * K + swz128(r, lane & 7) * 16;
    }
    const uint32_t lds0 = lds_addr(smem);
    auto issue_one = [&](int j, int kk, uint32_t st) {
      if (j < na) {
#pragma unroll
        for (int q = 0; q < A_HI; ++q)
          if (q == j) dma16(asrc[q] + size_t(kk) * BK, st + (wv + kWaves * q) * 1024);
      } else {
#pragma unroll
        for (int q = 0; q < F::INSTR; ++q)
          if (q == j - na) dma16(bsrc[q] + size_t(kk) * (F::ROW), st + AB + (F::INSTR * wv + q) * 1024);
      }
    };
    auto issue_step = [&](int kk, uint32_t st) {
#pragma unroll
      for (int j = 0; j < A_HI + F::INSTR; ++j)
        if (j < nl) issue_one(j, kk, st);
    };

    f32x16_t acc[NS], tmp[NS];
#pragma unroll
    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ms][r] = tmp[ms][r] = 0.0f;

    // prologue: side data visible, the scale rows and the first NST-1 steps in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (sc_async) {
      const uint32_t la = lds_addr(Sact);
      for (int c = wv; c * 64 < BM * gpr; c += kWaves) {
        const int L = c * 64 + lane;
        const int r = L / gpr, slot = L - r * gpr;
        int q = slot - sc_key(r);
        q += q < 0 ? gpr : 0;
        dma16(as + size_t(a_row(r)) * KB32 + q * 16, la + c * 1024);
      }
      if constexpr (WD == DT_MXFP4) {
        const uint32_t lb = lds_addr(Sfp4);
        for (int c = wv; c * 64 < BN * gpr; c += kWaves) {
          const int L = c * 64 + lane;
          const int r = L / gpr, slot = L - r * gpr;
          int q = slot - sc_key(r);
          q += q < 0 ? gpr : 0;
          dma16(fp4_src + size_t(brow_clamped(r)) * KB32 + q * 16, lb + c * 1024);
        }
      }
    }
#pragma unroll
    for (int p = 0; p < NST - 1; ++p) issue_step(min(p, nk - 1), lds0 + p * SB);
    int sr = 0, sw = NST - 1;
    for (int kk = 0; kk < nk; ++kk) {
      if (na == A_HI) wait_vmcnt<(A_HI + F::INSTR) * (NST - 2)>();
      else wait_vmcnt<(A_LO + F::INSTR) * (NST - 2)>();
      __builtin_amdgcn_s_barrier();
      const uint8_t* st = smem + sr * SB;
      const uint32_t wst = lds0 + sw * SB;
      const int kn = min(kk + NST - 1, nk - 1);
      sr = sr + 1 == NST ? 0 : sr + 1;
      sw = sw + 1 == NST ? 0 : sw + 1;
      issue_step(kn, wst);
      // two 64-wide MFMA sub-steps: lane (r, h) takes 8-bit granules 4s+h and 4s+2+h of its
      // 128-byte row, or the 4-bit granule 2s+h of a 64-byte weight row; scales of K block
      // 4kk + 2s + h
      const uint8_t* B = st + AB;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int kb = kk * 4 + 2 * sub + kh;
        i32x8_t b;
        int sb = 127;
        if constexpr (WD == DT_FP8) {
          const uint4 q0 = *reinterpret_cast<const uint4*>(B + bl * 128 + swz128(bl, 4 * sub + kh) * 16);
          const uint4 q1 = *reinterpret_cast<const uint4*>(B + bl * 128 + swz128(bl, 4 * sub + 2 + kh) * 16);
          b[0] = q0.x; b[1] = q0.y; b[2] = q0.z; b[3] = q0.w;
          b[4] = q1.x; b[5] = q1.y; b[6] = q1.z; b[7] = q1.w;
        } else {
          const uint4 q0 = *reinterpret_cast<const uint4*>(B + bl * 64 + swz64(bl, 2 * sub + kh) * 16);
          b[0] = q0.x; b[1] = q0.y; b[2] = q0.z; b[3] = q0.w;
          b[4] = 0; b[5] = 0; b[6] = 0; b[7] = 0;
          sb = Sfp4[sc_index(bl, kb)];
        }
        i32x8_t a[NS];
        int sa[NS];
#pragma unroll
        for (int ms = 0; ms < NS; ++ms) {
          const int m = ms * 32 + ln;
          const uint4 q0 = *reinterpret_cast<const uint4*>(st + m * 128 + swz128(m, 4 * sub + kh) * 16);
          const uint4 q1 = *reinterpret_cast<const uint4*>(st + m * 128 + swz128(m, 4 * sub + 2 + kh) * 16);
          a[ms][0] = q0.x; a[ms][1] = q0.y; a[ms][2] = q0.z; a[ms][3] = q0.w;
          a[ms][4] = q1.x; a[ms][5] = q1.y; a[ms][6] = q1.z; a[ms][7] = q1.w;
          sa[ms] = Sact[sc_index(m, kb)];
        }
#pragma unroll
        for (int ms = 0; ms < NS; ++ms) {
          if constexpr (WD == DT_FP8)
            tmp[ms] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[ms], b, tmp[ms], 0, 0, 0, sa[ms], 0, sb);
          else
            acc[ms] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[ms], b, acc[ms], 0, 4, 0, sa[ms], 0, sb);
        }
      }
      if constexpr (WD == DT_FP8) {  // a step is one 128-wide K block
        const float sc = Ssc[srow][kk];
#pragma unroll
        for (int ms = 0; ms < NS; ++ms)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            acc[ms][r] = fmaf(sc, tmp[ms][r], acc[ms][r]);
            tmp[ms][r] = 0.0f;
          }
      }
    }
    wait_vmcnt<0>();

    if constexpr (GATEUP) {
      // a = silu(g) * u of the tile (rows x 128 columns; I is a multiple of 128 here) goes through
      // LDS and leaves quantised, per row and 32 columns, by the rule of the quantisation kernel
      // (the down projection's input): one write of 1 + 1/32 bytes per element instead of an fp32
      // store and a second pass over it
      float* at = reinterpret_cast<float*>(smem);  // [BM][128] fp32 (64 KiB of the stages)
      __syncthreads();  // every wave's direct loads have landed and its stage reads are done
#pragma unroll
      for (int ms = 0; ms < NS; ++ms) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          // one silu(g)*u per lane and register pair, as in mode A
          const bool lo = ln < 16;
          const float x0 = acc[ms][r], x1 = acc[ms][r + 1];
          const float recv = __shfl_xor(lo ? x1 : x0, 16);
          const float g = lo ? x0 : recv, u = lo ? recv : x1;
          const int m = ms * 32 + 8 * (r >> 2) + 4 * kh + (r & 3) + (lo ? 0 : 1);
          if (m < rows) at[m * 128 + 16 * wv + (ln & 15)] = rowok[m] ? silu_fast(g) * u : 0.0f;
        }
      }
      __syncthreads();
      const int KB = I >> 5;
      // four lanes per 32-column block (eight columns each), the block maximum by two lane swaps;
      // groups of four lanes are active together (rows * 16 is a multiple of 4)
      for (int t = tid; t < rows * 16; t += kThreads) {
        const int m = t >> 4, blk = (t >> 2) & 3, part = t & 3;
        const float4 p = *reinterpret_cast<const float4*>(at + m * 128 + blk * 32 + part * 8);
        const float4 q = *reinterpret_cast<const float4*>(at + m * 128 + blk * 32 + part * 8 + 4);
        const float v[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
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
        uint2 o2;
        o2.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
        o2.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
        *reinterpret_cast<uint2*>(aq_out + size_t(m0 + m) * I + n0 + blk * 32 + part * 8) = o2;
        if (part == 0) as_out[size_t(m0 + m) * KB + (n0 >> 5) + blk] = uint8_t(X + 127);
      }
    } else {
      store_y_tile<NS, 1, false>([&](int i, int, int r) { return acc[i][r]; }, smem, out, m0, rows, n0, N, (NS + 1) / 2);
    }
  };
  switch (nsub) {
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 3: run(std::integral_constant<int, 3>{}); break;
    default: run(std::integral_constant<int, 4>{}); break;
  }
}

// fp32 activations -> bf16 (nearest even) for the matrix-core path
__global__ void cast_bf16_kernel(const float* __restrict__ x, uint16_t* __restrict__ y, size_t n) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += size_t(gridDim.x) * blockDim.x)
    y[i] = f32_to_bf16(x[i]);
}

// ---------------------------------------------------------------------------------------------
// Tile scheduler (one work-group; S <= 1024, so thread t owns slot t).  Each GEMM block runs one
// (slot, M tile, N tile) entry {slot, first row, rows, n_tile}.  The tiles are dealt to the eight
// XCDs, block b of a launch of 8 * cap blocks running entry j = b / 8 of XCD x = b % 8 (blocks are
// dealt to the XCDs round robin): tiles[x * cap + j], j < counts[x] (counts[8 + x] for the down
// GEMM).  With one work-group per CU, each XCD's 32 CUs take its entries in order as they free up.
//
// Balanced order.  The unit of work is up to kUnitM consecutive M tiles of one slot with all their
// N tiles, which an XCD's CUs run side by side, so that the slot's weight slices come from L2 once
// per unit.  A unit costs about the bytes its tiles move per K step: an M tile of ns 32-row
// blocks moves ns activation blocks and a weight tile worth 4 of them, so its key is
// sum(ns + 4) over its M tiles (5 .. 32; 32 = kUnitM full tiles).  Units are sorted by key,
// largest first (ties in slot order), and dealt serpentine (XCD 0..7, then 7..0, ...), so that the
// XCDs get similar shares of the bytes and each ends on small units.  Against the (slot, M, N)
// order in eight equal runs this evens out the XCDs' work on skewed routing: a model of one tile
// per CU at a time, tile time proportional to those bytes, gives 1.03x the ideal makespan instead
// of 1.12x on the Zipf prefill batch and 1.10x instead of 1.35x on the 110-slot compact one
// (measured: the compact gate/up GEMM 16 % faster, the Zipf one 2-4 %).
// Only every slot's last unit can be partial; the others all have key 32.
// Fallback (the units' table beyond the LDS the host granted, or an XCD's list beyond its
// capacity): the (slot, M tile, N tile) order cut into eight contiguous runs.
// ---------------------------------------------------------------------------------------------
constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / 64;
constexpr int kUnitM = 4;  // M tiles per unit (2 and 8 measured no better at the prefill shapes)
constexpr int kKeys = kUnitM * (BM / 32 + 4) + 1;  // unit keys 0 .. 32

__device__ __forceinline__ int serp_xcd(int i) { return ((i >> 3) & 1) ? 7 - (i & 7) : (i & 7); }

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const int32_t* __restrict__ off, int S,
                                                                 int cap, int nt_gu, int nt_dn, int slots_gu,
                                                                 int slots_dn, int umax,
                                                                 int4* __restrict__ tiles_gu,
                                                                 int4* __restrict__ tiles_dn,
                                                                 int32_t* __restrict__ counts) {
  // [S + 1] M-tile bases; then (balanced) useq[umax], toff[umax], and per listed M tile its slot and
  // row count (tma) and first row (tmr)
  extern __shared__ int32_t mbase[];
  __shared__ int32_t wsum[kSchedWaves];
  __shared__ int32_t wkey[kSchedWaves][kKeys];  // per-wave key counts, then their bases
  __shared__ int32_t kbase[kKeys];
  __shared__ int32_t xcnt[8], xbase[9];
  __shared__ int32_t nunits, balanced;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int cap_gu = slots_gu >> 3, cap_dn = slots_dn >> 3;
  // this thread's slot: rows, M tiles, units, key of the last unit
  int mt = 0, nu = 0, klast = 0;
  if (tid < S) {
    const int lo = min(max(off[tid], 0), cap), hi = min(max(off[tid + 1], lo), cap);
    const int n = hi - lo;
    mt = (n + BM - 1) / BM;
    if (mt > 0) {
      nu = (mt + kUnitM - 1) / kUnitM;
      const int mtl = mt - kUnitM * (nu - 1);              // M tiles of the last unit
      const int rl = n - BM * (mt - 1);                    // rows of the slot's last M tile
      klast = (BM / 32 + 4) * (mtl - 1) + (rl + 31) / 32 + 4;
    }
  }
  for (int i = tid; i < kSchedWaves * kKeys; i += kSchedThreads) (&wkey[0][0])[i] = 0;
  // exclusive scans over slots: M tiles (mbase) and units of key kKeys-1 (f32)
  const int nfull = nu > 0 ? (nu - 1) + (klast == kKeys - 1 ? 1 : 0) : 0;
  auto block_scan = [&](int v, int& total) -> int {
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o);
      if (lane >= o) incl += u;
    }
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    int run = incl - v;
    total = 0;
    for (int w = 0; w < kSchedWaves; ++w) {
      if (w < wid) run += wsum[w];
      total += wsum[w];
    }
    __syncthreads();
    return run;
  };
  int MT = 0, nfull_tot = 0;
  const int mb = block_scan(mt, MT);
  const int fb = block_scan(nfull, nfull_tot);
  if (tid < S) mbase[tid] = mb;
  if (tid == 0) mbase[S] = MT;
  // the last unit of a slot with key below the maximum: its rank among equal keys in lower slots
  const int ksmall = (nu > 0 && klast < kKeys - 1) ? klast : -1;
  int rank = 0;
  {
    unsigned long long todo = __ballot(ksmall >= 0);
    while (todo) {
      const int leader = __ffsll((long long)todo) - 1;
      const int lk = __shfl(ksmall, leader);
      const unsigned long long m = __ballot(ksmall == lk);
      if (ksmall == lk) rank = __popcll(m & ((1ull << lane) - 1ull));
      if (lane == leader) wkey[wid][lk] = __popcll(m);
      todo &= ~m;
    }
  }
  __syncthreads();
  if (tid < kKeys) {  // per key: wave bases, key total
    int run = 0;
    for (int w = 0; w < kSchedWaves; ++w) {
      const int c = wkey[w][tid];
      wkey[w][tid] = run;
      run += c;
    }
    kbase[tid] = run;
  }
  __syncthreads();
  if (tid == 0) {  // key bases, largest key first: the full units, then keys kKeys-2 .. 0
    int run = nfull_tot;
    for (int key = kKeys - 2; key >= 0; --key) {
      const int c = kbase[key];
      kbase[key] = run;
      run += c;
    }
    kbase[kKeys - 1] = 0;
    nunits = run;
    balanced = umax > 0 && run <= umax;
  }
  __syncthreads();
  const int U = nunits;
  if (balanced) {
    int32_t* useq = mbase + S + 1;  // sorted units: (unit index << 10) | slot
    int32_t* toff = useq + umax;    // M-tile offset of a unit in its XCD's list
    int32_t* tma = toff + umax;     // listed M tile (XCD x's M tiles from xbase[x]): slot | rows << 16
    int32_t* tmr = tma + umax;      // its first row
    if (tid < S) {
      const int nf = nu - (ksmall >= 0 ? 1 : 0);
      for (int i = 0; i < nf; ++i) useq[fb + i] = (i << 10) | tid;
      if (ksmall >= 0) useq[kbase[ksmall] + wkey[wid][ksmall] + rank] = ((nu - 1) << 10) | tid;
    }
    __syncthreads();
    if (wid < 8) {  // wave x: the units of XCD x (sorted positions 8j + x, or 8j + 7 - x for odd j)
      const int x = wid;
      // XCD x holds J units j = 0 .. J-1 (largest first); its list takes them from the larger and
      // the smaller half in turn (even XCDs start with the larger, odd ones with the smaller), so
      // that matrix-bound and HBM-bound units run side by side and the list ends on a small one
      const int jl = U >> 3;
      const int J = jl + (8 * jl + ((jl & 1) ? 7 - x : x) < U ? 1 : 0);
      const int JH = (J + 1) >> 1, JC = J >> 1;
      int carry = 0;
      for (int p0 = 0; p0 < J; p0 += 64) {
        const int p = p0 + lane;
        int j;
        if ((x & 1) == 0) j = (p & 1) ? JH + (p >> 1) : (p >> 1);
        else j = (p & 1) ? (p >> 1) : ((p >> 1) < JC ? JH + (p >> 1) : (p >> 1));
        const int i = p < J ? 8 * j + ((j & 1) ? 7 - x : x) : U;
        int m = 0;
        if (i < U) {
          const int q = useq[i], s = q & 1023, ui = q >> 10;
          m = min(kUnitM, (mbase[s + 1] - mbase[s]) - kUnitM * ui);
        }
        int incl = m;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int u = __shfl_up(incl, o);
          if (lane >= o) incl += u;
        }
        if (i < U) toff[i] = carry + incl - m;
        carry += __shfl(incl, 63);
      }
      if (lane == 0) xcnt[x] = carry;
    }
    __syncthreads();
    if (tid == 0) {
      for (int x = 0; x < 8; ++x)
        if (xcnt[x] * nt_gu > cap_gu || xcnt[x] * nt_dn > cap_dn) balanced = 0;
    }
    __syncthreads();
    if (balanced) {
      if (tid == 0) {
        int run = 0;
        for (int x = 0; x < 8; ++x) {
          xbase[x] = run;
          run += xcnt[x];
        }
        xbase[8] = run;
      }
      __syncthreads();
      // every listed M tile: slot, rows, first row (a unit's M tiles are consecutive in its list)
      for (int i = tid; i < U; i += kSchedThreads) {
        const int q = useq[i], s = q & 1023, m0 = kUnitM * (q >> 10);
        const int mu = min(kUnitM, (mbase[s + 1] - mbase[s]) - m0);
        const int lo = min(max(off[s], 0), cap), hi = min(max(off[s + 1], lo), cap);
        const int b = xbase[serp_xcd(i)] + toff[i];
        for (int mm = 0; mm < mu; ++mm) {
          const int r0 = lo + (m0 + mm) * BM;
          tma[b + mm] = s | (min(BM, hi - r0) << 16);
          tmr[b + mm] = r0;
        }
      }
      __syncthreads();
      // the lists, written in order (consecutive threads, consecutive entries): entry j of XCD x is
      // N tile j % NT of listed M tile j / NT
      for (int g = 0; g < 2; ++g) {
        const int NT = g ? nt_dn : nt_gu;
        int4* tl = g ? tiles_dn : tiles_gu;
        const size_t cx = g ? cap_dn : cap_gu;
        for (int e = tid; e < xbase[8] * NT; e += kSchedThreads) {
          int x = 0;
          while (x < 7 && e >= xbase[x + 1] * NT) ++x;
          const int j = e - xbase[x] * NT, m = j / NT;
          const int a = tma[xbase[x] + m];
          tl[size_t(x) * cx + j] = make_int4(a & 0xFFFF, tmr[xbase[x] + m], a >> 16, j - m * NT);
        }
      }
      if (tid < 8) {
        counts[tid] = xcnt[tid] * nt_gu;
        counts[8 + tid] = xcnt[tid] * nt_dn;
      }
      return;
    }
  }
  // fallback: entry L of a GEMM with NT column tiles belongs to the last slot s with
  // mbase[s] * NT <= L; within the slot, L - mbase[s]*NT = m_tile * NT + n_tile; XCD x takes the
  // contiguous run of ceil((total - x) / 8) entries after those of XCDs 0 .. x-1
  for (int g = 0; g < 2; ++g) {
    const int NT = g ? nt_dn : nt_gu;
    const int cx = g ? cap_dn : cap_gu;
    int4* tl = g ? tiles_dn : tiles_gu;
    // the host sized the lists for consistent offsets (sum of rows <= T*k); never write past them
    const int total = min(MT * NT, 8 * cx);
    for (int L = tid; L < total; L += kSchedThreads) {
      const int q = L / NT;
      int lo = 0, hi = S - 1;  // last s in [0, S) with mbase[s] <= q
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (mbase[mid] <= q) lo = mid;
        else hi = mid - 1;
      }
      const int s = lo;
      const int local2 = L - mbase[s] * NT;
      const int m = local2 / NT, n = local2 - m * NT;
      int x = 0, base = 0;
      while (x < 7 && L >= base + (total - x + 7) / 8) {
        base += (total - x + 7) / 8;
        ++x;
      }
      const int slo = min(max(off[s], 0), cap), shi = min(max(off[s + 1], slo), cap);
      const int r0 = slo + m * BM;
      tl[size_t(x) * cx + (L - base)] = make_int4(s, r0, min(BM, shi - r0), n);
    }
    if (tid < 8) counts[8 * g + tid] = (total - tid + 7) / 8;
  }
}

}  // namespace gemm

size_t gemm_tiles_max(int T, int k, int S, int nt) {
  const long long R = (long long)T * k;
  const long long mt = R / gemm::BM + (R < S ? R : S);
  return size_t(mt) * nt;
}

// eight per-XCD lists, each an eighth of the bound plus one unit of kUnitM M tiles (the balanced
// order can put up to a unit more than an even share on one XCD)
size_t gemm_tile_slots(int T, int k, int S, int nt) {
  const size_t m = gemm_tiles_max(T, k, S, nt);
  return m == 0 ? 0 : ((m + 7) / 8 + size_t(gemm::kUnitM) * nt) * 8;
}

int gemm_nt_gate_up(int I) { return (I + gemm::BN / 2 - 1) / (gemm::BN / 2); }
int gemm_nt_down(int H) { return (H + gemm::BN - 1) / gemm::BN; }

hipError_t launch_gemm_schedule(const GemmArgs& g, hipStream_t st) {
  const int ngu = gemm_nt_gate_up(g.I), ndn = gemm_nt_down(g.H);
  // the balanced order keeps two words per unit and two per M tile in LDS (units <= M tiles <= the
  // bound below); beyond the LDS budget the scheduler falls back to contiguous runs
  constexpr size_t kDynLdsMax = 150 * 1024;
  const size_t base = sizeof(int32_t) * size_t(g.S + 1);
  const size_t umax = gemm_tiles_max(g.T, g.k, g.S, 1);
  // the caller may ask for the fallback order (same results, other placement)
  const bool fits = !g.tiles_contiguous && base + 4 * sizeof(int32_t) * umax <= kDynLdsMax;
  const size_t lds = fits ? base + 4 * sizeof(int32_t) * umax : base;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm::schedule_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  gemm::schedule_kernel<<<1, gemm::kSchedThreads, lds, st>>>(
      g.off, g.S, g.T * g.k, ngu, ndn, int(gemm_tile_slots(g.T, g.k, g.S, ngu)),
      int(gemm_tile_slots(g.T, g.k, g.S, ndn)), fits ? int(umax) : 0, g.tiles_gu, g.tiles_dn, g.counts);
  return hipGetLastError();
}

template <int WD>
static hipError_t gate_up_t(const GemmArgs& g, hipStream_t st) {
  const size_t grid = gemm_tile_slots(g.T, g.k, g.S, gemm_nt_gate_up(g.I));
  if (grid == 0) return hipSuccess;
  const void* x = g.x;
  if (g.xdt == DT_F32) {  // the matrix cores read bf16: round the activations once
    const size_t n = size_t(g.T) * g.H;
    gemm::cast_bf16_kernel<<<dim3(unsigned((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)), dim3(256), 0, st>>>(
        static_cast<const float*>(g.x), static_cast<uint16_t*>(g.xb), n);
    x = g.xb;
  }
  gemm::gemm_kernel<WD, true><<<dim3(unsigned(grid)), dim3(gemm::kThreads), 0, st>>>(
      static_cast<const uint8_t*>(g.w_gu), g.s_gu, static_cast<const uint16_t*>(x), g.perm, g.tiles_gu,
      g.counts, g.S, g.T, g.k, g.H, 2 * g.I, g.I, g.asplit, g.a);
  return hipGetLastError();
}

template <int WD>
static hipError_t down_t(const GemmArgs& g, hipStream_t st) {
  const size_t grid = gemm_tile_slots(g.T, g.k, g.S, gemm_nt_down(g.H));
  if (grid == 0) return hipSuccess;
  gemm::gemm_kernel<WD, false><<<dim3(unsigned(grid)), dim3(gemm::kThreads), 0, st>>>(
      static_cast<const uint8_t*>(g.w_d), g.s_d, static_cast<const uint16_t*>(g.a), nullptr, g.tiles_dn,
      g.counts + 8, g.S, g.T, g.k, g.I, g.H, g.I, g.asplit, g.y);
  return hipGetLastError();
}

template <int WD>
static hipError_t gate_up_q_t(const GemmArgs& g, hipStream_t st) {
  const size_t grid = gemm_tile_slots(g.T, g.k, g.S, gemm_nt_gate_up(g.I));
  if (grid == 0) return hipSuccess;
  gemm::gemm_q_kernel<WD, true><<<dim3(unsigned(grid)), dim3(gemm::kThreads), 0, st>>>(
      static_cast<const uint8_t*>(g.w_gu), g.s_gu, g.xq, g.xs, g.perm, g.tiles_gu, g.counts, g.S, g.T,
      g.k, g.H, 2 * g.I, g.I, nullptr, g.aq, g.as);
  return hipGetLastError();
}

template <int WD>
static hipError_t down_q_t(const GemmArgs& g, hipStream_t st) {
  const size_t grid = gemm_tile_slots(g.T, g.k, g.S, gemm_nt_down(g.H));
  if (grid == 0) return hipSuccess;
  gemm::gemm_q_kernel<WD, false><<<dim3(unsigned(grid)), dim3(gemm::kThreads), 0, st>>>(
      static_cast<const uint8_t*>(g.w_d), g.s_d, g.aq, g.as, nullptr, g.tiles_dn, g.counts + 8, g.S,
      g.T, g.k, g.I, g.H, g.I, g.y, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_gemm_gate_up_q(const GemmArgs& g, hipStream_t st) {
  switch (g.wdt) {
    case DT_FP8: return gate_up_q_t<DT_FP8>(g, st);
    case DT_MXFP4: return gate_up_q_t<DT_MXFP4>(g, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_down_q(const GemmArgs& g, hipStream_t st) {
  switch (g.wdt) {
    case DT_FP8: return down_q_t<DT_FP8>(g, st);
    case DT_MXFP4: return down_q_t<DT_MXFP4>(g, st);
  }
  return hipErrorInvalidValue;
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
