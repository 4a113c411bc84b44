// Internal launch interface between the C ABI (moe_abi.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

hipError_t launch_router_logits(const void* x, int xdt, const float* wr, const float* bias,
                                float* logits, int T, int H, int E, hipStream_t st);
hipError_t launch_topk(const float* logits, const float* bias, int add_bias, int T, int E, int k,
                       int score, int renorm, int32_t* idx, float* w, hipStream_t st);

size_t permute_lds_bytes(int E, int S);
hipError_t launch_permute(const int32_t* topk_idx, const float* topk_w, int T, int k, int E,
                          const int32_t* slot_map, int S, int32_t* counts, int32_t* slot_offsets,
                          int32_t* perm, int32_t* inv_perm, int32_t* miss_count,
                          int32_t* miss_token, int32_t* miss_expert, float* miss_weight,
                          uint32_t* err, int32_t* scratch, hipStream_t st);
// device scratch (bytes) launch_permute needs for T*k rows: 0 when one work-group does it all
size_t permute_scratch_bytes(int T, int k, int E, int S);
// top-k of every token and the permutation in one work-group (small batches)
size_t route_permute_lds_bytes(int T, int k, int E, int S);
hipError_t launch_route_permute(const float* logits, const float* bias, int T, int k, int E,
                                int score, int renorm, int32_t* idx, float* w,
                                const int32_t* slot_map, int S, int32_t* counts, int32_t* off,
                                int32_t* perm, int32_t* inv, int32_t* mc, int32_t* mt, int32_t* me,
                                float* mw, uint32_t* err, hipStream_t st);

struct GemvArgs {
  int wdt, xdt;
  int S, T, k, H, I;
  int n_ord;  // grid rows: an upper bound on the number of non-empty slots
  const void* w_gu;
  const void* s_gu;
  const void* w_d;
  const void* s_d;
  const void* x;
  const int32_t* perm;
  const int32_t* off;
  float* a;  // [T*k, I] fp32
  float* y;  // [T*k, H] fp32
};
hipError_t launch_gemv_gate_up(const GemvArgs& g, hipStream_t st);
hipError_t launch_gemv_down(const GemvArgs& g, hipStream_t st);

// Fused decode layer for small batches (two launches, see gemv_impl.h): routing, permutation and
// gate/up in the first; down projection and combine in the second.
constexpr int kDecMaxT = 4;    // tokens: one wave of a work-group selects each token's experts
constexpr int kDecMaxR = 64;   // rows T*k: one wave holds the slot of every row
constexpr int kDecFuseRows = 32;      // rows T*k up to which moe_layer takes the decode layer (MXFP4 weights)
constexpr int kDecFuseRowsWide = 8;   // the same for bf16, FP8 and fp32 weights
constexpr int kDecRB = 16;     // output columns per work-group of the down + combine launch
struct DecodeArgs {
  int wdt, xdt, odt;
  int S, T, k, H, I, E;
  int score, renorm;
  const float* logits;     // [T, E] router logits
  const float* bias;       // [E] selection bias or null
  const int32_t* slot_map; // [E] expert -> slot (-1: absent) or null (slot = expert)
  const void* w_gu;
  const void* s_gu;
  const void* w_d;
  const void* s_d;
  const void* x;           // [T, H]
  int32_t* topk_idx;       // [T*k] out
  float* topk_w;           // [T*k] out
  int32_t* rkey;           // [T*k] out: slot of row t*k+j, -1 when the row is not computed here
  int32_t* miss_count;     // [1] out
  int32_t* miss_token;     // [T*k] out (null without a slot map)
  int32_t* miss_expert;
  float* miss_weight;
  uint32_t* err;           // [1] out: 1 when a slot_map entry is out of range
  float* a;                // [T*k, I] fp32, by row index t*k+j
  void* out;               // [T, H]
};
// whether the two-launch decode layer takes this shape (LDS budgets, row and token limits)
bool decode_fused_fits(int T, int k, int E, int H, int I, int xdt, int wdt);
hipError_t launch_decode_gate_up(const DecodeArgs& d, hipStream_t st);
hipError_t launch_decode_down_combine(const DecodeArgs& d, hipStream_t st);

struct GemmArgs {
  int wdt, xdt;
  int S, T, k, H, I;
  const void* w_gu;
  const void* s_gu;
  const void* w_d;
  const void* s_d;
  const void* x;        // [T, H] bf16 or fp32
  void* xb;             // [T, H] bf16 scratch: fp32 activations rounded once for the matrix cores
  const int32_t* perm;
  const int32_t* off;
  void* a;              // [T*k, I] bf16 (mode A); unused in mode B, which writes aq/as directly
  float* y;             // [T*k, H] fp32
  // mode B: E4M3 codes and E8M0 scales (per row and 32 K) of x and a
  uint8_t* xq;          // [T, H]
  uint8_t* xs;          // [T, H/32]
  uint8_t* aq;          // [T*k, I]
  uint8_t* as;          // [T*k, I/32]
  int4* tiles_gu;       // tile lists written by the scheduler: {slot, first row, rows, n tile}
  int4* tiles_dn;
  int32_t* counts;      // [16]: tiles per XCD of the gate/up GEMM, then of the down GEMM
  bool tiles_contiguous;  // deal the tiles in (slot, M tile, N tile) order in eight runs
  int asplit;             // mode A: 1 = a in bf16; 2 = a as a bf16 (hi, lo) pair, rows of 2I values
};
size_t gemm_tiles_max(int T, int k, int S, int nt);
// entries of a GEMM's tile list (eight per-XCD lists of gemm_tile_slots / 8) = its launch grid
size_t gemm_tile_slots(int T, int k, int S, int nt);
int gemm_nt_gate_up(int I);
int gemm_nt_down(int H);
hipError_t launch_gemm_schedule(const GemmArgs& g, hipStream_t st);
hipError_t launch_gemm_gate_up(const GemmArgs& g, hipStream_t st);
hipError_t launch_gemm_down(const GemmArgs& g, hipStream_t st);
// mode B (FP8 / MXFP4 weights, quantised activations xq/xs and aq/as)
hipError_t launch_gemm_gate_up_q(const GemmArgs& g, hipStream_t st);
hipError_t launch_gemm_down_q(const GemmArgs& g, hipStream_t st);

// Mode B activation quantisation of `rows` rows of K elements (K % 32 == 0): per 32 consecutive
// elements an E8M0 scale 2^X, X = floor(log2 amax) - 8 (0 for an all-zero block), and E4M3 codes
// of v / 2^X (nearest even, saturating at +-448).  Writes codes [rows][K] and scales
// [rows][K/32] when non-null, and the dequantised values (code * 2^X, exact) to deq (bf16 or
// fp32, may alias an fp32 input) when non-null.  Rows at or beyond *nrows (when given) are skipped.
hipError_t launch_act_quant(const void* in, int in_dt, int rows, int K, const int32_t* nrows, uint8_t* codes,
                            uint8_t* scales, void* deq, int deq_dt, hipStream_t st);

hipError_t launch_combine(const float* y, const int32_t* inv, const float* y_b, const int32_t* inv_b,
                          const float* w, int T, int k, int H, void* out, int odt, hipStream_t st);

// hot-set placement (plan.hip)
hipError_t launch_accumulate_counts(const int32_t* counts, int E, int64_t* hist, hipStream_t st);
hipError_t launch_plan_slots(const int64_t* hist, int E, int S, int32_t* slot_map, hipStream_t st);
hipError_t launch_refill(const int32_t* counts, int E, int S, long long step, int32_t* slot_map,
                         int32_t* slot_expert, int64_t* last_use, int2* plan, int32_t* nplan,
                         const uint8_t* const src[4], uint8_t* const dst[4], const size_t bytes[4], hipStream_t st);

}  // namespace moe
