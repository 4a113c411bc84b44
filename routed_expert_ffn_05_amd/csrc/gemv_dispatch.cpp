// Routes a GEMV launch to the translation unit compiled for the weight format.
#include "kernels.h"
#include "common.h"

namespace moe {

hipError_t launch_gemv_gate_up_f32(const GemvArgs& g, hipStream_t st);
hipError_t launch_gemv_gate_up_bf16(const GemvArgs& g, hipStream_t st);
hipError_t launch_gemv_gate_up_fp8(const GemvArgs& g, hipStream_t st);
hipError_t launch_gemv_gate_up_mxfp4(const GemvArgs& g, hipStream_t st);
hipError_t launch_gemv_down_f32(const GemvArgs& g, hipStream_t st);
hipError_t launch_gemv_down_bf16(const GemvArgs& g, hipStream_t st);
hipError_t launch_gemv_down_fp8(const GemvArgs& g, hipStream_t st);
hipError_t launch_gemv_down_mxfp4(const GemvArgs& g, hipStream_t st);
hipError_t launch_decode_gate_up_f32(const DecodeArgs& d, hipStream_t st);
hipError_t launch_decode_gate_up_bf16(const DecodeArgs& d, hipStream_t st);
hipError_t launch_decode_gate_up_fp8(const DecodeArgs& d, hipStream_t st);
hipError_t launch_decode_gate_up_mxfp4(const DecodeArgs& d, hipStream_t st);
hipError_t launch_decode_down_combine_f32(const DecodeArgs& d, hipStream_t st);
hipError_t launch_decode_down_combine_bf16(const DecodeArgs& d, hipStream_t st);
hipError_t launch_decode_down_combine_fp8(const DecodeArgs& d, hipStream_t st);
hipError_t launch_decode_down_combine_mxfp4(const DecodeArgs& d, hipStream_t st);

hipError_t launch_gemv_gate_up(const GemvArgs& g, hipStream_t st) {
  switch (g.wdt) {
    case DT_F32: return launch_gemv_gate_up_f32(g, st);
    case DT_BF16: return launch_gemv_gate_up_bf16(g, st);
    case DT_FP8: return launch_gemv_gate_up_fp8(g, st);
    case DT_MXFP4: return launch_gemv_gate_up_mxfp4(g, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_down(const GemvArgs& g, hipStream_t st) {
  switch (g.wdt) {
    case DT_F32: return launch_gemv_down_f32(g, st);
    case DT_BF16: return launch_gemv_down_bf16(g, st);
    case DT_FP8: return launch_gemv_down_fp8(g, st);
    case DT_MXFP4: return launch_gemv_down_mxfp4(g, st);
  }
  return hipErrorInvalidValue;
}

// Which batches take the two-launch decode layer.  Every wave forms its column block's sums for
// all of the batch's slots, so batches touching many slots stream better on the staged launches
// (a slot per row of work-groups); measured per step (T, k = 8): MXFP4 110 of 384 slots T=1
// 21.0 vs 25.6 us, T=2 27.8 vs 31.6; bf16 T=1 48.1 vs 50.4, T=2 78.6 vs 76.5; FP8 T=1 34.9 vs
// 36.0, T=2 55.3 vs 53.6.  Then the LDS: the T token rows and the slot map; every row of a and y.
bool decode_fused_fits(int T, int k, int E, int H, int I, int xdt, int wdt) {
  const long long rows = (long long)T * k;
  const int max_rows = wdt == DT_MXFP4 ? kDecFuseRows : kDecFuseRowsWide;
  if (T < 1 || T > kDecMaxT || k < 1 || rows > max_rows || E < 1 || E > 1024) return false;
  const size_t R = size_t(rows);
  const size_t lds_gu = size_t(T) * H * (xdt == DT_F32 ? 4 : 2) + size_t(E) * 4;
  const size_t lds_dn = R * I * 4 + R * kDecRB * 4;
  return lds_gu <= 96 * 1024 && lds_dn <= 144 * 1024;
}

hipError_t launch_decode_gate_up(const DecodeArgs& d, hipStream_t st) {
  switch (d.wdt) {
    case DT_F32: return launch_decode_gate_up_f32(d, st);
    case DT_BF16: return launch_decode_gate_up_bf16(d, st);
    case DT_FP8: return launch_decode_gate_up_fp8(d, st);
    case DT_MXFP4: return launch_decode_gate_up_mxfp4(d, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_down_combine(const DecodeArgs& d, hipStream_t st) {
  switch (d.wdt) {
    case DT_F32: return launch_decode_down_combine_f32(d, st);
    case DT_BF16: return launch_decode_down_combine_bf16(d, st);
    case DT_FP8: return launch_decode_down_combine_fp8(d, st);
    case DT_MXFP4: return launch_decode_down_combine_mxfp4(d, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
