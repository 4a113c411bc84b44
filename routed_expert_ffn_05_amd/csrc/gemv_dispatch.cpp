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

}  // namespace moe
