// Decode GEMVs for fp8 expert weights (see gemv_impl.h).
#define MOE_GEMV_WD moe::DT_FP8
#include "gemv_impl.h"

namespace moe {

hipError_t launch_gemv_gate_up_fp8(const GemvArgs& g, hipStream_t st) {
  return g.xdt == DT_F32 ? gemv::gate_up_dispatch<DT_FP8, DT_F32>(g, st) : gemv::gate_up_dispatch<DT_FP8, DT_BF16>(g, st);
}

hipError_t launch_gemv_down_fp8(const GemvArgs& g, hipStream_t st) { return gemv::down_dispatch<DT_FP8>(g, st); }

hipError_t launch_decode_gate_up_fp8(const DecodeArgs& d, hipStream_t st) {
  return d.xdt == DT_F32 ? gemv::decode_gate_up_dispatch<DT_FP8, DT_F32>(d, st)
                         : gemv::decode_gate_up_dispatch<DT_FP8, DT_BF16>(d, st);
}

hipError_t launch_decode_down_combine_fp8(const DecodeArgs& d, hipStream_t st) {
  return gemv::decode_down_dispatch<DT_FP8>(d, st);
}

}  // namespace moe
