// Wavefront-per-token top-k selection with scores and renormalised gates.
#pragma once
#include "common.h"

namespace moe {

// One wave selects the k experts of one token from its E logits (lane l holds logits
// l, l+64, ...; E <= 64*VPL).  Selection order: logit descending, expert id ascending.  Scores:
// softmax over all E (score == 0) or the logistic sigmoid; gates renormalised over the k chosen
// scores when renorm != 0.  Lane j < k returns the j-th expert and its gate.
template <int VPL>
__device__ __forceinline__ void topk_wave(const float* __restrict__ lrow, const float* __restrict__ bias,
                                          int E, int k, int score, int renorm, int& my_e, float& my_w) {
  const int lane = threadIdx.x & 63;
  const float NEG = -__builtin_huge_valf();
  // every load is issued before the first use (indices clamped, lanes past E masked afterwards)
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) v[i] = lrow[min(lane + 64 * i, E - 1)];
  if (bias) {
    float b[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) b[i] = bias[min(lane + 64 * i, E - 1)];
#pragma unroll
    for (int i = 0; i < VPL; ++i) v[i] += b[i];
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i) v[i] = lane + 64 * i < E ? v[i] : NEG;
  float mx = 0.0f, z = 1.0f;
  if (score == 0) {  // softmax statistics over all E
    float m = NEG;
#pragma unroll
    for (int i = 0; i < VPL; ++i) m = fmaxf(m, v[i]);
    mx = wave_max_all(m);
    float zs = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) zs += expf(v[i] - mx);
    z = wave_total(zs);
  }
  unsigned taken = 0;  // bit i: v[i] already selected
  float my_s = 0.0f, ssum = 0.0f;
  my_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = NEG;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      const bool better = (v[i] > bv) | ((v[i] == bv) & (e < bi));
      const bool ok = (e < E) & !((taken >> i) & 1u) & better;
      bv = ok ? v[i] : bv;
      bi = ok ? e : bi;
    }
    wave_argmax(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    const float s = (score == 0) ? expf(bv - mx) / z : 1.0f / (1.0f + expf(-bv));
    ssum += s;  // ascending j, the same on every lane
    if (lane == j) {
      my_s = s;
      my_e = bi;
    }
  }
  my_w = renorm ? my_s / ssum : my_s;
}

}  // namespace moe
