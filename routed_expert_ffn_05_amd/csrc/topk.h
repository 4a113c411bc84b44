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
  // Selection key per value: orderable logit bits (high word; -0 taken as +0), inverted expert id
  // (low word), so the unsigned maximum is the largest logit with the smallest id.  A selected or
  // absent value gets key 0, below every real key.
  uint64_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    const uint32_t b = __float_as_uint(v[i] + 0.0f);
    const uint32_t h = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    key[i] = e < E ? ((uint64_t(h) << 32) | uint32_t(~e)) : 0ull;
  }
  float my_l = 0.0f;
  my_e = 0;
  for (int j = 0; j < k; ++j) {
    // the lane's best key by a pairwise tree (log2 VPL dependent steps)
    uint64_t b[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) b[i] = key[i];
#pragma unroll
    for (int w = 1; w < VPL; w *= 2)
#pragma unroll
      for (int i = 0; i + w < VPL; i += 2 * w) b[i] = b[i + w] > b[i] ? b[i + w] : b[i];
    const uint64_t best = b[0];
    // the largest logit over the wave (high words); its lane, or among equal logits the smallest id
    const uint32_t bh = uint32_t(best >> 32);
    const uint32_t h = wave_max_u32(bh);
    const unsigned long long tie = __ballot(bh == h);
    int e;
    if (__popcll(tie) == 1) {
      e = int(~uint32_t(__builtin_amdgcn_readlane(int(uint32_t(best)), __ffsll((long long)tie) - 1)));
    } else {
      e = int(~wave_max_u32(bh == h ? uint32_t(best) : 0u));
    }
    const float l = __uint_as_float((h & 0x80000000u) ? (h & 0x7FFFFFFFu) : ~h);
    // the winner's key leaves the race (selects, no branch)
    const bool mine = (e & 63) == lane;
    const int col = e >> 6;
#pragma unroll
    for (int i = 0; i < VPL; ++i) key[i] = (mine && i == col) ? 0ull : key[i];
    my_l = lane == j ? l : my_l;
    my_e = lane == j ? e : my_e;
  }
  // scores of the k chosen (lane j holds the j-th), gates renormalised in ascending j
  const float my_s = (score == 0) ? expf(my_l - mx) / z : 1.0f / (1.0f + expf(-my_l));
  float ssum = 0.0f;
  for (int j = 0; j < k; ++j) ssum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), j));
  my_w = renorm ? my_s / ssum : my_s;
}

}  // namespace moe
