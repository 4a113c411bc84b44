// Wavefront-per-token top-k selection with scores and renormalised gates.
#pragma once
#include "common.h"

namespace moe {

// Fast selection of up to 8 of at most 512 values (below).  Each value gets a 32-bit short key:
// its orderable logit bits with the low 9 bits cleared, and in those 9 bits the inverted expert
// id, so short keys are distinct and ordered by (rounded-down logit, id).  Each lane sorts its
// short keys, then sorted lists of 8 are merged across lanes: two sorted lists A and B
// (descending) give their 8 largest keys as the bitonic sequence max(A[i], B[7 - i]), sorted by
// three half-cleaner levels.  Six merges, each with a partner lane in the other half of an
// aligned group of 2, 4, 8, 16, 32 and 64 lanes (DPP quad permutations, the half-row and row
// mirrors, then the row and half-wave swaps), leave the wave's 8 largest short keys, in order, in
// every lane.  Rounding down never reverses two logits, only merges them, so the list
// is the exact selection in the exact order when no two of its entries share a rounded logit and
// no value outside it shares the last entry's; otherwise the exact rounds decide.
constexpr uint32_t kShortIdBits = 9;
constexpr uint32_t kShortIdMask = (1u << kShortIdBits) - 1u;

// descending compare-exchange: a takes the larger key
__device__ __forceinline__ void skey_ce(uint32_t& a, uint32_t& b) {
  const uint32_t hi = max(a, b), lo = min(a, b);
  a = hi;
  b = lo;
}

// sorts a bitonic sequence of 8 keys descending (three half-cleaner levels)
__device__ __forceinline__ void skey_clean8(uint32_t (&a)[8]) {
#pragma unroll
  for (int stride = 4; stride > 0; stride >>= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i ^ stride) > i) skey_ce(a[i], a[i ^ stride]);
}

// bitonic sort of 8 keys, descending
__device__ __forceinline__ void skey_sort8(uint32_t (&a)[8]) {
#pragma unroll
  for (int size = 2; size <= 8; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          if ((i & size) == 0)
            skey_ce(a[i], a[j]);
          else
            skey_ce(a[j], a[i]);
        }
      }
}

// merge with the list of the partner lane given by an in-row DPP permutation (an involution)
template <int CTRL>
__device__ __forceinline__ void skey_merge_dpp(uint32_t (&c)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t pi = uint32_t(dpp_src_or<CTRL>(0, int(c[i])));
    const uint32_t pj = uint32_t(dpp_src_or<CTRL>(0, int(c[7 - i])));
    c[i] = max(c[i], pj);
    c[7 - i] = max(c[7 - i], pi);
  }
  skey_clean8(c);
}

// merge the lists of paired 16-lane rows (ROWS = 16) or 32-lane halves (ROWS = 32): the swap gives
// every lane both lists of its pair
template <int ROWS>
__device__ __forceinline__ void skey_merge_swap(uint32_t (&c)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (ROWS == 16) {
      const auto si = __builtin_amdgcn_permlane16_swap(c[i], c[i], false, false);
      const auto sj = __builtin_amdgcn_permlane16_swap(c[7 - i], c[7 - i], false, false);
      c[i] = max(uint32_t(si[0]), uint32_t(sj[1]));
      c[7 - i] = max(uint32_t(sj[0]), uint32_t(si[1]));
    } else {
      const auto si = __builtin_amdgcn_permlane32_swap(c[i], c[i], false, false);
      const auto sj = __builtin_amdgcn_permlane32_swap(c[7 - i], c[7 - i], false, false);
      c[i] = max(uint32_t(si[0]), uint32_t(sj[1]));
      c[7 - i] = max(uint32_t(sj[0]), uint32_t(si[1]));
    }
  }
  skey_clean8(c);
}

// the wave's 8 largest short keys, descending, in every lane (all 64 lanes active, VPL <= 8)
template <int VPL>
__device__ __forceinline__ void wave_top8_short(const uint32_t (&key)[VPL], uint32_t (&c)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = i < VPL ? key[i] : 0u;
  skey_sort8(c);
  skey_merge_dpp<0xB1>(c);   // quad_perm [1,0,3,2]: the other lane of each pair
  skey_merge_dpp<0x4E>(c);   // quad_perm [2,3,0,1]: the other pair of each quad
  skey_merge_dpp<0x141>(c);  // row_half_mirror: the other quad of each 8 lanes
  skey_merge_dpp<0x140>(c);  // row_mirror: the other 8 lanes of each row
  skey_merge_swap<16>(c);
  skey_merge_swap<32>(c);
}

// One wave selects the k experts of one token from its E logits (lane l holds logits
// l, l+64, ...; E <= 64*VPL).  Selection order: logit descending, expert id ascending.  Scores:
// softmax over all E (score == 0) or the logistic sigmoid; gates renormalised over the k chosen
// scores when renorm != 0.  Lane j < k returns the j-th expert and its gate.  With k <= 8 and
// E <= 512 the short-key merge selects when its exactness test passes; otherwise k rounds each take
// the wave's largest remaining key.  Both give the same experts in the same order.
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
  bool exact = false;
  if constexpr (VPL <= 8) {
    if (k <= 8) {
      uint32_t sk[VPL];
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        sk[i] = key[i] ? ((uint32_t(key[i] >> 32) & ~kShortIdMask) | (uint32_t(key[i]) & kShortIdMask)) : 0u;
      uint32_t c[8];
      wave_top8_short<VPL>(sk, c);
      // exact when the values whose rounded logit reaches the last entry's are exactly the 8
      // listed and no two listed share a rounded logit
      const uint32_t floor7 = c[7] & ~kShortIdMask;
      int reach = 0;
#pragma unroll
      for (int i = 0; i < VPL; ++i) reach += __popcll(__ballot(sk[i] >= floor7));
      bool distinct = true;
#pragma unroll
      for (int j = 0; j < 7; ++j) distinct = distinct && (c[j] & ~kShortIdMask) != (c[j + 1] & ~kShortIdMask);
      exact = __builtin_amdgcn_readfirstlane(int(floor7 != 0u && reach == 8 && distinct)) != 0;  // the same in every lane
      if (exact) {
        uint32_t mk = c[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mk = lane == j ? c[j] : mk;
        const int e = int(~mk & kShortIdMask);
        // the chosen value's own logit, from lane e % 64, column e / 64
        const int src = (e & 63) << 2;
        float l = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
          const float x = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(v[i])));
          l = (e >> 6) == i ? x : l;
        }
        if (lane < k) {
          my_l = l + 0.0f;
          my_e = e;
        }
      }
    }
  }
  for (int j = 0; !exact && j < k; ++j) {
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
