// Router building blocks shared by the router kernel and the fused small-T
// router + permutation kernel (internal; not part of the public ABI).
//
// A logit becomes a 64-bit key: its order-preserving bit pattern (with -0
// folded onto +0) above the inverted expert index, so the largest key is the
// largest logit and, among equal logits, the lowest expert index.
#pragma once

#include <math.h>

#include "common.h"

namespace moe {

__device__ __forceinline__ uint64_t logit_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;   // -0 ranks with +0
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
}

__device__ __forceinline__ float key_logit(uint64_t k) {
  const uint32_t ord = static_cast<uint32_t>(k >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

__device__ __forceinline__ int key_expert(uint64_t k) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(k));
}

__device__ __forceinline__ uint64_t max64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t x) {
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(x >> 32), CTRL, 0xF, 0xF, false);
  return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

// Maximum over the wave, returned in every lane.  The row swaps hand each lane
// its partner 16 (32) lanes away in one of their two results, and the other
// result is the lane's own value, so the maximum of all three is the pair's.
__device__ __forceinline__ uint64_t wave_max(uint64_t k) {
  k = max64(k, dpp64<0xB1>(k));    // quad_perm [1,0,3,2]
  k = max64(k, dpp64<0x4E>(k));    // quad_perm [2,3,0,1]
  k = max64(k, dpp64<0x141>(k));   // row_half_mirror
  k = max64(k, dpp64<0x140>(k));   // row_mirror
  {
    const uint32_t lo = static_cast<uint32_t>(k), hi = static_cast<uint32_t>(k >> 32);
    const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    k = max64(k, max64((static_cast<uint64_t>(h[0]) << 32) | l[0], (static_cast<uint64_t>(h[1]) << 32) | l[1]));
  }
  {
    const uint32_t lo = static_cast<uint32_t>(k), hi = static_cast<uint32_t>(k >> 32);
    const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    k = max64(k, max64((static_cast<uint64_t>(h[0]) << 32) | l[0], (static_cast<uint64_t>(h[1]) << 32) | l[1]));
  }
  return k;
}

// Maximum of a 32-bit value over the wave, in every lane: DPP within rows of
// 16 lanes, then the row swaps (each hands a lane its partner 16 or 32 lanes
// away in one of its two results, the lane's own value in the other).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x140, 0xF, 0xF, false)));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(v, max(a[0], a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(v, max(b[0], b[1]));
}

// Top-k of one token's E logits (`row`) by one wave: lane l holds the keys of
// experts l, l + 64, ..., sorted once in descending order; each of the top_k
// rounds takes the wave maximum of the lanes' first keys and the winning lane
// drops its first key.  The wave maximum of a 64-bit key is taken in two
// 32-bit passes (upper word, then the lower word among the lanes that hold
// the maximal upper word), which is the same maximum.  Lane j < top_k ends
// with the expert and logit of rank j; every lane gets the logit of rank 0.
template <int NPL>  // logits per lane; E <= 64 * NPL, NPL a power of two
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int top_k,
                                          int& my_id, float& my_logit, float& top_logit) {
  const int lane = threadIdx.x & 63;
  uint64_t key[NPL];  // 0: absent or taken (every real key is larger)
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? logit_key(row[e], e) : 0ull;
  }
  // bitonic sort, descending
#pragma unroll
  for (int size = 2; size <= NPL; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          const bool desc = (i & size) == 0;
          const uint64_t a = key[i], b = key[j];
          const bool swap = desc ? a < b : a > b;
          key[i] = swap ? b : a;
          key[j] = swap ? a : b;
        }
      }
  my_id = -1;
  my_logit = 0.f;
  top_logit = 0.f;
  for (int j = 0; j < top_k; ++j) {
    const uint32_t hi = static_cast<uint32_t>(key[0] >> 32), lo = static_cast<uint32_t>(key[0]);
    const uint32_t mhi = wave_max_u32(hi);
    // lanes holding the largest value: almost always one, whose index word
    // is then read directly; equal values take the maximum of the index
    // words among them (the lowest expert)
    const uint64_t cand = __ballot(hi == mhi);
    uint32_t mlo;
    if (__popcll(cand) == 1)
      mlo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lo), __ffsll(static_cast<long long>(cand)) - 1));
    else
      mlo = wave_max_u32(hi == mhi ? lo : 0u);
    const uint64_t best = (static_cast<uint64_t>(mhi) << 32) | mlo;
    // the winning lane drops its first key (written with masks: as selects the
    // compiler turns the shift into an indexed pick over all slots)
    const uint64_t m = key[0] == best ? ~0ull : 0ull;
#pragma unroll
    for (int i = 0; i + 1 < NPL; ++i) key[i] = (key[i + 1] & m) | (key[i] & ~m);
    key[NPL - 1] &= ~m;
    const int e = key_expert(best);
    const float v = key_logit(best);
    if (j == 0) top_logit = v;
    if (lane == j) {
      my_id = e;
      my_logit = v;
    }
  }
}

// Renormalised weight of the lane's rank: exp(l_j - l_0) / sum_j' exp(l_j' -
// l_0) over the top_k ranks (the full-softmax denominator cancels).  Called
// by all 64 lanes; meaningful in lanes j < top_k.
__device__ __forceinline__ float wave_topk_weight(float my_logit, float top_logit, int top_k) {
  const int lane = threadIdx.x & 63;
  const float num = (lane < top_k) ? expf(my_logit - top_logit) : 0.f;
  float den = num;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off, 64);
  return num / den;
}

}  // namespace moe
