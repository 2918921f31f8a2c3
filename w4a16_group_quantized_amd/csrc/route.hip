// Router: softmax over E expert logits, top-k, renormalised weights.
//
// One 64-lane wavefront per token.  Lane l holds logits l, l+64, ... in
// registers; each of the top_k rounds takes every lane's best remaining logit
// and reduces it across the wave with a butterfly on (value, index) pairs,
// ordered by value descending and index ascending, so ties go to the lower
// expert index and every lane ends the round with the same winner.  The
// renormalised weights exp(l_j - l_0) / sum_j' exp(l_j' - l_0) equal the
// renormalised softmax probabilities (the full-softmax denominator cancels).
// Geometry source: the 512-expert top-10 routed experts of "[Model][SM70]
// Adapt Qwen3.8 Flash Next NVFP4", section "Implemented route".
#include <float.h>
#include <limits.h>
#include <math.h>

#include "common.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <int NPL>  // logits per lane; E <= 64 * NPL
__global__ __launch_bounds__(64 * kWavesPerBlock) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int top_k,
    int* __restrict__ ids, float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* row = logits + static_cast<size_t>(t) * E;

  float v[NPL];
  uint64_t taken = 0;  // bit i set: element lane + 64 i is taken or absent
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      v[i] = row[e];
    } else {
      v[i] = -INFINITY;
      taken |= 1ull << i;
    }
  }

  float mine = 0.f;  // lane j keeps the logit chosen in round j
  float top = 0.f;   // logit of rank 0
  for (int j = 0; j < top_k; ++j) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + 64 * i;
      if (!((taken >> i) & 1ull) && ranks_before(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ranks_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi != INT_MAX && (bi & 63) == lane) taken |= 1ull << (bi >> 6);
    if (j == 0) top = bv;
    if (lane == j) {
      mine = bv;
      ids[static_cast<size_t>(t) * top_k + j] = bi;
    }
  }

  const float num = (lane < top_k) ? expf(mine - top) : 0.f;
  float den = num;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off, 64);
  if (lane < top_k) weights[static_cast<size_t>(t) * top_k + lane] = num / den;
}

template <int NPL>
void launch_npl(const float* logits, int T, int E, int top_k, int* ids,
                float* weights, hipStream_t stream) {
  const int blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(route_topk_kernel<NPL>, dim3(blocks), dim3(64 * kWavesPerBlock), 0,
                     stream, logits, T, E, top_k, ids, weights);
}

}  // namespace

void launch_route(const float* logits, int T, int E, int top_k, int* ids,
                  float* weights, hipStream_t stream) {
  if (E <= 64)
    launch_npl<1>(logits, T, E, top_k, ids, weights, stream);
  else if (E <= 128)
    launch_npl<2>(logits, T, E, top_k, ids, weights, stream);
  else if (E <= 256)
    launch_npl<4>(logits, T, E, top_k, ids, weights, stream);
  else if (E <= 512)
    launch_npl<8>(logits, T, E, top_k, ids, weights, stream);
  else if (E <= 1024)
    launch_npl<16>(logits, T, E, top_k, ids, weights, stream);
  else if (E <= 2048)
    launch_npl<32>(logits, T, E, top_k, ids, weights, stream);
  else
    launch_npl<64>(logits, T, E, top_k, ids, weights, stream);
}

}  // namespace moe
