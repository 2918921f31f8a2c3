// Router: softmax over E expert logits, top-k, renormalised weights.
//
// One 64-lane wavefront per token.  Each logit becomes a 64-bit key: its
// order-preserving bit pattern (with -0 folded onto +0) above the inverted
// expert index, so the largest key is the largest logit and, among equal
// logits, the lowest expert index.  Lane l holds the keys of experts l,
// l + 64, ...; each of the top_k rounds takes the wave maximum of the lanes'
// best keys (DPP within rows of 16 lanes, then v_permlane16/32_swap across
// rows, all plain vector operations) and clears the winner.  The renormalised
// weights exp(l_j - l_0) / sum_j' exp(l_j' - l_0) equal the renormalised
// softmax probabilities (the full-softmax denominator cancels).  Geometry
// source: the 512-expert top-10 routed experts of "[Model][SM70] Adapt
// Qwen3.8 Flash Next NVFP4", section "Implemented route".
//
// With a shared expert (`shared` = 1) each token's row of ids and weights has
// top_k + 1 entries, the last one the shared expert E with weight 1: it takes
// part in the permutation, the FFN and the combine like a routed choice.
#include <math.h>

#include "route.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

template <int NPL>  // logits per lane; E <= 64 * NPL
__global__ __launch_bounds__(64 * kWavesPerBlock) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int top_k, int shared,
    int* __restrict__ ids, float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  int id;
  float logit, top;
  wave_topk<NPL>(logits + static_cast<size_t>(t) * E, E, top_k, id, logit, top);
  const float w = wave_topk_weight(logit, top, top_k);
  const int kk = top_k + shared;
  if (lane < kk) {
    const bool sh = lane == top_k;  // only when shared
    ids[static_cast<size_t>(t) * kk + lane] = sh ? E : id;
    weights[static_cast<size_t>(t) * kk + lane] = sh ? 1.f : w;
  }
}

template <int NPL>
void launch_npl(const float* logits, int T, int E, int top_k, int shared, int* ids,
                float* weights, hipStream_t stream) {
  const int blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(route_topk_kernel<NPL>, dim3(blocks), dim3(64 * kWavesPerBlock), 0,
                     stream, logits, T, E, top_k, shared, ids, weights);
}

}  // namespace

void launch_route(const float* logits, int T, int E, int top_k, int shared, int* ids,
                  float* weights, hipStream_t stream) {
  if (E <= 64)
    launch_npl<1>(logits, T, E, top_k, shared, ids, weights, stream);
  else if (E <= 128)
    launch_npl<2>(logits, T, E, top_k, shared, ids, weights, stream);
  else if (E <= 256)
    launch_npl<4>(logits, T, E, top_k, shared, ids, weights, stream);
  else if (E <= 512)
    launch_npl<8>(logits, T, E, top_k, shared, ids, weights, stream);
  else if (E <= 1024)
    launch_npl<16>(logits, T, E, top_k, shared, ids, weights, stream);
  else if (E <= 2048)
    launch_npl<32>(logits, T, E, top_k, shared, ids, weights, stream);
  else
    launch_npl<64>(logits, T, E, top_k, shared, ids, weights, stream);
}

}  // namespace moe
