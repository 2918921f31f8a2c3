// Router and permutation in one launch for small token counts (decode): the
// same results as the router kernel followed by the single-workgroup
// permutation, bit for bit, from one workgroup of 1024 threads.  Saves a
// launch and the round trip of the expert ids through global memory on the
// decode path, where both kernels are latency-bound ("[Perf][SM70] Narrow
// Qwen3.8 AWQ active grouped decode", section "Purpose": the active-expert
// segments and offsets; routing of "[Model][SM70] Adapt Qwen3.8 Flash Next
// NVFP4", section "Implemented route").
//
// The 16 waves route tokens t = wave, wave + 16, ...; the lane holding rank j
// of token t writes the id and weight, keeps the id in LDS, and sets bit t of
// the chosen expert's 64-bit mask (LDS atomic OR, independent of order).
// After a barrier the masks give the counts, the scans give the offsets and
// the active list, and each slot's sorted row is its expert's offset plus the
// number of earlier tokens in the mask, exactly as in the permutation kernel.
// With a shared expert (`shared` = 1) slot top_k of every token is expert E
// with weight 1 (as the router kernel writes it), and the permutation runs
// over E + 1 experts.
#include "permute.h"
#include "route.h"

namespace moe {
namespace {

constexpr int kFusedMaxE = 1024;                 // experts: 16 logits per lane at most
constexpr int kFusedMaxSlots = kPermBlockTokens * (kMaxTopK + 1);

template <int NPL>
__global__ __launch_bounds__(kScanThreads) void route_permute_small_kernel(
    const float* __restrict__ logits, int T, int E, int top_k, int shared, int* __restrict__ ids,
    float* __restrict__ weights, int* __restrict__ offsets, int* __restrict__ sorted_slots,
    int* __restrict__ slot_rows, int* __restrict__ active, int* __restrict__ num_active) {
  __shared__ unsigned long long masks[kFusedMaxE];
  __shared__ int seg[kFusedMaxE];
  __shared__ unsigned short slot_id[kFusedMaxSlots];
  __shared__ int wave_tot[kScanThreads / 64 + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int kk = top_k + shared;  // slots per token
  const int EP = E + shared;      // experts of the permutation
  const int S = T * kk;
  for (int e = tid; e < EP; e += kScanThreads) masks[e] = 0ull;
  __syncthreads();

  for (int t = tid >> 6; t < T; t += kScanThreads / 64) {
    int id;
    float logit, top;
    wave_topk<NPL>(logits + static_cast<size_t>(t) * E, E, top_k, id, logit, top);
    const float w = wave_topk_weight(logit, top, top_k);
    if (lane < kk) {
      const bool sh = lane == top_k;  // only when shared
      const int s = t * kk + lane;
      const int e = sh ? E : id;
      ids[s] = e;
      weights[s] = sh ? 1.f : w;
      slot_id[s] = static_cast<unsigned short>(e);
      atomicOr(&masks[e], 1ull << t);
    }
  }
  __syncthreads();

  int cnt[kPerThread], off[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int e = kPerThread * tid + i;
    cnt[i] = (e < EP) ? __popcll(masks[e]) : 0;
  }
  write_offsets_and_active(cnt, EP, S, offsets, active, num_active, wave_tot, off);
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int e = kPerThread * tid + i;
    if (e < EP) seg[e] = off[i];
  }
  __syncthreads();
  for (int s = tid; s < S; s += kScanThreads) {
    const int t = s / kk;
    const int e = slot_id[s];
    const int r = seg[e] + __popcll(masks[e] & ((1ull << t) - 1ull));
    sorted_slots[r] = s;
    slot_rows[s] = r;
  }
}

template <int NPL>
void launch_fused(const float* logits, int T, int E, int top_k, int shared, int* ids,
                  float* weights, int* offsets, int* sorted_slots, int* slot_rows, int* active,
                  int* num_active, hipStream_t stream) {
  hipLaunchKernelGGL(route_permute_small_kernel<NPL>, dim3(1), dim3(kScanThreads), 0, stream,
                     logits, T, E, top_k, shared, ids, weights, offsets, sorted_slots, slot_rows,
                     active, num_active);
}

}  // namespace

void launch_route_permute(const float* logits, int T, int E, int top_k, int shared, int* ids,
                          float* weights, int* offsets, int* sorted_slots, int* slot_rows,
                          int* active, int* num_active, void* workspace, bool one_launch,
                          hipStream_t stream) {
  if (!one_launch) {
    launch_route(logits, T, E, top_k, shared, ids, weights, stream);
    launch_permute(ids, T, top_k + shared, E + shared, offsets, sorted_slots, slot_rows, active,
                   num_active, workspace, stream);
    return;
  }
  if (E <= 64)
    launch_fused<1>(logits, T, E, top_k, shared, ids, weights, offsets, sorted_slots, slot_rows, active,
                    num_active, stream);
  else if (E <= 128)
    launch_fused<2>(logits, T, E, top_k, shared, ids, weights, offsets, sorted_slots, slot_rows, active,
                    num_active, stream);
  else if (E <= 256)
    launch_fused<4>(logits, T, E, top_k, shared, ids, weights, offsets, sorted_slots, slot_rows, active,
                    num_active, stream);
  else if (E <= 512)
    launch_fused<8>(logits, T, E, top_k, shared, ids, weights, offsets, sorted_slots, slot_rows, active,
                    num_active, stream);
  else
    launch_fused<16>(logits, T, E, top_k, shared, ids, weights, offsets, sorted_slots, slot_rows, active,
                     num_active, stream);
}

}  // namespace moe
