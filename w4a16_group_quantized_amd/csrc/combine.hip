// Router-weighted combine back to token order:
//   out[t, h] = fp16_rne( sum_{j ascending} w[t, j] * y_sorted[slot_rows[t*k + j], h] )
// A gather with fp32 accumulation in a fixed order (no atomics), so the result
// does not depend on scheduling.  Each thread produces 4 consecutive h values
// from 16-byte loads of the k selected fp32 rows, taken kChunk at a time: the
// chunk's row indices and weights are loaded together, then all its row
// loads are issued, then they are summed in order, so a token costs two
// round trips per chunk instead of two per selected row.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 16;  // selected rows whose loads are in flight together

__global__ __launch_bounds__(kThreads) void combine_kernel(
    const float* __restrict__ y_sorted, const float* __restrict__ weights,
    const int* __restrict__ slot_rows, int top_k, int H, int blocks_per_token,
    uint16_t* __restrict__ out) {
  const int t = blockIdx.x / blocks_per_token;
  const int h4 = (blockIdx.x - t * blocks_per_token) * kThreads + threadIdx.x;  // 4-wide chunk
  if (h4 * 4 >= H) return;
  const size_t slot0 = static_cast<size_t>(t) * top_k;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < top_k; j0 += kChunk) {
    const int n = min(kChunk, top_k - j0);
    // Branch-free: past the chunk's n rows the index repeats its last row (a
    // load already in flight) and the term is skipped by a select.
    int r[kChunk];
    float w[kChunk];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const size_t sl = slot0 + j0 + min(j, n - 1);
      r[j] = slot_rows[sl];
      w[j] = weights[sl];
    }
    float4 y[kChunk];
#pragma unroll
    for (int j = 0; j < kChunk; ++j)
      y[j] = *reinterpret_cast<const float4*>(y_sorted + static_cast<size_t>(r[j]) * H + 4 * h4);
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {  // j ascending, as before: the same sum bit for bit
      const bool on = j < n;
      acc.x = on ? fmaf(w[j], y[j].x, acc.x) : acc.x;
      acc.y = on ? fmaf(w[j], y[j].y, acc.y) : acc.y;
      acc.z = on ? fmaf(w[j], y[j].z, acc.z) : acc.z;
      acc.w = on ? fmaf(w[j], y[j].w, acc.w) : acc.w;
    }
  }
  uint2 packed;
  packed.x = static_cast<uint32_t>(float_to_half_bits(acc.x)) |
             (static_cast<uint32_t>(float_to_half_bits(acc.y)) << 16);
  packed.y = static_cast<uint32_t>(float_to_half_bits(acc.z)) |
             (static_cast<uint32_t>(float_to_half_bits(acc.w)) << 16);
  *reinterpret_cast<uint2*>(out + static_cast<size_t>(t) * H + 4 * h4) = packed;
}

}  // namespace

void launch_combine(const float* y_sorted, const float* weights, const int* slot_rows, int T,
                    int top_k, int H, uint16_t* out, hipStream_t stream) {
  const int chunks = H / 4;
  const int bpt = (chunks + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>(T) * bpt), dim3(kThreads), 0,
                     stream, y_sorted, weights, slot_rows, top_k, H, bpt, out);
}

}  // namespace moe
