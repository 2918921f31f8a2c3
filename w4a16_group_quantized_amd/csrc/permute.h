// Permutation building blocks shared by the permutation kernels and the
// fused small-T router + permutation kernel (internal; not part of the public
// ABI): block-wide exclusive scans over 1024 threads and the offsets /
// active-list writer.
#pragma once

#include "common.h"

namespace moe {

constexpr int kScanThreads = 1024;
constexpr int kPerThread = kMaxExperts / kScanThreads;  // experts per thread in scans
static_assert(kPerThread * kScanThreads == kMaxExperts, "scan covers kMaxExperts");

// Exclusive prefix sum across the block of a per-thread value; `wave_tot` is
// LDS of at least kScanThreads / 64 + 1 ints.  Returns this thread's exclusive
// prefix and sets `total`.
__device__ inline int block_exclusive_scan(int value, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int kWaves = kScanThreads / 64;
  int inc = value;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int w = (lane < kWaves) ? wave_tot[lane] : 0;
    int winc = w;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(winc, d, 64);
      if (lane >= d) winc += o;
    }
    if (lane < kWaves) wave_tot[lane] = winc - w;
    if (lane == kWaves - 1) wave_tot[kWaves] = winc;
  }
  __syncthreads();
  const int excl = wave_tot[wave] + inc - value;
  total = wave_tot[kWaves];
  __syncthreads();  // wave_tot may be reused by the caller
  return excl;
}

// Given per-expert row counts (thread owns experts kPerThread*tid + i), write
// offsets[0..E], active[0..E) (-1 padded) and num_active; also return each
// owned expert's offset in `off`.
__device__ inline void write_offsets_and_active(const int (&cnt)[kPerThread], int E, int S,
                                         int* __restrict__ offsets, int* __restrict__ active,
                                         int* __restrict__ num_active, int* wave_tot,
                                         int (&off)[kPerThread]) {
  const int tid = threadIdx.x;
  int csum = 0, fsum = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    csum += cnt[i];
    fsum += cnt[i] > 0;
  }
  int ctot, ftot;
  int cpre = block_exclusive_scan(csum, wave_tot, ctot);
  int fpre = block_exclusive_scan(fsum, wave_tot, ftot);
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int e = kPerThread * tid + i;
    off[i] = cpre;
    if (e < E) {
      offsets[e] = cpre;
      if (cnt[i] > 0) active[fpre++] = e;
    }
    cpre += cnt[i];
  }
  for (int e = ftot + tid; e < E; e += kScanThreads) active[e] = -1;
  if (tid == 0) {
    offsets[E] = S;
    *num_active = ftot;
  }
}

}  // namespace moe
