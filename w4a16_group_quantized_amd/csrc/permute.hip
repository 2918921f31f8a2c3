// Token-to-expert permutation: stable counting sort of the S = T * top_k slots
// by expert, producing the per-expert segment offsets, the sorted slot list,
// its inverse, and the compact ascending list of active experts ("multi-row
// active-expert segments and offsets-based scheduling", "[Perf][SM70] Narrow
// Qwen3.8 AWQ active grouped decode", section "Purpose").
//
// Stability without order-dependent atomics.  A token picks an expert at most
// once, so within one expert's segment the slots are ordered by token.  Tokens
// are cut into blocks of 64; for each (block, expert) a 64-bit mask records
// which tokens of the block chose the expert (built with LDS atomic OR, which
// does not depend on thread order).  The sorted row of slot (t, j) with expert
// e is then
//     offsets[e] + (rows of e in earlier blocks) + popcount(mask & below(t)).
// One workgroup does everything when T <= 64 (decode); otherwise three
// kernels: masks per block, a scan over blocks and experts, and the scatter.
#include "permute.h"

namespace moe {
namespace {

// ---- T <= 64: one workgroup ------------------------------------------------
__global__ __launch_bounds__(kScanThreads) void permute_single_block_kernel(
    const int* __restrict__ ids, int T, int top_k, int E, int* __restrict__ offsets,
    int* __restrict__ sorted_slots, int* __restrict__ slot_rows, int* __restrict__ active,
    int* __restrict__ num_active) {
  __shared__ unsigned long long masks[kMaxExperts];
  __shared__ int seg[kMaxExperts];
  __shared__ int wave_tot[kScanThreads / 64 + 1];
  const int tid = threadIdx.x;
  const int S = T * top_k;
  for (int e = tid; e < E; e += kScanThreads) masks[e] = 0ull;
  __syncthreads();
  for (int s = tid; s < S; s += kScanThreads) atomicOr(&masks[ids[s]], 1ull << (s / top_k));
  __syncthreads();

  int cnt[kPerThread], off[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int e = kPerThread * tid + i;
    cnt[i] = (e < E) ? __popcll(masks[e]) : 0;
  }
  write_offsets_and_active(cnt, E, S, offsets, active, num_active, wave_tot, off);
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int e = kPerThread * tid + i;
    if (e < E) seg[e] = off[i];
  }
  __syncthreads();

  for (int s = tid; s < S; s += kScanThreads) {
    const int t = s / top_k;
    const int e = ids[s];
    const int r = seg[e] + __popcll(masks[e] & ((1ull << t) - 1ull));
    sorted_slots[r] = s;
    slot_rows[s] = r;
  }
}

// ---- T > 64: masks per 64-token block ---------------------------------------
__global__ __launch_bounds__(256) void permute_mask_kernel(
    const int* __restrict__ ids, int T, int top_k, int E,
    unsigned long long* __restrict__ gmasks, int* __restrict__ gcount) {
  __shared__ unsigned long long masks[kMaxExperts];
  const int b = blockIdx.x;
  const int t0 = b * kPermBlockTokens;
  const int nt = min(kPermBlockTokens, T - t0);
  for (int e = threadIdx.x; e < E; e += blockDim.x) masks[e] = 0ull;
  __syncthreads();
  const int* bid = ids + static_cast<size_t>(t0) * top_k;
  for (int i = threadIdx.x; i < nt * top_k; i += blockDim.x)
    atomicOr(&masks[bid[i]], 1ull << (i / top_k));
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const unsigned long long m = masks[e];
    gmasks[static_cast<size_t>(b) * E + e] = m;
    gcount[static_cast<size_t>(b) * E + e] = __popcll(m);
  }
}

// Scan over blocks (per expert, in place: counts become rows in earlier
// blocks) and over experts (offsets, active list).  With E <= kScanThreads
// every expert's blocks are split over P = kScanThreads / E threads: each
// scans its own range, the part totals meet in LDS, and a second pass adds
// the earlier parts' totals (a few round trips however many blocks, instead
// of one per 16 blocks and expert in turn).
__global__ __launch_bounds__(kScanThreads) void permute_scan_kernel(
    int nblocks, int S, int E, int* __restrict__ gcount, int* __restrict__ offsets,
    int* __restrict__ active, int* __restrict__ num_active) {
  __shared__ int wave_tot[kScanThreads / 64 + 1];
  __shared__ int part_tot[kScanThreads];
  const int tid = threadIdx.x;
  int cnt[kPerThread], off[kPerThread];
  if (E <= kScanThreads) {
    const int P = kScanThreads / E;
    const int e = tid % E, part = tid / E;
    const int b0 = part < P ? nblocks * part / P : 0;
    const int b1 = part < P ? nblocks * (part + 1) / P : 0;
    int run = 0;
    for (int bb = b0; bb < b1; bb += 16) {
      int c[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) c[u] = bb + u < b1 ? gcount[static_cast<size_t>(bb + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (bb + u < b1) gcount[static_cast<size_t>(bb + u) * E + e] = run;
        run += c[u];
      }
    }
    if (part < P) part_tot[part * E + e] = run;
    __syncthreads();
    if (part < P) {
      int base = 0;
      for (int q = 0; q < part; ++q) base += part_tot[q * E + e];
      if (base != 0)
        for (int bb = b0; bb < b1; ++bb) gcount[static_cast<size_t>(bb) * E + e] += base;
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int ee = kPerThread * tid + i;
      int tot = 0;
      if (ee < E)
        for (int q = 0; q < P; ++q) tot += part_tot[q * E + ee];
      cnt[i] = tot;
    }
    write_offsets_and_active(cnt, E, S, offsets, active, num_active, wave_tot, off);
    return;
  }
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int e = kPerThread * tid + i;
    int run = 0;
    if (e < E) {
      // 16 block counts in flight at a time, then their exclusive prefixes
      for (int b0 = 0; b0 < nblocks; b0 += 16) {
        int c[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          c[u] = b0 + u < nblocks ? gcount[static_cast<size_t>(b0 + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (b0 + u < nblocks) gcount[static_cast<size_t>(b0 + u) * E + e] = run;
          run += c[u];
        }
      }
    }
    cnt[i] = run;
  }
  write_offsets_and_active(cnt, E, S, offsets, active, num_active, wave_tot, off);
}

__global__ __launch_bounds__(256) void permute_scatter_kernel(
    const int* __restrict__ ids, int T, int top_k, int E,
    const unsigned long long* __restrict__ gmasks, const int* __restrict__ gbase,
    const int* __restrict__ offsets, int* __restrict__ sorted_slots,
    int* __restrict__ slot_rows) {
  const int b = blockIdx.x;
  const int t0 = b * kPermBlockTokens;
  const int nt = min(kPermBlockTokens, T - t0);
  const size_t s0 = static_cast<size_t>(t0) * top_k;
  for (int i = threadIdx.x; i < nt * top_k; i += blockDim.x) {
    const int s = static_cast<int>(s0) + i;
    const int e = ids[s];
    const size_t be = static_cast<size_t>(b) * E + e;
    const int r = offsets[e] + gbase[be] +
                  __popcll(gmasks[be] & ((1ull << (i / top_k)) - 1ull));
    sorted_slots[r] = s;
    slot_rows[s] = r;
  }
}

inline size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

}  // namespace

size_t permute_workspace_bytes(int64_t T, int E) {
  if (T <= kPermBlockTokens) return 0;
  const size_t nb = static_cast<size_t>((T + kPermBlockTokens - 1) / kPermBlockTokens);
  return align256(nb * E * sizeof(unsigned long long)) + align256(nb * E * sizeof(int));
}

void launch_permute(const int* ids, int T, int top_k, int E, int* offsets,
                    int* sorted_slots, int* slot_rows, int* active,
                    int* num_active, void* workspace, hipStream_t stream) {
  const int S = T * top_k;
  if (T <= kPermBlockTokens) {
    hipLaunchKernelGGL(permute_single_block_kernel, dim3(1), dim3(kScanThreads), 0, stream,
                       ids, T, top_k, E, offsets, sorted_slots, slot_rows, active,
                       num_active);
    return;
  }
  const int nb = (T + kPermBlockTokens - 1) / kPermBlockTokens;
  auto* gmasks = static_cast<unsigned long long*>(workspace);
  auto* gcount = reinterpret_cast<int*>(static_cast<char*>(workspace) +
                                        align256(static_cast<size_t>(nb) * E * 8));
  hipLaunchKernelGGL(permute_mask_kernel, dim3(nb), dim3(256), 0, stream, ids, T, top_k, E,
                     gmasks, gcount);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, nb, S, E,
                     gcount, offsets, active, num_active);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nb), dim3(256), 0, stream, ids, T, top_k, E,
                     gmasks, gcount, offsets, sorted_slots, slot_rows);
}

}  // namespace moe
