// Matrix-core grouped expert FFN for larger token counts (prefill).
//
// Same two stages as the decode path ("[Perf][SM70] Narrow Qwen3.8 AWQ active
// grouped decode", section "Purpose": a grouped W4A16 operator over the
// active experts' multi-row segments; group size 32 along K):
//   stage 1: act[r, c] = SiLU(h_gate) * h_up,  h = x[token(r)] . W13[e]^T
//   stage 2: y_sorted[r, n] = act[r] . W2[e]^T
// but as dense tiles on v_mfma_f32_16x16x32_f16.
//
// Schedule.  A tile-list kernel cuts every active expert's segment of sorted
// rows into M-tiles of kBM rows (so a heavily loaded expert becomes many
// tiles) and the GEMM grid is (M-tile slot, N-tile); slots past the list
// exit at once.  Consecutive workgroups share an M-tile, and the M-tiles of
// one expert are consecutive, so the tiles reading the same weights run at
// about the same time.
//
// Operands.  One MFMA covers exactly one quantisation group (K = 32), so each
// group's product P = A . (q - z) is formed with an exact integer B (q - z is
// an integer in [-15, 15], exact in fp16) and a zero accumulator, then
// scaled in fp32: acc += s[n, g] * P.  A lane holds 8 values of a row of A
// and 8 of a column of B over the same k-slots; within each 8-wide block the
// k order is (0, 4, 1, 5, 2, 6, 3, 7), the order in which the nibble unpack
// produces (q - z) pairs, so A is stored permuted the same way.  Stage 2 runs
// act_hi and act_lo through two MFMAs into the same partial, carrying act at
// about 22 bits.  Inputs are staged in LDS two groups at a time, double
// buffered; weights are read with buffer loads so rows past the matrix read
// as zeros.
#include <math.h>

#include "common.h"

namespace moe {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kBM = 64;                    // rows of A per M-tile
constexpr int kBN = 128;                   // weight rows (output columns) per N-tile
constexpr int kThreads = 256;              // 4 waves: 2 (M) x 2 (N)
constexpr int kKC = 2;                     // groups per LDS stage
constexpr int kAStride = kKC * 32 + 8;     // halfs per staged A row (padded)
constexpr int kBufferFlags = 0x00020000;   // buffer descriptor word 3 for raw dword access on gfx9
constexpr int kBStride = kBN + 16;         // dwords per (group, word) row of staged codes (bank spread)

struct PrefillArgs {
  const uint16_t* x;   // stage 1 A source
  int T, top_k, E, H, I;
  const int* offsets;
  const int* sorted_slots;
  const int* qw;
  const uint16_t* sc;
  const int* qz;
  float* y;            // stage 2 output
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           kBufferFlags);
}

// 8 consecutive fp16 (4 dwords: (a0,a1) (a2,a3) (a4,a5) (a6,a7)) reordered
// to the k-slot order (a0,a4) (a1,a5) (a2,a6) (a3,a7).
__device__ __forceinline__ uint4 permute8(uint4 d) {
  return make_uint4((d.x & 0xFFFFu) | (d.z << 16), (d.x >> 16) | (d.z & 0xFFFF0000u),
                    (d.y & 0xFFFFu) | (d.w << 16), (d.y >> 16) | (d.w & 0xFFFF0000u));
}

// (q - z) of one packed word as 8 fp16 in k-slot order, exactly.
__device__ __forceinline__ half8 exact_codes(uint32_t w, uint32_t z) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const uint32_t w8 = w >> 8;
  const uint32_t bias = 0x64006400u;
  const h2 pa = __builtin_bit_cast(h2, (w & 0x000F000Fu) | bias);   // 1024 + q0, 1024 + q4
  const h2 pb = __builtin_bit_cast(h2, (w & 0x00F000F0u) | bias);   // 1024 + 16 q1, ...
  const h2 pc = __builtin_bit_cast(h2, (w8 & 0x000F000Fu) | bias);  // 1024 + q2, 1024 + q6
  const h2 pd = __builtin_bit_cast(h2, (w8 & 0x00F000F0u) | bias);  // 1024 + 16 q3, ...
  const _Float16 zf = static_cast<_Float16>(static_cast<float>(z));
  const h2 m1024 = {static_cast<_Float16>(-1024.f) - zf, static_cast<_Float16>(-1024.f) - zf};
  const h2 m64 = {static_cast<_Float16>(-64.f) - zf, static_cast<_Float16>(-64.f) - zf};
  const h2 sixteenth = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
  const h2 r0 = pa + m1024;              // q0 - z, q4 - z (exact)
  const h2 r1 = pb * sixteenth + m64;    // q1 - z, q5 - z (exact)
  const h2 r2 = pc + m1024;
  const h2 r3 = pd * sixteenth + m64;
  half8 out;
  out[0] = r0[0]; out[1] = r0[1]; out[2] = r1[0]; out[3] = r1[1];
  out[4] = r2[0]; out[5] = r2[1]; out[6] = r3[0]; out[7] = r3[1];
  return out;
}

// Shared-memory stage of both operands (one buffer of the double buffer).
template <bool GATE_UP>
struct Stage {
  static constexpr int kARows = GATE_UP ? 1 : 2;           // A copies: x, or act hi/lo
  uint16_t a[kARows][kBM * kAStride];                     // A rows, k-slot order
  uint32_t bq[kKC * 4 * kBStride];                         // codes: [group][word][row]
  uint16_t bs[kKC * kBN];                                  // scales: [group][row]
  uint32_t bz[kKC * (kBN / 8)];                            // zero words: [group][row block]
};

// Weight row of the N-tile's row r.  Stage 1: rows [0, 64) gate columns,
// [64, 128) the matching up columns.
template <bool GATE_UP>
__device__ __forceinline__ int tile_weight_row(int nt, int r, int I) {
  if (GATE_UP) return r < kBN / 2 ? nt * (kBN / 2) + r : I + nt * (kBN / 2) + (r - kBN / 2);
  return nt * kBN + r;
}

// Global loads of one stage into registers (issued before the previous
// stage is computed).
struct StageRegs {
  uint4 a[2][2];   // [chunk][copy]
  uint4 q;
  uint32_t s;
  uint32_t z;
};

template <bool GATE_UP>
__device__ __forceinline__ void load_stage(const PrefillArgs& p, const uint16_t* act_hi,
                                           const uint16_t* act_lo, const int* a_rows, int rows,
                                           int K, int N, int G, int g0,
                                           __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rs,
                                           __amdgpu_buffer_rsrc_t rz, int nt, StageRegs& st) {
  const int t = threadIdx.x;
  // A: kBM rows x kKC*32 k = 8 chunks of 8 halfs per row, 2 chunks per thread
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int id = t + c * kThreads;
    const int r = id >> 3;
    const int ch = id & 7;
    const int k = g0 * 32 + ch * 8;
    const bool live = r < rows && k < K;
    if (GATE_UP) {
      st.a[c][0] = live ? *reinterpret_cast<const uint4*>(p.x + static_cast<size_t>(a_rows[r]) * K + k)
                        : make_uint4(0u, 0u, 0u, 0u);
    } else {
      const size_t off = static_cast<size_t>(a_rows[r]) * K + k;
      st.a[c][0] = live ? *reinterpret_cast<const uint4*>(act_hi + off) : make_uint4(0u, 0u, 0u, 0u);
      st.a[c][1] = live ? *reinterpret_cast<const uint4*>(act_lo + off) : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // B: kBN rows x kKC groups of 16 bytes, one per thread
  const int r = t >> 1;
  const int gl = t & 1;
  const int g = g0 + gl;
  const uint32_t n = static_cast<uint32_t>(tile_weight_row<GATE_UP>(nt, r, p.I));
  // a group past G is loaded from one past the end of the buffers: zeros
  const uint32_t idx = g < G ? __umul24(n, G) + g : static_cast<uint32_t>(N) * G;
  const auto qv = __builtin_amdgcn_raw_buffer_load_b128(rq, static_cast<int>(idx * 16u), 0, 0);
  st.q = make_uint4(qv[0], qv[1], qv[2], qv[3]);
  st.s = __builtin_amdgcn_raw_buffer_load_b16(rs, static_cast<int>(idx * 2u), 0, 0);
  // zero words: kBN / 8 row blocks x kKC groups, threads 0..31
  st.z = 0;
  if (t < (kBN / 8) * kKC) {
    const int rb = t >> 1;
    const int zg = g0 + (t & 1);
    const uint32_t n0 = static_cast<uint32_t>(tile_weight_row<GATE_UP>(nt, rb * 8, p.I));
    if (zg < G)
      st.z = __builtin_amdgcn_raw_buffer_load_b32(rz, static_cast<int>((__umul24(n0 >> 3, G) + zg) * 4u), 0, 0);
  }
}

template <bool GATE_UP>
__device__ __forceinline__ void store_stage(const StageRegs& st, Stage<GATE_UP>& sm) {
  const int t = threadIdx.x;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int id = t + c * kThreads;
    const int r = id >> 3;
    const int ch = id & 7;
#pragma unroll
    for (int cp = 0; cp < Stage<GATE_UP>::kARows; ++cp)
      *reinterpret_cast<uint4*>(&sm.a[cp][r * kAStride + ch * 8]) = permute8(st.a[c][cp]);
  }
  const int r = t >> 1;
  const int gl = t & 1;
  sm.bq[(gl * 4 + 0) * kBStride + r] = st.q.x;
  sm.bq[(gl * 4 + 1) * kBStride + r] = st.q.y;
  sm.bq[(gl * 4 + 2) * kBStride + r] = st.q.z;
  sm.bq[(gl * 4 + 3) * kBStride + r] = st.q.w;
  sm.bs[gl * kBN + r] = static_cast<uint16_t>(st.s);
  if (t < (kBN / 8) * kKC) sm.bz[(t & 1) * (kBN / 8) + (t >> 1)] = st.z;
}

// Wave tile: 2 M-subtiles (16 rows each) x 4 N-subtiles (16 weight rows each).
// Stage 1: N-subtiles 0,1 are gate columns, 2,3 the matching up columns.
template <bool GATE_UP>
__device__ __forceinline__ int wave_nrow(int wn, int s) {
  if (GATE_UP) return (s < 2 ? 0 : kBN / 2) + wn * 32 + (s & 1) * 16;
  return wn * 64 + s * 16;
}

template <bool GATE_UP>
__device__ __forceinline__ void compute_stage(const Stage<GATE_UP>& sm, int ngroups, int wm, int wn,
                                              float4v (&acc)[2][4]) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
  const int q = lane >> 4;
  for (int gl = 0; gl < ngroups; ++gl) {
    half8 a[Stage<GATE_UP>::kARows][2];
#pragma unroll
    for (int cp = 0; cp < Stage<GATE_UP>::kARows; ++cp)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int row = wm * 32 + m * 16 + j;
        a[cp][m] = __builtin_bit_cast(
            half8, *reinterpret_cast<const uint4*>(&sm.a[cp][row * kAStride + gl * 32 + q * 8]));
      }
    float4v p[2][4];
    float sc[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int nr = wave_nrow<GATE_UP>(wn, s) + j;
      const uint32_t w = sm.bq[(gl * 4 + q) * kBStride + nr];
      const uint32_t z = (sm.bz[gl * (kBN / 8) + (nr >> 3)] >> (4 * (nr & 7))) & 0xFu;
      sc[s] = half_bits_to_float(sm.bs[gl * kBN + nr]);
      const half8 b = exact_codes(w, z);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const float4v zero = {0.f, 0.f, 0.f, 0.f};
        p[m][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0][m], b, zero, 0, 0, 0);
        if (!GATE_UP)
          p[m][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[Stage<GATE_UP>::kARows - 1][m], b,
                                                           p[m][s], 0, 0, 0);
      }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[m][s][v] = fmaf(sc[s], p[m][s][v], acc[m][s][v]);
  }
}

// ------------------------------------------------------------------ kernels --
// Tile list: for every active expert, ceil(rows / kBM) entries (expert, first
// row); tile_count entries in total, in active-expert order.
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int* __restrict__ offsets,
                                                          const int* __restrict__ active,
                                                          const int* __restrict__ num_active,
                                                          int* __restrict__ tiles,
                                                          int* __restrict__ tile_count) {
  __shared__ int wave_tot[17];
  constexpr int kPer = kMaxExperts / 1024;
  const int tid = threadIdx.x;
  const int na = *num_active;
  int cnt[kPer];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int a = tid * kPer + i;
    cnt[i] = 0;
    if (a < na) {
      const int e = active[a];
      cnt[i] = (offsets[e + 1] - offsets[e] + kBM - 1) / kBM;
    }
    sum += cnt[i];
  }
  // block exclusive scan of `sum`
  const int lane = tid & 63, wave = tid >> 6;
  int inc = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < 16 ? wave_tot[lane] : 0;
    int winc = w;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(winc, d, 64);
      if (lane >= d) winc += o;
    }
    if (lane < 16) wave_tot[lane] = winc - w;
    if (lane == 15) wave_tot[16] = winc;
  }
  __syncthreads();
  int pos = wave_tot[wave] + inc - sum;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int a = tid * kPer + i;
    if (a < na) {
      const int e = active[a];
      const int r0 = offsets[e];
      for (int t = 0; t < cnt[i]; ++t) {
        tiles[2 * (pos + t)] = e;
        tiles[2 * (pos + t) + 1] = r0 + t * kBM;
      }
    }
    pos += cnt[i];
  }
  if (tid == 0) *tile_count = wave_tot[16];
}

template <bool GATE_UP>
__global__ __launch_bounds__(kThreads) void ffn_mfma_kernel(PrefillArgs p, FfnWorkspace ws,
                                                            int n_ntiles) {
  __shared__ Stage<GATE_UP> sm[2];
  __shared__ int a_rows[kBM];
  const int slot = blockIdx.x / n_ntiles;
  const int nt = blockIdx.x - slot * n_ntiles;
  if (slot >= *ws.tile_count) return;
  const int e = ws.tiles[2 * slot];
  const int row0 = ws.tiles[2 * slot + 1];
  const int rows = min(kBM, p.offsets[e + 1] - row0);
  const int K = GATE_UP ? p.H : p.I;
  const int N = GATE_UP ? 2 * p.I : p.H;
  const int G = K / kGroup;
  const size_t wbase = static_cast<size_t>(e) * N;
  const auto rq = make_rsrc(p.qw + wbase * (G * 4), static_cast<uint32_t>(N) * G * 16u);
  const auto rs = make_rsrc(p.sc + wbase * G, static_cast<uint32_t>(N) * G * 2u);
  const auto rz = make_rsrc(p.qz + (wbase / 8) * G, static_cast<uint32_t>(N / 8) * G * 4u);

  if (threadIdx.x < kBM) {
    const int r = threadIdx.x;
    int src = 0;
    if (r < rows) src = GATE_UP ? p.sorted_slots[row0 + r] / p.top_k : row0 + r;
    a_rows[r] = src;
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  float4v acc[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[m][s] = float4v{0.f, 0.f, 0.f, 0.f};

  const int nstages = (G + kKC - 1) / kKC;
  StageRegs st;
  load_stage<GATE_UP>(p, ws.act_hi, ws.act_lo, a_rows, rows, K, N, G, 0, rq, rs, rz, nt, st);
  store_stage<GATE_UP>(st, sm[0]);
  __syncthreads();
  for (int s = 0; s < nstages; ++s) {
    const int g0 = s * kKC;
    if (s + 1 < nstages)
      load_stage<GATE_UP>(p, ws.act_hi, ws.act_lo, a_rows, rows, K, N, G, g0 + kKC, rq, rs, rz, nt, st);
    compute_stage<GATE_UP>(sm[s & 1], min(kKC, G - g0), wm, wn, acc);
    if (s + 1 < nstages) store_stage<GATE_UP>(st, sm[(s + 1) & 1]);
    __syncthreads();
  }

  // epilogue: lane holds rows 4 (lane / 16) + v and column lane % 16 of each subtile
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = wm * 32 + m * 16 + (lane >> 4) * 4 + v;
      if (r >= rows) continue;
      if (GATE_UP) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int col = nt * (kBN / 2) + wn * 32 + s * 16 + j;
          if (col < p.I) {
            const float gate = acc[m][s][v];
            const float up = acc[m][s + 2][v];
            const float act = gate / (1.f + expf(-gate)) * up;
            const uint16_t hi = float_to_half_bits(act);
            const uint16_t lo = float_to_half_bits(act - half_bits_to_float(hi));
            const size_t idx = static_cast<size_t>(row0 + r) * p.I + col;
            ws.act_hi[idx] = hi;
            ws.act_lo[idx] = lo;
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int col = nt * kBN + wn * 64 + s * 16 + j;
          if (col < p.H) p.y[static_cast<size_t>(row0 + r) * p.H + col] = acc[m][s][v];
        }
      }
    }
  }
}

int max_tiles(int S, int E) { return (S + kBM - 1) / kBM + min(E, S); }

}  // namespace

void launch_build_tiles(const int* offsets, const int* active, const int* num_active,
                        const FfnWorkspace& ws, hipStream_t stream) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, stream, offsets, active,
                     num_active, ws.tiles, ws.tile_count);
}

void launch_gate_up_prefill(const GateUpArgs& a, const FfnWorkspace& ws, hipStream_t stream) {
  PrefillArgs p{a.x, a.T, a.top_k, a.E, a.H, a.I, a.offsets, a.sorted_slots, a.qw, a.sc, a.qz,
                nullptr};
  const int n_ntiles = (a.I + kBN / 2 - 1) / (kBN / 2);
  const int slots = max_tiles(a.T * a.top_k, a.E);
  hipLaunchKernelGGL((ffn_mfma_kernel<true>), dim3(static_cast<unsigned>(slots) * n_ntiles),
                     dim3(kThreads), 0, stream, p, ws, n_ntiles);
}

void launch_down_prefill(const DownArgs& a, const FfnWorkspace& ws, hipStream_t stream) {
  PrefillArgs p{nullptr, a.T, a.top_k, a.E, a.H, a.I, a.offsets, nullptr, a.qw, a.sc, a.qz, a.y};
  const int n_ntiles = (a.H + kBN - 1) / kBN;
  const int slots = max_tiles(a.T * a.top_k, a.E);
  hipLaunchKernelGGL((ffn_mfma_kernel<false>), dim3(static_cast<unsigned>(slots) * n_ntiles),
                     dim3(kThreads), 0, stream, p, ws, n_ntiles);
}

int prefill_max_tiles(int64_t S, int E) { return max_tiles(static_cast<int>(S), E); }

}  // namespace moe
