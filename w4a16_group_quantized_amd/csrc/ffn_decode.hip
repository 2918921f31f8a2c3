// Bandwidth-bound grouped expert FFN for small token counts (decode).
//
// Stage 1 (gate/up):  act[r, c] = SiLU(h_gate) * h_up,  h = x[token(r)] . W13[e]^T
// Stage 2 (down):     y_sorted[r, n] = act[r] . W2[e]^T
// for every sorted row r of every active expert e (the grouped W4A16 operator
// over active experts of "[Perf][SM70] Narrow Qwen3.8 AWQ active grouped
// decode", section "Purpose"; group size 32 along K).
//
// Work split.  A workgroup takes one active expert and one tile of weight rows
// (stage 1: NT gate rows with the matching NT up rows, so SiLU(gate)*up is
// formed in the epilogue).  Its G * P threads form a G x P grid: thread
// (g, p) owns quantisation group g (32 consecutive k, one 16-byte load per
// weight row) and the tile rows p, p + P, ...  The weight words, fp16 scale
// and 4-bit zero of its rows are loaded once into registers, so each weight
// byte is read from HBM exactly once; the expert's rows of A (x rows gathered
// through the sorted slots, or the act rows) are processed in chunks of up to
// two, each chunk's 32-value slice of A sitting in registers.
//
// Arithmetic.  A nibble q is turned into the fp16 number 1024 + q by OR-ing
// it into the mantissa of 0x6400 (nibbles in bits 4..7 of a half give
// 1024 + 16 q the same way), and v_dot2_f32_f16 multiplies two of these by
// two fp16 A values with exact products and fp32 accumulation.  The bias and
// the zero point are removed once per group:
//   sum_k (q_k - z) a_k = accA + accB / 16 - (1024 S_lo + 64 S_hi) - z S,
// with S_lo, S_hi the sums of A over the two nibble position classes and
// S = S_lo + S_hi; the group's fp16 scale is applied in fp32.  Partial sums of
// the G groups are combined in a fixed order through LDS.
//
// Precision of the down product.  act is stored as act_hi = fp16(act) and
// act_lo = fp16(act - act_hi) and both halves are multiplied, which carries
// act at about 22 bits instead of fp16's 11.
#include <math.h>

#include "common.h"

namespace moe {
namespace {

constexpr uint32_t kBias = 0x64006400u;  // fp16 1024.0 in both halves
constexpr uint32_t kOnes = 0x3C003C00u;  // fp16 1.0 in both halves
constexpr int kMaxThreads = 512;

// One A row's 32 values of this thread's group, paired to match the nibble
// positions: for 8-value block w, pairs (a0,a4), (a1,a5), (a2,a6), (a3,a7).
struct AFrag {
  uint32_t p[4][4];
  float c1;  // 1024 * S_lo + 64 * S_hi
  float s;   // S_lo + S_hi
};

__device__ __forceinline__ void load_afrag(const uint16_t* __restrict__ src, AFrag& f) {
  const uint4* q = reinterpret_cast<const uint4*>(src);
  float slo = 0.f, shi = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint4 d = q[w];  // d.x = (a0,a1), d.y = (a2,a3), d.z = (a4,a5), d.w = (a6,a7)
    f.p[w][0] = (d.x & 0xFFFFu) | (d.z << 16);
    f.p[w][1] = (d.x >> 16) | (d.z & 0xFFFF0000u);
    f.p[w][2] = (d.y & 0xFFFFu) | (d.w << 16);
    f.p[w][3] = (d.y >> 16) | (d.w & 0xFFFF0000u);
    slo = dot2_f16(f.p[w][0], kOnes, slo);
    slo = dot2_f16(f.p[w][2], kOnes, slo);
    shi = dot2_f16(f.p[w][1], kOnes, shi);
    shi = dot2_f16(f.p[w][3], kOnes, shi);
  }
  f.c1 = 1024.f * slo + 64.f * shi;
  f.s = slo + shi;
}

// sum_k (q_k - z) a_k over one group for NA rows of A.
template <int NA>
__device__ __forceinline__ void group_dot(const uint4 qv, float z, const AFrag (&a)[NA],
                                          float (&res)[NA]) {
  float ta[NA], tb[NA];
#pragma unroll
  for (int m = 0; m < NA; ++m) {
    ta[m] = 0.f;
    tb[m] = 0.f;
  }
  const uint32_t words[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t v = words[w];
    const uint32_t v8 = v >> 8;
    const uint32_t pa = (v & 0x000F000Fu) | kBias;   // 1024 + q0, 1024 + q4
    const uint32_t pb = (v & 0x00F000F0u) | kBias;   // 1024 + 16 q1, 1024 + 16 q5
    const uint32_t pc = (v8 & 0x000F000Fu) | kBias;  // 1024 + q2, 1024 + q6
    const uint32_t pd = (v8 & 0x00F000F0u) | kBias;  // 1024 + 16 q3, 1024 + 16 q7
#pragma unroll
    for (int m = 0; m < NA; ++m) {
      ta[m] = dot2_f16(pa, a[m].p[w][0], ta[m]);
      tb[m] = dot2_f16(pb, a[m].p[w][1], tb[m]);
      ta[m] = dot2_f16(pc, a[m].p[w][2], ta[m]);
      tb[m] = dot2_f16(pd, a[m].p[w][3], tb[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < NA; ++m) res[m] = fmaf(-z, a[m].s, fmaf(tb[m], 0.0625f, ta[m]) - a[m].c1);
}

// Register-resident quantised rows of one thread.
template <int RT>
struct WRows {
  uint4 q[RT];
  float s[RT];
  float z[RT];
};

template <int RT>
__device__ __forceinline__ void load_wrows(const int* __restrict__ qw, const uint16_t* __restrict__ sc,
                                           const int* __restrict__ qz, int G, int g,
                                           const int (&n)[RT], const bool (&valid)[RT],
                                           WRows<RT>& w) {
  const int KW = G * 4;  // int32 words per row
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    if (valid[i]) {
      w.q[i] = *reinterpret_cast<const uint4*>(qw + static_cast<size_t>(n[i]) * KW + 4 * g);
      w.s[i] = half_bits_to_float(sc[static_cast<size_t>(n[i]) * G + g]);
      const uint32_t zw = static_cast<uint32_t>(qz[static_cast<size_t>(n[i] >> 3) * G + g]);
      w.z[i] = static_cast<float>((zw >> (4 * (n[i] & 7))) & 0xFu);
    } else {
      w.q[i] = make_uint4(0u, 0u, 0u, 0u);
      w.s[i] = 0.f;
      w.z[i] = 0.f;
    }
  }
}

// Sum red[(lr * SL + m) * G + 0..G-1] into sum[lr * SL + m] for lr < rows, m < na.
template <int SL>
__device__ __forceinline__ void reduce_groups(const float* red, float* sum, int rows, int na, int G) {
  for (int o = threadIdx.x; o < rows * na; o += blockDim.x) {
    const int lr = o / na;
    const int m = o - lr * na;
    const float* src = red + (lr * SL + m) * G;
    float acc = 0.f;
    for (int gg = 0; gg < G; ++gg) acc += src[gg];
    sum[lr * SL + m] = acc;
  }
}

// ---------------------------------------------------------------- stage 1 ---
template <int NA, int RT, int SL>
__device__ __forceinline__ void gate_up_chunk(const GateUpArgs& args, const FfnWorkspace& ws,
                                              const WRows<RT>& w, int G, int P, int NT,
                                              int tile, int r0, int m0, float* red, float* sum) {
  const int g = threadIdx.x % G;
  const int p = threadIdx.x / G;
  AFrag a[NA];
#pragma unroll
  for (int m = 0; m < NA; ++m) {
    const int token = args.sorted_slots[r0 + m0 + m] / args.top_k;
    load_afrag(args.x + static_cast<size_t>(token) * args.H + 32 * g, a[m]);
  }
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    float d[NA];
    group_dot<NA>(w.q[i], w.z[i], a, d);
    const int lr = p + P * i;
#pragma unroll
    for (int m = 0; m < NA; ++m) red[(lr * SL + m) * G + g] = w.s[i] * d[m];
  }
  __syncthreads();
  reduce_groups<SL>(red, sum, P * RT, NA, G);
  __syncthreads();
  for (int o = threadIdx.x; o < NT * NA; o += blockDim.x) {
    const int c = o / NA;
    const int m = o - c * NA;
    const int col = tile * NT + c;
    if (col < args.I) {
      const float gate = sum[c * SL + m];
      const float up = sum[(NT + c) * SL + m];
      const float act = gate / (1.f + expf(-gate)) * up;
      const uint16_t hi = float_to_half_bits(act);
      const uint16_t lo = float_to_half_bits(act - half_bits_to_float(hi));
      const size_t idx = static_cast<size_t>(r0 + m0 + m) * args.I + col;
      ws.act_hi[idx] = hi;
      ws.act_lo[idx] = lo;
    }
  }
  __syncthreads();  // red / sum are reused by the next chunk
}

template <int RT, int NAMAX>
__global__ __launch_bounds__(kMaxThreads) void gate_up_decode_kernel(GateUpArgs args,
                                                                     FfnWorkspace ws, int G,
                                                                     int P, int NT,
                                                                     int n_tiles) {
  extern __shared__ float lds[];
  const int a_idx = blockIdx.x / n_tiles;
  const int tile = blockIdx.x - a_idx * n_tiles;
  if (a_idx >= *args.num_active) return;
  const int e = args.active[a_idx];
  const int r0 = args.offsets[e];
  const int rows_e = args.offsets[e + 1] - r0;
  const int I = args.I;
  const int g = threadIdx.x % G;
  const int p = threadIdx.x / G;

  int n[RT];
  bool valid[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const int lr = p + P * i;
    const int c = (lr < NT) ? lr : lr - NT;
    const int col = tile * NT + c;
    valid[i] = col < I;
    n[i] = (lr < NT) ? col : I + col;
  }
  const size_t rows_w = static_cast<size_t>(2 * I);
  WRows<RT> w;
  load_wrows<RT>(args.qw + static_cast<size_t>(e) * rows_w * (G * 4),
                 args.sc + static_cast<size_t>(e) * rows_w * G,
                 args.qz + static_cast<size_t>(e) * (rows_w / 8) * G, G, g, n, valid, w);

  float* red = lds;
  float* sum = lds + P * RT * NAMAX * G;
  for (int m0 = 0; m0 < rows_e; m0 += NAMAX) {
    if (NAMAX == 1 || rows_e - m0 == 1)
      gate_up_chunk<1, RT, NAMAX>(args, ws, w, G, P, NT, tile, r0, m0, red, sum);
    else
      gate_up_chunk<(NAMAX > 1 ? 2 : 1), RT, NAMAX>(args, ws, w, G, P, NT, tile, r0, m0, red, sum);
  }
}

// ---------------------------------------------------------------- stage 2 ---
template <int MR, int RT, int SL>
__device__ __forceinline__ void down_chunk(const DownArgs& args, const FfnWorkspace& ws,
                                           const WRows<RT>& w, int G, int P, int tile, int r0,
                                           int m0, float* red, float* sum) {
  const int g = threadIdx.x % G;
  const int p = threadIdx.x / G;
  AFrag a[2 * MR];  // [hi rows..., lo rows...]
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const size_t off = static_cast<size_t>(r0 + m0 + m) * args.I + 32 * g;
    load_afrag(ws.act_hi + off, a[m]);
    load_afrag(ws.act_lo + off, a[MR + m]);
  }
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    float d[2 * MR];
    group_dot<2 * MR>(w.q[i], w.z[i], a, d);
    const int lr = p + P * i;
#pragma unroll
    for (int m = 0; m < MR; ++m) red[(lr * SL + m) * G + g] = w.s[i] * (d[m] + d[MR + m]);
  }
  __syncthreads();
  reduce_groups<SL>(red, sum, P * RT, MR, G);
  __syncthreads();
  const int rows = P * RT;
  for (int o = threadIdx.x; o < rows * MR; o += blockDim.x) {
    const int m = o / rows;
    const int lr = o - m * rows;
    const int nrow = tile * rows + lr;
    if (nrow < args.H) args.y[static_cast<size_t>(r0 + m0 + m) * args.H + nrow] = sum[lr * SL + m];
  }
  __syncthreads();
}

template <int RT, int MRMAX>
__global__ __launch_bounds__(kMaxThreads) void down_decode_kernel(DownArgs args, FfnWorkspace ws,
                                                                  int G, int P, int n_tiles) {
  extern __shared__ float lds[];
  const int a_idx = blockIdx.x / n_tiles;
  const int tile = blockIdx.x - a_idx * n_tiles;
  if (a_idx >= *args.num_active) return;
  const int e = args.active[a_idx];
  const int r0 = args.offsets[e];
  const int rows_e = args.offsets[e + 1] - r0;
  const int g = threadIdx.x % G;
  const int p = threadIdx.x / G;
  const int rows = P * RT;

  int n[RT];
  bool valid[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    n[i] = tile * rows + p + P * i;
    valid[i] = n[i] < args.H;
  }
  const size_t H = static_cast<size_t>(args.H);
  WRows<RT> w;
  load_wrows<RT>(args.qw + static_cast<size_t>(e) * H * (G * 4),
                 args.sc + static_cast<size_t>(e) * H * G,
                 args.qz + static_cast<size_t>(e) * (H / 8) * G, G, g, n, valid, w);

  float* red = lds;
  float* sum = lds + rows * MRMAX * G;
  for (int m0 = 0; m0 < rows_e; m0 += MRMAX) {
    if (MRMAX == 1 || rows_e - m0 == 1)
      down_chunk<1, RT, MRMAX>(args, ws, w, G, P, tile, r0, m0, red, sum);
    else
      down_chunk<(MRMAX > 1 ? 2 : 1), RT, MRMAX>(args, ws, w, G, P, tile, r0, m0, red, sum);
  }
}

// Largest power of two P with G * P <= kMaxThreads.
int row_phases(int G) {
  int P = 1;
  while (G * P * 2 <= kMaxThreads) P *= 2;
  return P;
}

// Rows per thread: the largest of 4, 2, 1 (at least min_rt) that still gives
// >= 512 workgroups, else the smallest allowed.
template <typename TilesFn>
int pick_rows_per_thread(int min_rt, int slots, TilesFn tiles_for) {
  int rt = 4;
  while (rt > min_rt && static_cast<long long>(slots) * tiles_for(rt) < 512) rt >>= 1;
  return rt;
}

size_t chunk_lds_bytes(int threads, int rows, int RT, int slots_per_row) {
  return (static_cast<size_t>(threads) * RT * slots_per_row +
          static_cast<size_t>(rows) * slots_per_row) * sizeof(float);
}

}  // namespace

void launch_gate_up_decode(const GateUpArgs& a, const FfnWorkspace& ws, hipStream_t stream) {
  const int G = a.H / kGroup;
  const int P = row_phases(G);
  const int threads = G * P;
  const int slots = min(a.E, a.T * a.top_k);
  auto tiles_for = [&](int rt) {
    const int nt = P * rt / 2;
    return (a.I + nt - 1) / nt;
  };
  const int RT = pick_rows_per_thread(P == 1 ? 2 : 1, slots, tiles_for);
  const int NAMAX = a.T == 1 ? 1 : 2;
  const int NT = P * RT / 2;
  const int n_tiles = tiles_for(RT);
  const size_t lds = chunk_lds_bytes(threads, P * RT, RT, NAMAX);
  const dim3 grid(static_cast<unsigned>(slots) * n_tiles);
#define MOE_GU(rt, na)                                                                  \
  hipLaunchKernelGGL((gate_up_decode_kernel<rt, na>), grid, dim3(threads), lds, stream, a, ws, G, \
                     P, NT, n_tiles)
  if (NAMAX == 1) {
    switch (RT) {
      case 4: MOE_GU(4, 1); break;
      case 2: MOE_GU(2, 1); break;
      default: MOE_GU(1, 1); break;
    }
  } else {
    switch (RT) {
      case 4: MOE_GU(4, 2); break;
      case 2: MOE_GU(2, 2); break;
      default: MOE_GU(1, 2); break;
    }
  }
#undef MOE_GU
}

void launch_down_decode(const DownArgs& a, const FfnWorkspace& ws, hipStream_t stream) {
  const int G = a.I / kGroup;
  const int P = row_phases(G);
  const int threads = G * P;
  const int slots = min(a.E, a.T * a.top_k);
  auto tiles_for = [&](int rt) { return (a.H + P * rt - 1) / (P * rt); };
  const int RT = pick_rows_per_thread(1, slots, tiles_for);
  const int MRMAX = a.T == 1 ? 1 : 2;
  const int n_tiles = tiles_for(RT);
  const size_t lds = chunk_lds_bytes(threads, P * RT, RT, MRMAX);
  const dim3 grid(static_cast<unsigned>(slots) * n_tiles);
#define MOE_DN(rt, mr)                                                                          \
  hipLaunchKernelGGL((down_decode_kernel<rt, mr>), grid, dim3(threads), lds, stream, a, ws, G, P, \
                     n_tiles)
  if (MRMAX == 1) {
    switch (RT) {
      case 4: MOE_DN(4, 1); break;
      case 2: MOE_DN(2, 1); break;
      default: MOE_DN(1, 1); break;
    }
  } else {
    switch (RT) {
      case 4: MOE_DN(4, 2); break;
      case 2: MOE_DN(2, 2); break;
      default: MOE_DN(1, 2); break;
    }
  }
#undef MOE_DN
}

}  // namespace moe
