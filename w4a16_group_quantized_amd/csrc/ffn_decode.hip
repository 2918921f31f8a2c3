// Bandwidth-bound grouped expert FFN for small token counts (decode).
//
// Stage 1 (gate/up):  act[r, c] = SiLU(h_gate) * h_up,  h = x[token(r)] . W13[e]^T
// Stage 2 (down):     y_sorted[r, n] = act[r] . W2[e]^T
// for every sorted row r of every active expert e (the grouped W4A16 operator
// over active experts of "[Perf][SM70] Narrow Qwen3.8 AWQ active grouped
// decode", section "Purpose"; group size 32 along K).
//
// Work split.  A cluster of C lanes owns one weight row; lane c of the
// cluster takes the row's quantisation groups c, c + C, ... (one 16-byte load
// of codes per group), so each step of a wave reads C * 16 contiguous bytes
// from each of its 64 / C rows.  A wave owns a contiguous run of row blocks of
// one expert (stage 1: a block is R/2 gate rows in the lower half of the wave
// and the matching R/2 up rows in the upper half, R = 64 / C), steps through
// them with a ring of kDepth register slots of weight loads in flight, and
// sums a row's groups within the cluster with DPP once the row is done;
// nothing is synchronised across waves in the streaming loop.  The expert's
// rows of A (x rows gathered through the sorted slots, or act rows) are staged
// once per workgroup in LDS, already paired to the nibble layout, and read
// back as broadcasts.  The grid is sized to what the chip holds at once.
//
// Arithmetic.  A nibble q is turned into the fp16 number 1024 + q by OR-ing
// it into the mantissa of 0x6400 (nibbles in bits 4..7 of a half give
// 1024 + 16 q the same way), and v_dot2_f32_f16 multiplies two of these by
// two fp16 A values with exact products and fp32 accumulation.  The bias and
// the zero point are removed once per group:
//   sum_k (q_k - z) a_k = accA + accB / 16 - (1024 S_lo + 64 S_hi) - z S,
// with S_lo, S_hi the sums of A over the two nibble position classes and
// S = S_lo + S_hi; the group's fp16 scale is applied in fp32.  The order of
// every sum is fixed, so results do not depend on scheduling.
//
// Precision of the down product.  act is stored as act_hi = fp16(act) and
// act_lo = fp16(act - act_hi) and both halves are multiplied, which carries
// act at about 22 bits instead of fp16's 11.
#include <math.h>

#include "common.h"

namespace moe {
namespace {

constexpr uint32_t kOnes = 0x3C003C00u;   // fp16 1.0 in both halves
constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kDepth = 4;                 // weight loads in flight per lane (ring slots)
constexpr int kBufferFlags = 0x00020000;  // buffer descriptor word 3 for raw dword access on gfx9
constexpr int kFragDwords = 20;           // LDS dwords per (A row, group): 16 pairs, c1, s, pad

// ------------------------------------------------------------ A fragments ---
// One A row's 32 values of a group, paired to match the nibble positions: for
// 8-value block w, pairs (a0,a4), (a1,a5), (a2,a6), (a3,a7); plus
// c1 = 1024 S_lo + 64 S_hi and s = S_lo + S_hi.  Written to LDS once.
__device__ __forceinline__ void stage_frag(const uint16_t* __restrict__ src, uint32_t* dst) {
  const uint4* q = reinterpret_cast<const uint4*>(src);
  uint32_t p[16];
  float slo = 0.f, shi = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint4 d = q[w];  // d.x = (a0,a1), d.y = (a2,a3), d.z = (a4,a5), d.w = (a6,a7)
    p[4 * w + 0] = (d.x & 0xFFFFu) | (d.z << 16);
    p[4 * w + 1] = (d.x >> 16) | (d.z & 0xFFFF0000u);
    p[4 * w + 2] = (d.y & 0xFFFFu) | (d.w << 16);
    p[4 * w + 3] = (d.y >> 16) | (d.w & 0xFFFF0000u);
    slo = dot2_f16(p[4 * w + 0], kOnes, slo);
    slo = dot2_f16(p[4 * w + 2], kOnes, slo);
    shi = dot2_f16(p[4 * w + 1], kOnes, shi);
    shi = dot2_f16(p[4 * w + 3], kOnes, shi);
  }
  uint4* d4 = reinterpret_cast<uint4*>(dst);
#pragma unroll
  for (int i = 0; i < 4; ++i) d4[i] = make_uint4(p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]);
  *reinterpret_cast<uint2*>(dst + 16) =
      make_uint2(__builtin_bit_cast(uint32_t, 1024.f * slo + 64.f * shi),
                 __builtin_bit_cast(uint32_t, slo + shi));
}

// Nibble codes of one group as biased fp16 pairs (see the file comment).
struct Codes {
  uint32_t a[4], b[4], c[4], d[4];
};

__device__ __forceinline__ Codes expand_codes(const uint4 qv) {
  // The bias lives in a vector register: gfx9 VOP3 takes no literal and one
  // scalar operand, so with the mask in a scalar register each mask-and-insert
  // is a single v_and_or_b32.
  uint32_t bias;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(bias));
  const uint32_t words[4] = {qv.x, qv.y, qv.z, qv.w};
  Codes k;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t v = words[w];
    const uint32_t v8 = v >> 8;
    k.a[w] = (v & 0x000F000Fu) | bias;   // 1024 + q0, 1024 + q4
    k.b[w] = (v & 0x00F000F0u) | bias;   // 1024 + 16 q1, 1024 + 16 q5
    k.c[w] = (v8 & 0x000F000Fu) | bias;  // 1024 + q2, 1024 + q6
    k.d[w] = (v8 & 0x00F000F0u) | bias;  // 1024 + 16 q3, 1024 + 16 q7
  }
  return k;
}

// sum_k (q_k - z) a_k over one group, A fragment read from LDS.
__device__ __forceinline__ float group_dot(const Codes& k, float z, const uint32_t* frag) {
  const uint4* f4 = reinterpret_cast<const uint4*>(frag);
  float ta = 0.f, tb = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint4 f = f4[w];
    ta = dot2_f16(k.a[w], f.x, ta);
    tb = dot2_f16(k.b[w], f.y, tb);
    ta = dot2_f16(k.c[w], f.z, ta);
    tb = dot2_f16(k.d[w], f.w, tb);
  }
  const uint2 cs = *reinterpret_cast<const uint2*>(frag + 16);
  return fmaf(-z, __builtin_bit_cast(float, cs.y),
              fmaf(tb, 0.0625f, ta) - __builtin_bit_cast(float, cs.x));
}

// ------------------------------------------------------------ weight ring ---
// One step's loads, kept exactly as loaded until the step is computed.
struct Slot {
  uint4 q;
  uint32_t s;
  uint32_t zw;
};

struct ExpertBufs {
  __amdgpu_buffer_rsrc_t q, s, z;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           kBufferFlags);
}

// Raw buffer loads take a 32-bit offset against a uniform base and return 0
// past the end without touching memory, so a row index of `rows` is a free
// "no load".
__device__ __forceinline__ ExpertBufs expert_bufs(const int* qw, const uint16_t* sc, const int* qz,
                                                  int rows, int G) {
  ExpertBufs b;
  b.q = make_rsrc(qw, static_cast<uint32_t>(rows) * G * 16u);
  b.s = make_rsrc(sc, static_cast<uint32_t>(rows) * G * 2u);
  b.z = make_rsrc(qz, static_cast<uint32_t>(rows / 8) * G * 4u);
  return b;
}

__device__ __forceinline__ void load_slot(const ExpertBufs& b, int G, uint32_t row, uint32_t g,
                                          Slot& s) {
  const uint32_t idx = __umul24(row, G) + g;
  const auto qv = __builtin_amdgcn_raw_buffer_load_b128(b.q, static_cast<int>(idx * 16u), 0, 0);
  s.q = make_uint4(qv[0], qv[1], qv[2], qv[3]);
  s.s = __builtin_amdgcn_raw_buffer_load_b16(b.s, static_cast<int>(idx * 2u), 0, 0);
  s.zw = __builtin_amdgcn_raw_buffer_load_b32(
      b.z, static_cast<int>((__umul24(row >> 3, G) + g) * 4u), 0, 0);
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false);
  return v + __builtin_bit_cast(float, moved);
}

// Sum over each aligned cluster of C lanes (C a power of two <= 16); every
// lane of the cluster gets the sum.  Called with all lanes of the wave active.
__device__ __forceinline__ float cluster_sum(float v, int C) {
  if (C >= 2) v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]: partner lane ^ 1
  if (C >= 4) v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]: partner lane ^ 2
  if (C >= 8) v = dpp_add<0x141>(v);  // row_half_mirror: lane i <-> 7 - i within 8
  if (C >= 16) v = dpp_add<0x140>(v); // row_mirror: lane i <-> 15 - i within 16
  return v;
}

// Geometry of one stage, fixed per launch.
struct Geom {
  int G;       // groups along K
  int C;       // lanes per row (cluster); rows per wave block R = 64 / C
  int spb;     // steps per block = ceil(G / C)
  int nb;      // blocks per expert
  int bpw;     // blocks per wave
  int splits;  // workgroups per active-expert slot
};

// Weight row that lane cluster k reads in block b, or `rows` when there is
// none.  Stage 1: lower half of the wave gate rows, upper half up rows.
template <bool GATE_UP>
__device__ __forceinline__ int block_row(int b, int k, int R, int I, int H) {
  if (GATE_UP) {
    const int half = R >> 1;
    const int col = b * half + (k < half ? k : k - half);
    if (col >= I) return 2 * I;
    return k < half ? col : I + col;
  }
  const int n = b * R + k;
  return n < H ? n : H;
}

// ------------------------------------------------------------------ kernel --
// Per-wave step geometry of one run of blocks [b0, b1).
struct WaveRun {
  int k, lc, R, S, b0;
};

__device__ __forceinline__ WaveRun wave_run(const Geom& geo, int b0, int b1) {
  const int lane = threadIdx.x & 63;
  WaveRun w;
  w.R = 64 / geo.C;
  w.k = lane / geo.C;
  w.lc = lane & (geo.C - 1);
  w.S = (b1 - b0) * geo.spb;
  w.b0 = b0;
  return w;
}

// Issue the loads of step s into a slot (a no-load when s is past the run).
template <bool GATE_UP>
__device__ __forceinline__ void load_step(const ExpertBufs& bufs, const Geom& geo, const WaveRun& w,
                                          int rows_w, int I, int H, int s, Slot& slot) {
  const int gg = (s % geo.spb) * geo.C + w.lc;
  const bool live = s < w.S && gg < geo.G;
  const uint32_t row = live ? block_row<GATE_UP>(w.b0 + s / geo.spb, w.k, w.R, I, H) : rows_w;
  load_slot(bufs, geo.G, row, live ? gg : 0, slot);
}

// Fill the ring with the first kDepth steps.  Needs only the expert, so it
// is issued before the A rows are staged.
template <bool GATE_UP>
__device__ __forceinline__ void prime_ring(const ExpertBufs& bufs, const Geom& geo,
                                           const WaveRun& w, int rows_w, int I, int H,
                                           Slot (&ring)[kDepth]) {
#pragma unroll
  for (int d = 0; d < kDepth; ++d) load_step<GATE_UP>(bufs, geo, w, rows_w, I, H, d, ring[d]);
}

// Streams the wave's run of blocks for mc (<= NA) rows of A, the ring already
// primed.  Stage 2 fragments come in (hi, lo) pairs: fragment 2m is act_hi of
// row m, 2m + 1 its act_lo.
template <bool GATE_UP, int NA>
__device__ __forceinline__ void stream_expert(const ExpertBufs& bufs, const Geom& geo,
                                              const WaveRun& wr, Slot (&ring)[kDepth], int rows_w,
                                              int I, int H, const uint32_t* frags, int mc,
                                              int r_first, uint16_t* act_hi, uint16_t* act_lo,
                                              float* y) {
  const int lane = threadIdx.x & 63;
  const int C = geo.C;
  const int R = wr.R;
  const int k = wr.k;
  const int lc = wr.lc;
  const int G = geo.G;
  const int spb = geo.spb;
  const int S = wr.S;
  const int b0 = wr.b0;

  constexpr int NF = GATE_UP ? NA : 2 * NA;  // fragments per chunk of A rows
  const int nf = GATE_UP ? mc : 2 * mc;
  float acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = 0.f;

  for (int s0 = 0; s0 < S; s0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int s = s0 + d;
      if (s < S) {
        const int b = b0 + s / spb;
        const int j = s - (s / spb) * spb;
        const int gg = j * C + lc;
        const uint32_t row = static_cast<uint32_t>(block_row<GATE_UP>(b, k, R, I, H));
        const Slot& sl = ring[d];
        const float scale = half_bits_to_float(static_cast<uint16_t>(sl.s));
        const float z = static_cast<float>((sl.zw >> (4u * (row & 7u))) & 0xFu);
        const Codes codes = expand_codes(sl.q);
        const uint32_t* fr = frags + (gg < G ? gg : 0) * kFragDwords;
#pragma unroll
        for (int f = 0; f < NF; ++f)
          if (f < nf) acc[f] = fmaf(scale, group_dot(codes, z, fr + f * G * kFragDwords), acc[f]);
        if (j == spb - 1) {  // block done: finish its rows
#pragma unroll
          for (int m = 0; m < NA; ++m) {
            if (m < mc) {
              if (GATE_UP) {
                const float v = cluster_sum(acc[m], C);
                const float u = __shfl_xor(v, 32, 64);  // up half of the wave -> gate half
                const int col = b * (R >> 1) + k;
                if (lane < 32 && lc == 0 && col < I) {
                  const float act = v / (1.f + expf(-v)) * u;
                  const uint16_t hi = float_to_half_bits(act);
                  const uint16_t lo = float_to_half_bits(act - half_bits_to_float(hi));
                  const size_t idx = static_cast<size_t>(r_first + m) * I + col;
                  act_hi[idx] = hi;
                  act_lo[idx] = lo;
                }
              } else {
                const float v = cluster_sum(acc[2 * m] + acc[2 * m + 1], C);
                const int n = b * R + k;
                if (lc == 0 && n < H) y[static_cast<size_t>(r_first + m) * H + n] = v;
              }
            }
          }
#pragma unroll
          for (int f = 0; f < NF; ++f) acc[f] = 0.f;
        }
      }
      // Refill this slot with the step kDepth ahead; past the end this is a
      // no-load, issued anyway so every path keeps the same wait counts.
      load_step<GATE_UP>(bufs, geo, wr, rows_w, I, H, s + kDepth, ring[d]);
    }
  }
}

template <int NA>
__global__ __launch_bounds__(kThreads) void gate_up_decode_kernel(GateUpArgs args, FfnWorkspace ws,
                                                                  Geom geo) {
  extern __shared__ uint32_t frags[];
  const int a_idx = blockIdx.x / geo.splits;
  const int split = blockIdx.x - a_idx * geo.splits;
  const int n_active = *args.num_active;
  const int e = args.active[a_idx];  // in bounds: a_idx < min(E, T * top_k)
  if (a_idx >= n_active) return;
  const int I = args.I, H = args.H, G = geo.G;
  const int wave_id = split * kWaves + (threadIdx.x >> 6);
  const int b0 = min(geo.nb, wave_id * geo.bpw);
  const int b1 = min(geo.nb, b0 + geo.bpw);
  const size_t rows_w = static_cast<size_t>(2 * I);
  const ExpertBufs bufs = expert_bufs(args.qw + static_cast<size_t>(e) * rows_w * (G * 4),
                                      args.sc + static_cast<size_t>(e) * rows_w * G,
                                      args.qz + static_cast<size_t>(e) * (rows_w / 8) * G,
                                      2 * I, G);
  const WaveRun wr = wave_run(geo, b0, b1);
  Slot ring[kDepth];
  prime_ring<true>(bufs, geo, wr, 2 * I, I, H, ring);
  const int r0 = args.offsets[e];
  const int rows_e = args.offsets[e + 1] - r0;
  for (int m0 = 0; m0 < rows_e; m0 += NA) {
    const int mc = min(NA, rows_e - m0);
    if (m0 > 0) {
      __syncthreads();  // previous chunk's fragments are no longer read
      prime_ring<true>(bufs, geo, wr, 2 * I, I, H, ring);
    }
    for (int i = threadIdx.x; i < mc * G; i += kThreads) {
      const int m = i / G;
      const int g = i - m * G;
      const int token = args.sorted_slots[r0 + m0 + m] / args.top_k;
      stage_frag(args.x + static_cast<size_t>(token) * H + 32 * g, frags + i * kFragDwords);
    }
    __syncthreads();
    stream_expert<true, NA>(bufs, geo, wr, ring, 2 * I, I, H, frags, mc, r0 + m0, ws.act_hi,
                            ws.act_lo, nullptr);
  }
}

template <int NA>
__global__ __launch_bounds__(kThreads) void down_decode_kernel(DownArgs args, FfnWorkspace ws,
                                                               Geom geo) {
  extern __shared__ uint32_t frags[];
  const int a_idx = blockIdx.x / geo.splits;
  const int split = blockIdx.x - a_idx * geo.splits;
  const int n_active = *args.num_active;
  const int e = args.active[a_idx];
  if (a_idx >= n_active) return;
  const int I = args.I, H = args.H, G = geo.G;
  const int wave_id = split * kWaves + (threadIdx.x >> 6);
  const int b0 = min(geo.nb, wave_id * geo.bpw);
  const int b1 = min(geo.nb, b0 + geo.bpw);
  const size_t rows_w = static_cast<size_t>(H);
  const ExpertBufs bufs = expert_bufs(args.qw + static_cast<size_t>(e) * rows_w * (G * 4),
                                      args.sc + static_cast<size_t>(e) * rows_w * G,
                                      args.qz + static_cast<size_t>(e) * (rows_w / 8) * G, H, G);
  const WaveRun wr = wave_run(geo, b0, b1);
  Slot ring[kDepth];
  prime_ring<false>(bufs, geo, wr, H, I, H, ring);
  const int r0 = args.offsets[e];
  const int rows_e = args.offsets[e + 1] - r0;
  for (int m0 = 0; m0 < rows_e; m0 += NA) {
    const int mc = min(NA, rows_e - m0);
    if (m0 > 0) {
      __syncthreads();
      prime_ring<false>(bufs, geo, wr, H, I, H, ring);
    }
    // fragment f = 2 m + {0: hi, 1: lo} of act row r0 + m0 + m, at f * G + g
    for (int i = threadIdx.x; i < 2 * mc * G; i += kThreads) {
      const int f = i / G;
      const int g = i - f * G;
      const size_t off = static_cast<size_t>(r0 + m0 + (f >> 1)) * I + 32 * g;
      stage_frag(((f & 1) ? ws.act_lo : ws.act_hi) + off, frags + i * kFragDwords);
    }
    __syncthreads();
    stream_expert<false, NA>(bufs, geo, wr, ring, H, I, H, frags, mc, r0 + m0, nullptr, nullptr,
                             args.y);
  }
}

// ----------------------------------------------------------------- host -----
// Lanes per row: the largest power of two <= 8 that divides G.
int cluster_lanes(int G) {
  int C = 1;
  while (C < 8 && G % (2 * C) == 0) C *= 2;
  return C;
}

// Spread each active-expert slot's blocks over as many waves as the chip
// holds at once (no second round), each wave taking a contiguous run.
void split_blocks(Geom& geo, int slots, int resident) {
  int splits = max(1, resident / max(1, slots));
  splits = min(splits, (geo.nb + kWaves - 1) / kWaves);
  geo.bpw = (geo.nb + splits * kWaves - 1) / (splits * kWaves);
  geo.splits = (geo.nb + geo.bpw * kWaves - 1) / (geo.bpw * kWaves);
}

template <int NA>
void launch_gate_up_na(const GateUpArgs& a, const FfnWorkspace& ws, Geom geo, hipStream_t stream) {
  const size_t lds = static_cast<size_t>(NA) * geo.G * kFragDwords * sizeof(uint32_t);
  const int slots = min(a.E, a.T * a.top_k);
  static OccTable occ;
  split_blocks(geo, slots, resident_workgroups(gate_up_decode_kernel<NA>, kThreads, lds, occ));
  hipLaunchKernelGGL((gate_up_decode_kernel<NA>), dim3(static_cast<unsigned>(slots) * geo.splits),
                     dim3(kThreads), lds, stream, a, ws, geo);
}

template <int NA>
void launch_down_na(const DownArgs& a, const FfnWorkspace& ws, Geom geo, hipStream_t stream) {
  const size_t lds = static_cast<size_t>(2 * NA) * geo.G * kFragDwords * sizeof(uint32_t);
  const int slots = min(a.E, a.T * a.top_k);
  static OccTable occ;
  split_blocks(geo, slots, resident_workgroups(down_decode_kernel<NA>, kThreads, lds, occ));
  hipLaunchKernelGGL((down_decode_kernel<NA>), dim3(static_cast<unsigned>(slots) * geo.splits),
                     dim3(kThreads), lds, stream, a, ws, geo);
}

}  // namespace

void launch_gate_up_decode(const GateUpArgs& a, const FfnWorkspace& ws, hipStream_t stream) {
  Geom geo;
  geo.G = a.H / kGroup;
  geo.C = cluster_lanes(geo.G);
  geo.spb = (geo.G + geo.C - 1) / geo.C;
  const int half = (64 / geo.C) / 2;  // gate (= up) rows per block
  geo.nb = (a.I + half - 1) / half;
  if (a.T == 1)
    launch_gate_up_na<1>(a, ws, geo, stream);
  else
    launch_gate_up_na<2>(a, ws, geo, stream);
}

void launch_down_decode(const DownArgs& a, const FfnWorkspace& ws, hipStream_t stream) {
  Geom geo;
  geo.G = a.I / kGroup;
  geo.C = cluster_lanes(geo.G);
  geo.spb = (geo.G + geo.C - 1) / geo.C;
  geo.nb = (a.H + 64 / geo.C - 1) / (64 / geo.C);
  if (a.T == 1)
    launch_down_na<1>(a, ws, geo, stream);
  else
    launch_down_na<2>(a, ws, geo, stream);
}

}  // namespace moe
