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
// from each of its 64 / C rows.  A block is the R = 64 / C rows a wave streams
// together (stage 1: R/2 gate rows in the lower half of the wave and the
// matching R/2 up rows in the upper half); a wave streams a block through a
// ring of kDepth register slots of weight loads in flight and sums each row's
// groups within its cluster with DPP when the block is done.  One workgroup
// of 16 waves runs per compute unit; it owns an equal share of the
// (expert, block) units and its waves take units from a counter in LDS, so
// that all of them finish together (see the units section below).
//
// Staging.  Before streaming, a workgroup copies into LDS its experts' rows
// of A (x rows gathered through the sorted slots, or act rows), already
// paired to the nibble layout.  The fp16 scales of a unit (below) are loaded
// with two 16-byte loads per lane by the wave that takes the unit, one unit
// ahead, and written to that unit's slot in LDS.  Per step a lane then issues
// one 16-byte code load and one 4-byte zero-word load to global memory; its
// scale and A values come from LDS.  (Loading each 2-byte scale from global
// memory in the step costs nearly as much in memory requests as the codes
// themselves.)  The workgroup's barriers order LDS only, so the weight loads
// issued before them stay in flight.
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
// act at about 22 bits instead of fp16's 11: each half's group dot has its
// bias removed on its own, and the two are added before the group's scale.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "permute.h"
#include "route.h"

namespace moe {
namespace {

constexpr uint32_t kOnes = 0x3C003C00u;   // fp16 1.0 in both halves
constexpr int kWaves = 16;                // waves per workgroup (one workgroup per compute unit)
constexpr int kThreads = 64 * kWaves;
constexpr int kDepth = 4;                 // weight loads in flight per lane (ring slots)
constexpr int kBufferFlags = 0x00020000;  // buffer descriptor word 3 for raw dword access on gfx9
constexpr int kFragDwords = 20;           // LDS dwords per (A row, group): 16 pairs, c1, s, pad

// ------------------------------------------------------------ A fragments ---
// One A row's 32 values of a group, paired to match the nibble positions: for
// 8-value block w, pairs (a0,a4), (a1,a5), (a2,a6), (a3,a7); plus
// c1 = 1024 S_lo + 64 S_hi and s = S_lo + S_hi.  Written to LDS once.
__device__ __forceinline__ void build_frag(const uint4 (&q)[4], uint32_t* dst) {
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

__device__ __forceinline__ void load_group(const uint16_t* __restrict__ src, uint4 (&q)[4]) {
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
  for (int w = 0; w < 4; ++w) q[w] = s4[w];
}

__device__ __forceinline__ void stage_frag(const uint16_t* __restrict__ src, uint32_t* dst) {
  uint4 q[4];
  load_group(src, q);
  build_frag(q, dst);
}

// A fragment as read back from LDS.
struct Frag {
  uint4 v[4];
  uint2 c;
};

__device__ __forceinline__ Frag read_frag(const uint32_t* frag) {
  const uint4* f4 = reinterpret_cast<const uint4*>(frag);
  Frag f;
#pragma unroll
  for (int w = 0; w < 4; ++w) f.v[w] = f4[w];
  f.c = *reinterpret_cast<const uint2*>(frag + 16);
  return f;
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

// sum_k (q_k - z) a_k over one group.
__device__ __forceinline__ float group_dot(const Codes& k, float z, const Frag& f) {
  float ta = 0.f, tb = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    ta = dot2_f16(k.a[w], f.v[w].x, ta);
    tb = dot2_f16(k.b[w], f.v[w].y, tb);
    ta = dot2_f16(k.c[w], f.v[w].z, ta);
    tb = dot2_f16(k.d[w], f.v[w].w, tb);
  }
  return fmaf(-z, __builtin_bit_cast(float, f.c.y),
              fmaf(tb, 0.0625f, ta) - __builtin_bit_cast(float, f.c.x));
}

// ------------------------------------------------------------ weight ring ---
// One step's global loads, kept exactly as loaded until the step is computed.
struct Slot {
  uint4 q;
  uint32_t zw;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           kBufferFlags);
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

// ----------------------------------------------------------------- units ---
// Work is cut into units (active-expert slot a, block b), numbered a * nb + b.
// Workgroup w of nwg owns the units [U w / nwg, U (w + 1) / nwg), U =
// num_active * nb, when the experts' row counts are alike (routed experts at
// decode sizes hold one or two rows).  When an expert may hold many rows (a
// shared expert holds every token) units are shared out by cost instead: a
// unit of an expert with r rows costs
// passes(r) * kUnitBase + r (streaming its weights once per pass of na rows,
// plus the arithmetic of each row), so an expert with many rows (a shared
// expert runs on every token) spreads over more workgroups.  With P the
// exclusive prefix of the per-unit costs over the active experts and
// C = nb * P[num_active], unit (a, b) starts at cost nb * P[a] + b * cost(a),
// and workgroup w of nwg owns the units that start in [C w / nwg,
// C (w + 1) / nwg): a contiguous run of units, every unit owned exactly once.
// The gate/up kernel computes P (one block scan) and workgroup 0 writes it to
// the FFN workspace, where the down kernel reads it.  A workgroup works
// through its units in windows of at most kXE experts and wmax units.  For a window it stages in LDS the A rows of its experts
// (na rows per expert per pass; more passes when an expert has more rows),
// then its 16 waves take units from an LDS counter until the window is done
// (the first unit of wave i is unit w0 + i, primed before staging), each
// wave bringing its unit's scales into the unit's LDS slot.  Taking units
// dynamically matters: waves that share a SIMD are served oldest first, so
// equal static shares finish far apart in time.
struct Geom {
  int G;     // groups along K
  int C;     // lanes per row (cluster); rows per block R = 64 / C
  int spb;   // steps per block = G / C
  int nb;    // blocks per expert
  int nwg;   // workgroups (one per compute unit)
  int wmax;  // units per window (bounded by LDS)
  int ucap;  // ints of the LDS unit-cost table: prefix [slots + 1], then scan totals
  int weighted;  // units shared out by cost (an expert holds many rows); else evenly
};

constexpr int kUnitBase = 4;  // cost of streaming a unit's weights once, in rows of arithmetic

__device__ __forceinline__ int unit_cost(int rows, int na) {
  return ((rows + na - 1) / na) * kUnitBase + rows;
}

// First unit whose start cost is >= c (num_active * nb when none), for the
// per-unit cost prefix P[0..n] in LDS.
__device__ __forceinline__ int first_unit(const int* P, int n, int nb, int64_t c) {
  int lo = 0, hi = n;  // the largest a with nb * P[a] <= c (P[0] = 0 <= c)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (static_cast<int64_t>(nb) * P[mid] <= c) lo = mid; else hi = mid - 1;
  }
  if (lo == n) return n * nb;
  const int64_t cost = P[lo + 1] - P[lo];
  const int64_t b = (c - static_cast<int64_t>(nb) * P[lo] + cost - 1) / cost;
  return b >= nb ? (lo + 1) * nb : lo * nb + static_cast<int>(b);
}

constexpr int kXE = 2;  // experts per window

// Workgroup barrier that orders LDS accesses only.  (__syncthreads also
// waits for every global load in flight, here the weight loads issued ahead
// of the barrier on purpose.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Element i (0 or 1) of a two-entry per-window table, without indexing a
// private array by a run-time value.
__device__ __forceinline__ int pick(const int (&t)[kXE], int i) { return i == 0 ? t[0] : t[1]; }

struct DecodeArgs {
  const uint16_t* x;       // stage 1 A: x [T, H]
  const uint16_t* a_hi;    // stage 2 A: act_hi, act_lo [S, I]
  const uint16_t* a_lo;
  const int* offsets;
  const int* sorted_slots;
  const int* active;
  const int* num_active;
  const int* qw;
  const uint16_t* sc;
  const int* qz;
  int T, top_k, H, I;
  uint16_t* act_hi;        // stage 1 outputs
  uint16_t* act_lo;
  float* y;                // stage 2 output
  int* cost_out;           // stage 1: per-unit cost prefix [num_active + 1], workgroup 0 writes it
  const int* cost_in;      // stage 2: that prefix
  // a shared expert (the last expert, E - 1, holding sorted rows [shared_row0,
  // shared_row0 + T)) on the matrix cores in shared_wgs extra workgroups;
  // the units then cover the other active experts only
  int shared_wgs;
  int shared_row0;
  // stage 1 that routes the tokens itself: logits in; the routing (as
  // moe_route_permute returns it) written out by workgroup 0.  E and top_k
  // count the shared expert when `shared` is 1: the logits then have E - 1
  // columns, top_k - 1 choices are routed and slot top_k - 1 of every token
  // is expert E - 1 with weight 1.
  const float* logits;
  int E;
  int shared;
  int* r_ids;
  float* r_weights;
  int* r_offsets;
  int* r_sorted;
  int* r_slot_rows;
  int* r_active;
  int* r_num_active;
  // stage 2 with the combine folded in (down_fold_kernel): the routing's
  // weights and slot rows in, the layer output out
  const float* c_weights;
  const int* c_slot_rows;
  uint16_t* out;
};

// LDS bytes of the routing tables of a kernel that routes (T <= 64 tokens,
// E <= 1024 experts): token masks, offsets, active list, sorted slots, slot
// experts, the active count and the scans' wave totals.
__host__ __device__ inline size_t route_lds_bytes(int E, int S) {
  const size_t b = 8ull * E + 4ull * (E + 1) + 4ull * E + 8ull * S + 4 + 4 * (kScanThreads / 64 + 1);
  return (b + 15) & ~static_cast<size_t>(15);
}

// Scale halves of one unit: the R rows of its block (stage 1: R/2 gate rows,
// then R/2 up rows), G each; R * G = 64 * spb.
__device__ __host__ __forceinline__ int unit_scale_halves(int spb) { return 64 * spb; }

// Weight row that lane cluster k streams in block b, or `rows_w` when there
// is none.  Stage 1: lower half of the wave gate rows, upper half up rows.
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

// Scales of a unit, as staged in LDS: its R rows x G halves (stage 1: R/2
// gate rows, then R/2 up rows), 8 spb chunks of 16 bytes.  A unit's rows are
// one (stage 2) or two (stage 1) contiguous ranges of 32 spb halves, 16-byte
// aligned, so chunk i is one 16-byte load; its byte offset into the
// expert's scale array follows (a ragged last block reads past the end and
// gets zeros from the buffer load).
template <bool GATE_UP>
__device__ __forceinline__ uint32_t scale_chunk(int I, int G, int spb, int R, int b, int i) {
  const int x = i * 8;  // halves into the unit's block
  int row0, xr;
  if (GATE_UP) {
    const bool up = x >= 32 * spb;
    xr = up ? x - 32 * spb : x;
    row0 = (up ? I : 0) + b * (R >> 1);
  } else {
    xr = x;
    row0 = b * R;
  }
  return (static_cast<uint32_t>(row0) * G + xr) * 2u;
}

constexpr int kMaxSpbHeld = 16;  // units of up to 128 chunks are carried in two loads per lane

// Buffer descriptors of expert e's weights.  Raw buffer loads take a 32-bit
// offset against a uniform base and return 0 past the end without touching
// memory, so a row index of rows_w is a free "no load".
struct ExpertBufs {
  __amdgpu_buffer_rsrc_t q, z, s;
};

__device__ __forceinline__ ExpertBufs expert_bufs(const DecodeArgs& p, int rows_w, int G, int e) {
  ExpertBufs b;
  b.q = make_rsrc(p.qw + static_cast<size_t>(e) * rows_w * (G * 4),
                  static_cast<uint32_t>(rows_w) * G * 16u);
  b.z = make_rsrc(p.qz + static_cast<size_t>(e) * (rows_w / 8) * G,
                  static_cast<uint32_t>(rows_w / 8) * G * 4u);
  b.s = make_rsrc(p.sc + static_cast<size_t>(e) * rows_w * G, static_cast<uint32_t>(rows_w) * G * 2u);
  return b;
}

__device__ __forceinline__ void issue_step(const ExpertBufs& bufs, int G, uint32_t row, int gg,
                                           Slot& sl) {
  const uint32_t idx = row * static_cast<uint32_t>(G) + gg;
  const auto qv = __builtin_amdgcn_raw_buffer_load_b128(bufs.q, static_cast<int>(idx * 16u), 0, 0);
  sl.q = make_uint4(qv[0], qv[1], qv[2], qv[3]);
  sl.zw = __builtin_amdgcn_raw_buffer_load_b32(
      bufs.z, static_cast<int>(((row >> 3) * static_cast<uint32_t>(G) + gg) * 4u), 0, 0);
}

__device__ __forceinline__ uint4 load_b128(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(byte_off), 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Rows of A that the window's expert i holds in pass c, and where its
// fragments sit in LDS.
struct WinExpert {
  int e, r0, rows;
};

// ---------------------------------------------------------- shared expert --
// A shared expert holds all T tokens (sorted rows [shared_row0, +T)): a small
// dense GEMM, which extra workgroups of the launch run on the matrix cores
// while the others stream the routed experts.  A workgroup takes
// ShCfg::kTiles column tiles of 32 weight rows (stage 1: 16 gate columns in
// lanes j < 16 of each lane half and the matching 16 up columns in lanes
// j >= 16; stage 2: 32 output columns) and splits K over its
// 16 / ShCfg::kTiles waves per tile; their
// partial sums meet in LDS and are added in a fixed order.  A (the T x rows,
// or the T act rows hi and lo) is staged once in LDS, permuted to the nibble
// k-slot order; the weight loads run kShDepth groups ahead in a register
// ring.  Per quantisation group, two v_mfma_f32_32x32x16_f16 (stage 2: four,
// act hi then lo) with the exact integer B = q - z make a partial that is
// scaled by the group's scale in fp32, as in the matrix-core FFN.  Rows past T
// are zero operands; columns past the matrix read zeros.  Lane (h, j) ends
// with rows 8 (v / 4) + 4 h + v % 4 of column j.
constexpr int kShDepth = 4;                     // weight groups in flight per lane
template <bool GATE_UP>
struct ShCfg {
  static constexpr int kTiles = GATE_UP ? 4 : 8;           // column tiles per workgroup
  static constexpr int kSplits = kWaves / kTiles;          // waves per tile, over K
  static constexpr int kCopies = GATE_UP ? 1 : 2;          // A copies: x, or act hi and lo
};

// LDS bytes of the shared-expert path: A rows (row stride K + 8 halves, so
// that the 32 lanes reading one k offset of different rows use different
// banks) and the partial sums of all splits but the first.
__host__ __device__ inline size_t shared_lds_bytes(bool gate_up, int T, int K) {
  const int tiles = gate_up ? ShCfg<true>::kTiles : ShCfg<false>::kTiles;
  const int copies = gate_up ? 1 : 2;
  return static_cast<size_t>(copies) * T * (K + 8) * 2 +
         static_cast<size_t>(tiles) * (kWaves / tiles - 1) * 64 * 16 * 4;
}

struct ShSlot {
  uint4 q;
  uint32_t z, s;
};

template <bool GATE_UP>
__device__ __forceinline__ void shared_expert_mfma(const DecodeArgs& p, uint32_t* lds, int wg) {
  using Cfg = ShCfg<GATE_UP>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, j = lane & 31;
  const int I = p.I, H = p.H, T = p.T;
  const int K = GATE_UP ? H : I;
  const int G = K / kGroup;
  const int rows_w = GATE_UP ? 2 * I : H;
  const int stride = K + 8;                                // LDS row stride, halves
  uint16_t* as = reinterpret_cast<uint16_t*>(lds);
  float* part = reinterpret_cast<float*>(as + Cfg::kCopies * T * stride);

  // ---- stage A: T rows of K, 16 bytes per thread per step, k-slot order
  {
    const int chunks = T * (K / 8);
    for (int c = static_cast<int>(threadIdx.x); c < Cfg::kCopies * chunks; c += kThreads) {
      const int cp = c / chunks, cc = c - cp * chunks;
      const int r = cc / (K / 8), k8 = cc - r * (K / 8);
      const uint16_t* src = GATE_UP ? p.x + static_cast<size_t>(r) * H
                                    : (cp ? p.a_lo : p.a_hi) + static_cast<size_t>(p.shared_row0 + r) * I;
      const uint4 v = reinterpret_cast<const uint4*>(src)[k8];
      *reinterpret_cast<uint4*>(as + (cp * T + r) * stride + 8 * k8) = permute8(v);
    }
  }
  __syncthreads();

  const int tile = wg * Cfg::kTiles + wave % Cfg::kTiles;
  const int split = wave / Cfg::kTiles;
  int n, col;
  bool live;
  if (GATE_UP) {
    col = tile * 16 + (j & 15);
    live = tile * 16 < I;
    n = col < I ? (j < 16 ? col : I + col) : rows_w;   // rows_w: no row, zeros
  } else {
    col = tile * 32 + j;
    live = tile * 32 < H;
    n = col < H ? col : rows_w;
  }
  const int g0 = split * ((G + Cfg::kSplits - 1) / Cfg::kSplits);
  const int g1 = min(G, g0 + (G + Cfg::kSplits - 1) / Cfg::kSplits);
  const ExpertBufs wb = expert_bufs(p, rows_w, G, p.E - 1);
  const uint32_t zshift = 4u * static_cast<uint32_t>(n & 7);
  uint32_t bias;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(bias));
  float16v acc = {};
  if (live) {  // uniform: the whole wave
    ShSlot ring[kShDepth];
    auto issue = [&](int d, int g) {
      // past g1 (the ring's tail): a row index past the matrix, zeros
      const uint32_t row = g < g1 ? static_cast<uint32_t>(n) : static_cast<uint32_t>(rows_w);
      const uint32_t gg = static_cast<uint32_t>(g < g1 ? g : 0);
      ring[d].q = load_b128(wb.q, (row * G + gg) * 16u);
      ring[d].z = __builtin_amdgcn_raw_buffer_load_b32(
          wb.z, static_cast<int>(((row >> 3) * G + gg) * 4u), 0, 0);
      ring[d].s = __builtin_amdgcn_raw_buffer_load_b16(
          wb.s, static_cast<int>((row * G + gg) * 2u), 0, 0);
    };
#pragma unroll
    for (int d = 0; d < kShDepth; ++d) issue(d, g0 + d);
    const half8 zero8 = {};
    for (int g = g0; g < g1; g += kShDepth) {
#pragma unroll
      for (int d = 0; d < kShDepth; ++d) {
        const int gd = g + d;
        if (gd < g1) {
          auto a_op = [&](int cp, int t) -> half8 {
            if (j >= T) return zero8;
            return *reinterpret_cast<const half8*>(as + (cp * T + j) * stride + 32 * gd + 16 * t + 8 * h);
          };
          const half8 a0 = a_op(0, 0), a1 = a_op(0, 1);
          const ShSlot sl = ring[d];
          h2 m1024, m64;
          zero_terms((sl.z >> zshift) & 0xFu, m1024, m64);
          // MFMA t takes k [16 t + 8 h, +8) of the group: word 2 t + h of the codes
          const half8 b0 = dequant_word(h ? sl.q.y : sl.q.x, bias, m1024, m64);
          const half8 b1 = dequant_word(h ? sl.q.w : sl.q.z, bias, m1024, m64);
          float16v pr = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, float16v{}, 0, 0, 0);
          pr = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, pr, 0, 0, 0);
          if (!GATE_UP) {
            const half8 l0 = a_op(1, 0), l1 = a_op(1, 1);
            pr = __builtin_amdgcn_mfma_f32_32x32x16_f16(l0, b0, pr, 0, 0, 0);
            pr = __builtin_amdgcn_mfma_f32_32x32x16_f16(l1, b1, pr, 0, 0, 0);
          }
          const float sc = half_bits_to_float(static_cast<uint16_t>(sl.s));
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[v] = fmaf(sc, pr[v], acc[v]);
          issue(d, gd + kShDepth);  // refill the slot (a no-load past the end)
        }
      }
    }
  }
  // splits 1.. hand their partial sums to split 0 of their tile
  if (split > 0) {
    float* dst = part + ((wave % Cfg::kTiles) * (Cfg::kSplits - 1) + split - 1) * 64 * 16;
#pragma unroll
    for (int v = 0; v < 16; ++v) dst[v * 64 + lane] = acc[v];
  }
  __syncthreads();
  if (split > 0 || !live) return;
  for (int sp = 1; sp < Cfg::kSplits; ++sp) {
    const float* src = part + ((wave % Cfg::kTiles) * (Cfg::kSplits - 1) + sp - 1) * 64 * 16;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] += src[v * 64 + lane];
  }
  if (GATE_UP) {
    // lanes j < 16 hold gate and lanes j + 16 the up value of the same
    // column; each lane of the pair finishes 8 of the 16 rows
    const bool low = j < 16;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float send = low ? acc[u + 8] : acc[u];
      const float recv = __shfl_xor(send, 16, 64);
      const int v = low ? u : u + 8;
      const float gate = low ? acc[u] : recv;
      const float up = low ? recv : acc[u + 8];
      const int r = 8 * (v >> 2) + 4 * h + (v & 3);
      if (r < T && col < I) {
        const float act = gate / (1.f + expf(-gate)) * up;
        const uint16_t hi = float_to_half_bits(act);
        const uint16_t lo = float_to_half_bits(act - half_bits_to_float(hi));
        const size_t idx = static_cast<size_t>(p.shared_row0 + r) * I + col;
        p.act_hi[idx] = hi;
        p.act_lo[idx] = lo;
      }
    }
  } else {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 8 * (v >> 2) + 4 * h + (v & 3);
      if (r < T && col < H) p.y[static_cast<size_t>(p.shared_row0 + r) * H + col] = acc[v];
    }
  }
}

// Polls a stage-1 completion count (agent scope) until it reaches `target`.
// Bounded: it gives up after kWaitTicks of the 100 MHz real-time counter and
// returns false (the caller then writes NaN), so a wait never hangs.
constexpr uint64_t kWaitTicks = 20000000;  // 200 ms
__device__ __forceinline__ bool wait_count(const int* ctr, int target) {
  int* c = const_cast<int*>(ctr);
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) return false;
    __builtin_amdgcn_s_sleep(2);
  }
  return true;
}

// One stage of the one-launch FFN over this workgroup's share of the units,
// with the routing tables in LDS (ract, roff, rsorted); `area` holds the
// stage's LDS areas (frag_bytes, then wmax unit slots).  The stage body is
// decode_kernel's (decode_stage.inc).  WAIT (stage 2): a window's act rows
// are staged only once every stage-1 unit of its experts is done (done[a]
// reaches `target` for each of its active slots a); a wait that runs out
// (wait_count) makes the window write NaN instead of y.
template <bool GATE_UP, int NA, bool WAIT>
__device__ __forceinline__ void one_launch_stage(const DecodeArgs& p, const Geom& geo,
                                                 uint32_t* area, int& queue, int& poison,
                                                 const int* ract, const int* roff,
                                                 const int* rsorted, int n_active,
                                                 const int* done, int target) {
  constexpr int FPR = GATE_UP ? 1 : 2;        // fragments per A row (stage 2: hi, lo)
  constexpr int NF = NA * FPR;                // fragments per expert and pass
  const int G = geo.G, C = geo.C, spb = geo.spb, nb = geo.nb;
  const int I = p.I, H = p.H;
  const int rows_w = GATE_UP ? 2 * I : H;
  const int R = 64 / C, half = R >> 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int k = lane / C, lc = lane & (C - 1);
  uint32_t* frags = area;
  uint16_t* scales = reinterpret_cast<uint16_t*>(area + kXE * NF * G * kFragDwords);
  int* ucost = reinterpret_cast<int*>(scales + geo.wmax * unit_scale_halves(spb));
  auto active_at = [&](int a) { return ract[a]; };
  auto offset_at = [&](int e) { return roff[e]; };
  auto sorted_at = [&](int r) { return rsorted[r]; };
#include "decode_stage.inc"
}

// NPL > 0 (stage 1 only): the workgroup first routes the tokens itself, with
// the router's and permutation's own steps (route.h, permute.h), from
// logits of E <= 64 NPL experts; workgroup 0 writes the routing out.  Every
// workgroup computes the same routing, so none waits for another.
template <bool GATE_UP, int NA, int NPL>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs p, Geom geo) {
  // 16-byte aligned: fragments and scales are read with 16-byte LDS loads,
  // and the static counter below would otherwise shift the dynamic area
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ int queue;
  constexpr int FPR = GATE_UP ? 1 : 2;        // fragments per A row (stage 2: hi, lo)
  constexpr int NF = NA * FPR;                // fragments per expert and pass
  const int G = geo.G, C = geo.C, spb = geo.spb, nb = geo.nb;
  const int I = p.I, H = p.H;
  const int rows_w = GATE_UP ? 2 * I : H;
  const int R = 64 / C, half = R >> 1;
  const int lane = threadIdx.x & 63;
  // the wave index is the same in every lane; saying so keeps the unit
  // bookkeeping in scalar registers and its branches uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (static_cast<int>(blockIdx.x) >= geo.nwg) {  // the extra workgroups: the shared expert
    shared_expert_mfma<GATE_UP>(p, lds, static_cast<int>(blockIdx.x) - geo.nwg);
    return;
  }
  const int k = lane / C, lc = lane & (C - 1);
  uint32_t* frags = lds;
  uint16_t* scales = reinterpret_cast<uint16_t*>(lds + kXE * NF * G * kFragDwords);
  int* ucost = reinterpret_cast<int*>(scales + geo.wmax * unit_scale_halves(spb));

  // ---- routing: from the caller's arrays, or computed here (NPL > 0)
  int* ract = nullptr;     // LDS: active list, offsets, sorted slots
  int* roff = nullptr;
  int* rsorted = nullptr;
  int n_active;
  if constexpr (NPL > 0) {
    void* const rbase = ucost + geo.ucap;  // the routing tables, past the cost table
#include "decode_route.inc"
  } else {
    n_active = *p.num_active;
  }
  // the shared expert is the last active expert; its extra workgroups take it
  if (p.shared_wgs > 0) n_active -= 1;
  auto active_at = [&](int a) { if constexpr (NPL > 0) return ract[a]; else return p.active[a]; };
  auto offset_at = [&](int e) { if constexpr (NPL > 0) return roff[e]; else return p.offsets[e]; };
  auto sorted_at = [&](int r) { if constexpr (NPL > 0) return rsorted[r]; else return p.sorted_slots[r]; };

  // a kernel of its own never waits (the body's WAIT code compiles away)
  constexpr bool WAIT = false;
  const int* const done = nullptr;
  const int target = 0;
  int& poison = queue;
#include "decode_stage.inc"
}

// Completion counts of the one-launch FFN, per device: [a] the stage-1 units
// done of active slot a, [kOneLaunchMaxSlots] the workgroups that have
// finished.  Zero at module load; the last workgroup of every launch sets
// them back to zero.
constexpr int kOneLaunchMaxSlots = 1024;
__device__ int g_one_launch_sync[kOneLaunchMaxSlots + 1];

// Gate/up and down in one persistent launch (routing inside, T <= 64 tokens,
// E <= 1024 experts), one workgroup per compute unit.  Every workgroup routes
// the tokens (decode_route.inc) and runs its stage-1 share; once its act stores
// have completed it publishes, after an agent-scope release, how many stage-1
// units of each active expert it did, and runs its stage-2 share, whose
// windows issue their weight loads at once and stage their act rows once the
// experts' counts are complete (after an agent-scope acquire).  Stage 1 never
// waits, so with every workgroup resident every wait ends; a wait that runs
// out (another kernel holding compute units for 200 ms) makes its window
// write NaN.  The shares, units and arithmetic are those of the two separate
// kernels with an even split, so the results are theirs bit for bit.  Calls
// that overlap in time on one device share the counts and must not be issued.
template <int NA, int NPL>
__global__ __launch_bounds__(kThreads) void one_launch_kernel(DecodeArgs p1, Geom g1, DecodeArgs p2,
                                                              Geom g2, int table_bytes) {
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ int queue;
  __shared__ int poison;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int* ract = nullptr;     // LDS: active list, offsets, sorted slots
  int* roff = nullptr;
  int* rsorted = nullptr;
  int n_active;
  {
    const DecodeArgs& p = p1;
    void* const rbase = lds;  // the routing tables, at the start of LDS
#include "decode_route.inc"
  }
  uint32_t* area = lds + table_bytes / 4;  // each stage's fragments and unit slots, in turn
  int* sync = g_one_launch_sync;

  one_launch_stage<true, NA, false>(p1, g1, area, queue, poison, ract, roff, rsorted, n_active,
                                    nullptr, 0);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's act stores have completed
  __syncthreads();                // (and no wave reads stage 1's LDS areas any more)
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    // this workgroup's stage-1 share, as the stage body splits the units evenly
    const int nb = g1.nb;
    const int64_t U = static_cast<int64_t>(n_active) * nb;
    const int u0 = static_cast<int>(U * blockIdx.x / g1.nwg);
    const int u1 = static_cast<int>(U * (blockIdx.x + 1) / g1.nwg);
    for (int a = u0 / nb; a < n_active && a * nb < u1; ++a) {
      const int c = min(u1, (a + 1) * nb) - max(u0, a * nb);
      if (c > 0) __hip_atomic_fetch_add(sync + a, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  one_launch_stage<false, NA, true>(p2, g2, area, queue, poison, ract, roff, rsorted, n_active,
                                    sync, g1.nb);

  // the last workgroup out (every other one is past its waits) resets the counts
  __syncthreads();
  if (threadIdx.x == 0)
    poison = __hip_atomic_fetch_add(sync + kOneLaunchMaxSlots, 1, __ATOMIC_ACQ_REL,
                                    __HIP_MEMORY_SCOPE_AGENT) == static_cast<int>(gridDim.x) - 1;
  __syncthreads();
  if (poison) {
    for (int a = threadIdx.x; a <= kOneLaunchMaxSlots; a += kThreads)
      __hip_atomic_store(sync + a, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Stage 2 with the combine folded in, for T <= 2 tokens (an expert then holds
// one or two rows): workgroup b takes block b (R = 64 / C output rows) of
// every active expert, so the block's y rows of every token end up in one
// workgroup.  All S = T top_k act rows are staged in LDS once; wave w takes
// the active experts w, w + 8, ...; each lane cluster issues all spb loads of
// its row before using any.  The rows' sums are the stage-2 GEMV's, in the
// same order, bit for bit; they go to y_sorted and to LDS, where the
// workgroup then adds each token's rows with the router weights, j ascending
// from zero, and rounds once to fp16 (the combine kernel's order).
constexpr int kFoldMaxSpb = 8;   // steps per lane held in registers
constexpr int kFoldWaves = 8;    // 512 threads: 256 registers a lane for the held steps
constexpr int kFoldThreads = 64 * kFoldWaves;

__global__ __launch_bounds__(kFoldThreads) void down_fold_kernel(DecodeArgs p, Geom geo) {
  extern __shared__ __align__(16) uint32_t lds[];
  const int G = geo.G, C = geo.C, spb = geo.spb;
  const int H = p.H, I = p.I;
  const int R = 64 / C;
  const int S = p.T * p.top_k;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int k = lane / C, lc = lane & (C - 1);
  const int b = static_cast<int>(blockIdx.x);
  uint32_t* frags = lds;  // [S][hi, lo][G]
  float* ybuf = reinterpret_cast<float*>(frags + static_cast<size_t>(S) * 2 * G * kFragDwords);
  for (int i = threadIdx.x; i < S * 2 * G; i += kFoldThreads) {
    const int rf = i / G;  // row r = rf / 2, hi (0) or lo (1) = rf % 2
    const int g = i - rf * G;
    const uint16_t* src = ((rf & 1) ? p.a_lo : p.a_hi) + static_cast<size_t>(rf >> 1) * I;
    stage_frag(src + 32 * g, frags + i * kFragDwords);
  }
  __syncthreads();
  const int n_active = *p.num_active;
  const int n = b * R + k;
  const uint32_t row = n < H ? static_cast<uint32_t>(n) : static_cast<uint32_t>(H);  // past: zeros
  // a unit (one active expert's block): its loads, then its sums
  auto issue = [&](int e, Slot (&sl)[kFoldMaxSpb], uint32_t (&sh)[kFoldMaxSpb]) {
    const ExpertBufs bufs = expert_bufs(p, H, G, e);
#pragma unroll
    for (int j = 0; j < kFoldMaxSpb; ++j) {
      if (j < spb) {
        const int gg = j * C + lc;
        issue_step(bufs, G, row, gg, sl[j]);
        sh[j] = __builtin_amdgcn_raw_buffer_load_b16(
            bufs.s, static_cast<int>((row * static_cast<uint32_t>(G) + gg) * 2u), 0, 0);
      }
    }
  };
  auto finish = [&](int e, const Slot (&sl)[kFoldMaxSpb], const uint32_t (&sh)[kFoldMaxSpb]) {
    const int r0 = p.offsets[e];
    const int nr = min(2, p.offsets[e + 1] - r0);
    float acc0 = 0.f, acc1 = 0.f;
    const uint32_t* f0 = frags + static_cast<size_t>(r0) * 2 * G * kFragDwords;
    const uint32_t* f1 = f0 + 2 * G * kFragDwords;
#pragma unroll
    for (int j = 0; j < kFoldMaxSpb; ++j) {
      if (j < spb) {
        const int gg = j * C + lc;
        const float scale = half_bits_to_float(static_cast<uint16_t>(sh[j]));
        const float z = static_cast<float>((sl[j].zw >> (4u * (row & 7u))) & 0xFu);
        const Codes codes = expand_codes(sl[j].q);
        float d0 = group_dot(codes, z, read_frag(f0 + gg * kFragDwords));
        d0 += group_dot(codes, z, read_frag(f0 + (G + gg) * kFragDwords));
        acc0 = fmaf(scale, d0, acc0);
        if (nr > 1) {
          float d1 = group_dot(codes, z, read_frag(f1 + gg * kFragDwords));
          d1 += group_dot(codes, z, read_frag(f1 + (G + gg) * kFragDwords));
          acc1 = fmaf(scale, d1, acc1);
        }
      }
    }
    const float v0 = cluster_sum(acc0, C);
    const float v1 = cluster_sum(acc1, C);
    if (lc == 0 && n < H) {
      p.y[static_cast<size_t>(r0) * H + n] = v0;
      ybuf[r0 * R + k] = v0;
      if (nr > 1) {
        p.y[static_cast<size_t>(r0 + 1) * H + n] = v1;
        ybuf[(r0 + 1) * R + k] = v1;
      }
    }
  };
  // Experts a and a + kFoldWaves together: the second one's loads are out
  // before the first one's sums (10 experts over 8 waves at 1 token: two
  // waves hold two, and their second expert no longer waits on the first).
  for (int a = wave; a < n_active; a += 2 * kFoldWaves) {
    const bool two = a + kFoldWaves < n_active;
    const int e = p.active[a];
    const int e2 = p.active[two ? a + kFoldWaves : a];
    Slot sl[kFoldMaxSpb], sl2[kFoldMaxSpb];
    uint32_t sh[kFoldMaxSpb], sh2[kFoldMaxSpb];
    issue(e, sl, sh);
    if (two) issue(e2, sl2, sh2);
    finish(e, sl, sh);
    if (two) finish(e2, sl2, sh2);
  }
  __syncthreads();
  for (int i = static_cast<int>(threadIdx.x); i < p.T * R; i += kFoldThreads) {
    const int t = i / R;
    const int r = i - t * R;
    if (b * R + r < H) {
      float acc = 0.f;
      for (int j = 0; j < p.top_k; ++j) {
        const int sl = t * p.top_k + j;
        acc = fmaf(p.c_weights[sl], ybuf[p.c_slot_rows[sl] * R + r], acc);
      }
      p.out[static_cast<size_t>(t) * H + b * R + r] = float_to_half_bits(acc);
    }
  }
}

// ----------------------------------------------------------------- host -----

// LDS bytes of the A fragments: kXE experts x na rows (stage 2: hi and lo).
template <bool GATE_UP>
size_t frag_bytes(const Geom& geo, int na) {
  return static_cast<size_t>(kXE) * na * (GATE_UP ? 1 : 2) * geo.G * kFragDwords * 4;
}

// Rows per expert per pass (a template value of the kernel) and the window
// size, from the LDS a workgroup may hold.  Windows aim to cover a
// workgroup's whole share of units, which is at most ceil(slots * nb / nwg).
template <bool GATE_UP>
struct WindowBudget {
  size_t budget;  // LDS bytes for fragments and unit slots
  size_t unit;    // bytes of one unit slot
  int want;       // units of the largest share, plus one
  WindowBudget(const Geom& geo, int slots, const DeviceInfo& dev, size_t reserved)
      : budget(static_cast<size_t>(dev.lds) - kDecodeStaticLds - reserved),
        unit(static_cast<size_t>(unit_scale_halves(geo.spb)) * 2),
        want(static_cast<int>((static_cast<int64_t>(slots) * geo.nb + geo.nwg - 1) / geo.nwg) + 1) {}
  // na rows per pass leave room for a useful window
  bool roomy(const Geom& geo, int na) const {
    return frag_bytes<GATE_UP>(geo, na) + unit * min(want, 16) <= budget;
  }
  // the window size that fills the rest of the budget
  void set_wmax(Geom& geo, int na) const {
    const size_t fb = frag_bytes<GATE_UP>(geo, na);
    const size_t rest = budget > fb ? budget - fb : 0;
    size_t w = rest / unit;
    if (w > static_cast<size_t>(want)) w = want;
    geo.wmax = w < 1 ? 1 : static_cast<int>(w);
  }
};

template <bool GATE_UP>
int plan(Geom& geo, int slots, const DeviceInfo& dev, size_t reserved, int rows_per_pass) {
  const WindowBudget<GATE_UP> wb(geo, slots, dev, reserved);
  // the plan's rows per pass; stage 2 stops at 4 (eight rows of hi and lo
  // fragments would spill registers), and fewer when LDS is short
  int na = GATE_UP ? rows_per_pass : min(rows_per_pass, 4);
  while (na > 1 && !wb.roomy(geo, na)) na /= 2;
  wb.set_wmax(geo, na);
  return na;
}

template <bool GATE_UP>
size_t launch_lds(const Geom& geo, int na) {
  return frag_bytes<GATE_UP>(geo, na) +
         static_cast<size_t>(geo.wmax) * unit_scale_halves(geo.spb) * 2 +
         static_cast<size_t>(geo.ucap) * 4;
}

// Ints of the unit-cost table for `slots` active experts at most: the prefix
// and the block scan's wave totals, rounded to 16 bytes.
int cost_table_ints(int slots) { return (slots + 1 + kScanThreads / 64 + 1 + 3) & ~3; }

template <bool GATE_UP, int NPL>
void launch_decode_npl(const DecodeArgs& p, Geom geo, int na, size_t lds, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(geo.nwg + p.shared_wgs)), block(kThreads);
  if constexpr (GATE_UP) {
    if (na == 8) {
      hipLaunchKernelGGL((decode_kernel<GATE_UP, 8, NPL>), grid, block, lds, stream, p, geo);
      return;
    }
  }
  if (na == 4)
    hipLaunchKernelGGL((decode_kernel<GATE_UP, 4, NPL>), grid, block, lds, stream, p, geo);
  else if (na == 2)
    hipLaunchKernelGGL((decode_kernel<GATE_UP, 2, NPL>), grid, block, lds, stream, p, geo);
  else
    hipLaunchKernelGGL((decode_kernel<GATE_UP, 1, NPL>), grid, block, lds, stream, p, geo);
}

// route: stage 1 routes the tokens itself (p.logits, p.E <= 1024, T <= 64).
template <bool GATE_UP>
void launch_decode(const DecodeArgs& p, Geom geo, int slots, hipStream_t stream, bool route,
                   int rows_per_pass, int cost_split) {
  // (p.E is set by every caller: the share arithmetic's width depends on it)
  const DeviceInfo dev = device_info();
  geo.nwg = dev.cus - p.shared_wgs;  // with the shared expert's workgroups, one per compute unit
  geo.weighted = cost_split && slots <= kThreads;  // the cost scan: one expert per thread
  geo.ucap = geo.weighted ? cost_table_ints(slots) : 0;
  const size_t rbytes = route ? route_lds_bytes(p.E, p.T * p.top_k) : 0;
  const int na =
      plan<GATE_UP>(geo, slots, dev, rbytes + static_cast<size_t>(geo.ucap) * 4, rows_per_pass);
  size_t lds = launch_lds<GATE_UP>(geo, na) + rbytes;  // the cost table included
  if (p.shared_wgs > 0)
    lds = std::max(lds, shared_lds_bytes(GATE_UP, p.T, GATE_UP ? p.H : p.I));
  if constexpr (GATE_UP) {
    if (route) {
      const int El = p.E - p.shared;  // logits per token
      if (El <= 64) return launch_decode_npl<true, 1>(p, geo, na, lds, stream);
      if (El <= 128) return launch_decode_npl<true, 2>(p, geo, na, lds, stream);
      if (El <= 256) return launch_decode_npl<true, 4>(p, geo, na, lds, stream);
      if (El <= 512) return launch_decode_npl<true, 8>(p, geo, na, lds, stream);
      return launch_decode_npl<true, 16>(p, geo, na, lds, stream);
    }
  }
  launch_decode_npl<GATE_UP, 0>(p, geo, na, lds, stream);
}

// The shared expert (the last expert, holding the last T sorted rows) on the
// matrix cores: column tiles of 16 gate columns (stage 1) or 32 output
// columns (stage 2), ShCfg::kTiles of them per extra workgroup.
template <bool GATE_UP>
void set_shared(DecodeArgs& p, int shared_mfma, int T, int top_k, int I, int H) {
  if (!shared_mfma) {
    p.shared_wgs = 0;
    p.shared_row0 = 0;
    return;
  }
  const int tiles = GATE_UP ? (I + 15) / 16 : (H + 31) / 32;
  p.shared_wgs = (tiles + ShCfg<GATE_UP>::kTiles - 1) / ShCfg<GATE_UP>::kTiles;
  p.shared_row0 = T * (top_k - 1);
}

}  // namespace

// The least LDS a GEMV stage can run with: one A row per pass, one unit per
// window, plus the routing and cost tables it keeps.
size_t down_fold_lds(int64_t T, int top_k, int I, int lanes) {
  const size_t S = static_cast<size_t>(T) * top_k;
  const size_t b = S * 2 * (I / kGroup) * kFragDwords * 4 + S * (64 / lanes) * 4;
  return (b + 15) & ~static_cast<size_t>(15);
}

bool down_fold_ok(int64_t T, int top_k, int I, int lanes, size_t lds_bytes) {
  return T <= 2 && (I / kGroup) / lanes <= kFoldMaxSpb &&
         down_fold_lds(T, top_k, I, lanes) + kDecodeStaticLds <= lds_bytes;
}

size_t gemv_min_lds(bool gate_up, bool route, int64_t T, int top_k, int E, int H, int I,
                    int lanes, bool cost_split) {
  Geom geo{};
  geo.G = (gate_up ? H : I) / kGroup;
  geo.C = lanes;
  geo.spb = geo.G / geo.C;
  const int slots = static_cast<int>(std::min<int64_t>(E, T * top_k));
  const size_t frags = gate_up ? frag_bytes<true>(geo, 1) : frag_bytes<false>(geo, 1);
  size_t need = frags + static_cast<size_t>(unit_scale_halves(geo.spb)) * 2 + kDecodeStaticLds;
  if (route) need += route_lds_bytes(E, static_cast<int>(T * top_k));
  if (cost_split && slots <= kThreads) need += static_cast<size_t>(cost_table_ints(slots)) * 4;
  return need;
}

// LDS the shared expert's matrix-core workgroups take at T tokens: the larger
// of the two stages.
size_t shared_mfma_lds(int64_t T, int H, int I) {
  const int t = static_cast<int>(std::min<int64_t>(T, 32));
  return std::max(shared_lds_bytes(true, t, H), shared_lds_bytes(false, t, I));
}

void launch_gate_up_decode(const GateUpArgs& a, const FfnWorkspace& ws, hipStream_t stream) {
  Geom geo{};
  geo.G = a.H / kGroup;
  geo.C = a.lanes;  // a power of two <= 16 dividing G (the plan)
  geo.spb = geo.G / geo.C;
  const int half = (64 / geo.C) / 2;  // gate (= up) rows per block
  geo.nb = (a.I + half - 1) / half;
  DecodeArgs p{};
  p.x = a.x;
  p.offsets = a.offsets;
  p.sorted_slots = a.sorted_slots;
  p.active = a.active;
  p.num_active = a.num_active;
  p.qw = a.qw;
  p.sc = a.sc;
  p.qz = a.qz;
  p.T = a.T;
  p.top_k = a.top_k;
  p.H = a.H;
  p.I = a.I;
  p.E = a.E;
  p.act_hi = ws.act_hi;
  p.act_lo = ws.act_lo;
  p.cost_out = ws.tiles;  // the tile list region is free at decode sizes
  set_shared<true>(p, a.shared_mfma, a.T, a.top_k, a.I, a.H);
  launch_decode<true>(p, geo, min(a.E, a.T * a.top_k), stream, false, a.rows_per_pass, a.cost_split);
}

void launch_route_gate_up_decode(const float* logits, const GateUpArgs& a, const RouteOut& r,
                                 const FfnWorkspace& ws, hipStream_t stream) {
  Geom geo{};
  geo.G = a.H / kGroup;
  geo.C = a.lanes;
  geo.spb = geo.G / geo.C;
  const int half = (64 / geo.C) / 2;
  geo.nb = (a.I + half - 1) / half;
  DecodeArgs p{};
  p.x = a.x;
  p.qw = a.qw;
  p.sc = a.sc;
  p.qz = a.qz;
  p.T = a.T;
  p.top_k = a.top_k;
  p.H = a.H;
  p.I = a.I;
  p.act_hi = ws.act_hi;
  p.act_lo = ws.act_lo;
  p.cost_out = ws.tiles;
  set_shared<true>(p, a.shared_mfma, a.T, a.top_k, a.I, a.H);
  p.logits = logits;
  p.E = a.E;
  p.shared = a.shared;
  p.r_ids = r.ids;
  p.r_weights = r.weights;
  p.r_offsets = r.offsets;
  p.r_sorted = r.sorted_slots;
  p.r_slot_rows = r.slot_rows;
  p.r_active = r.active;
  p.r_num_active = r.num_active;
  launch_decode<true>(p, geo, min(a.E, a.T * a.top_k), stream, true, a.rows_per_pass, a.cost_split);
}

void launch_down_decode(const DownArgs& a, const FfnWorkspace& ws, hipStream_t stream) {
  Geom geo{};
  geo.G = a.I / kGroup;
  geo.C = a.lanes;
  geo.spb = geo.G / geo.C;
  geo.nb = (a.H + 64 / geo.C - 1) / (64 / geo.C);
  DecodeArgs p{};
  p.a_hi = ws.act_hi;
  p.a_lo = ws.act_lo;
  p.offsets = a.offsets;
  p.active = a.active;
  p.num_active = a.num_active;
  p.qw = a.qw;
  p.sc = a.sc;
  p.qz = a.qz;
  p.T = a.T;
  p.top_k = a.top_k;
  p.H = a.H;
  p.I = a.I;
  p.E = a.E;
  p.y = a.y;
  p.cost_in = ws.tiles;  // written by the gate/up kernel
  if (a.combine) {  // T <= 2, no shared-expert workgroups (the plan's check)
    p.c_weights = a.c_weights;
    p.c_slot_rows = a.c_slot_rows;
    p.out = a.out;
    hipLaunchKernelGGL(down_fold_kernel, dim3(static_cast<unsigned>(geo.nb)), dim3(kFoldThreads),
                       down_fold_lds(a.T, a.top_k, a.I, a.lanes), stream, p, geo);
    return;
  }
  set_shared<false>(p, a.shared_mfma, a.T, a.top_k, a.I, a.H);
  launch_decode<false>(p, geo, min(a.E, a.T * a.top_k), stream, false, a.rows_per_pass, a.cost_split);
}

// Gate/up and down in one launch (one_launch_kernel): the two stages'
// geometry as the separate launches set it, even split, no shared-expert
// workgroups; both stages take the same rows per pass (the largest <= 4 that
// leaves both of them a useful window), each its own window size.
void launch_one_launch_decode(const float* logits, const GateUpArgs& a, const DownArgs& d,
                              const RouteOut& r, const FfnWorkspace& ws, hipStream_t stream) {
  const DeviceInfo dev = device_info();
  Geom g1{}, g2{};
  g1.G = a.H / kGroup;
  g1.C = a.lanes;
  g1.spb = g1.G / g1.C;
  g1.nb = (a.I + (64 / g1.C) / 2 - 1) / ((64 / g1.C) / 2);
  g2.G = a.I / kGroup;
  g2.C = d.lanes;
  g2.spb = g2.G / g2.C;
  g2.nb = (a.H + 64 / g2.C - 1) / (64 / g2.C);
  g1.nwg = g2.nwg = dev.cus;
  DecodeArgs p1{};
  p1.x = a.x;
  p1.qw = a.qw;
  p1.sc = a.sc;
  p1.qz = a.qz;
  p1.T = a.T;
  p1.top_k = a.top_k;
  p1.H = a.H;
  p1.I = a.I;
  p1.E = a.E;
  p1.act_hi = ws.act_hi;
  p1.act_lo = ws.act_lo;
  p1.logits = logits;
  p1.r_ids = r.ids;
  p1.r_weights = r.weights;
  p1.r_offsets = r.offsets;
  p1.r_sorted = r.sorted_slots;
  p1.r_slot_rows = r.slot_rows;
  p1.r_active = r.active;
  p1.r_num_active = r.num_active;
  DecodeArgs p2{};
  p2.a_hi = ws.act_hi;
  p2.a_lo = ws.act_lo;
  p2.qw = d.qw;
  p2.sc = d.sc;
  p2.qz = d.qz;
  p2.T = d.T;
  p2.top_k = d.top_k;
  p2.H = d.H;
  p2.I = d.I;
  p2.E = d.E;
  p2.y = d.y;
  const int slots = min(a.E, a.T * a.top_k);
  const size_t rbytes = route_lds_bytes(a.E, a.T * a.top_k);
  const WindowBudget<true> b1(g1, slots, dev, rbytes);
  const WindowBudget<false> b2(g2, slots, dev, rbytes);
  int na = min(a.rows_per_pass, 4);
  while (na > 1 && !(b1.roomy(g1, na) && b2.roomy(g2, na))) na /= 2;
  b1.set_wmax(g1, na);
  b2.set_wmax(g2, na);
  const size_t lds = rbytes + std::max(launch_lds<true>(g1, na), launch_lds<false>(g2, na));
  const dim3 grid(static_cast<unsigned>(dev.cus)), block(kThreads);
  const int tb = static_cast<int>(rbytes);
  if (a.E <= 512) {
    if (na == 4)
      hipLaunchKernelGGL((one_launch_kernel<4, 8>), grid, block, lds, stream, p1, g1, p2, g2, tb);
    else if (na == 2)
      hipLaunchKernelGGL((one_launch_kernel<2, 8>), grid, block, lds, stream, p1, g1, p2, g2, tb);
    else
      hipLaunchKernelGGL((one_launch_kernel<1, 8>), grid, block, lds, stream, p1, g1, p2, g2, tb);
  } else {
    if (na == 4)
      hipLaunchKernelGGL((one_launch_kernel<4, 16>), grid, block, lds, stream, p1, g1, p2, g2, tb);
    else if (na == 2)
      hipLaunchKernelGGL((one_launch_kernel<2, 16>), grid, block, lds, stream, p1, g1, p2, g2, tb);
    else
      hipLaunchKernelGGL((one_launch_kernel<1, 16>), grid, block, lds, stream, p1, g1, p2, g2, tb);
  }
}

// The least LDS the one-launch FFN runs with: the routing tables and the
// larger of the two stages at one A row per pass and one unit per window.
size_t one_launch_min_lds(int64_t T, int top_k, int E, int H, int I, int lanes_gate_up,
                          int lanes_down) {
  return std::max(gemv_min_lds(true, true, T, top_k, E, H, I, lanes_gate_up, false),
                  gemv_min_lds(false, true, T, top_k, E, H, I, lanes_down, false));
}

}  // namespace moe
