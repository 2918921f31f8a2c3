// Matrix-core grouped expert FFN for larger token counts (prefill).
//
// Same two stages as the decode path ("[Perf][SM70] Narrow Qwen3.8 AWQ active
// grouped decode", section "Purpose": a grouped W4A16 operator over the
// active experts' multi-row segments; group size 32 along K):
//   stage 1: act[r, c] = SiLU(h_gate) * h_up,  h = x[token(r)] . W13[e]^T
//   stage 2: y_sorted[r, n] = act[r] . W2[e]^T
// as dense tiles on v_mfma_f32_32x32x16_f16.
//
// Schedule.  A tile list cuts every active expert's segment of sorted rows
// into M-tiles of MSUB * 32 rows (a heavily loaded expert becomes many tiles).
// A workgroup computes one M-tile against an N-tile of 128 weight rows; each
// of its 4 waves owns 32 weight rows and all of the M-tile's rows, so one
// dequantised weight fragment feeds MSUB matrix instructions.  Work items
// are numbered M-tile-major and every XCD takes a contiguous run of them, so
// the workgroups of one XCD share the A rows of an M-tile and, one expert at a
// time, that expert's weights in their L2.
//
// Operands.  One quantisation group (K = 32) is two MFMAs chained into a
// partial P = A . (q - z) with an exact integer B (q - z is an integer in
// [-15, 15], exact in fp16) and a zero accumulator; P is then scaled in fp32:
// acc += s[n, g] * P.  Rounding the dequantised weight to fp16 instead would
// cost as much precision as rounding act to fp16, which the layer tolerance
// does not allow.  Within each 8-wide k block the k order is
// (0, 4, 1, 5, 2, 6, 3, 7), the order in which the nibble unpack produces
// (q - z) pairs, so A is stored permuted the same way: x by a pre-pass, act
// by the stage-1 epilogue.  A lane of half h of the wave supplies, for MFMA t
// of a group, 8-value block 2h + t.  Stage 2: the two wave halves load the
// codes of two consecutive groups (16 bytes per lane), and two
// v_permlane32_swap exchanges give every lane its two blocks of each group.
// Stage 1: kKC lanes read a row's kKC consecutive groups (so one load
// instruction covers 64 / kKC rows of contiguous bytes instead of 32 rows of
// 32 bytes), and each wave passes its codes through a private LDS area from
// which every lane reads its two blocks of each group.  Stage 2 runs
// act_hi and act_lo through the same partial (act carried at about 22 bits).
//
// Staging.  A rows go through LDS in fragment order (one 1 KiB block per
// (group, 32-row subtile, MFMA), lane L at byte 16 L, so every fragment read
// is one contiguous ds_read_b128 per lane), kKC groups per stage, double
// buffered; weights, zeros and scales are read by each lane straight into
// registers with buffer loads (out-of-range reads return zeros), one stage
// ahead.
#include <math.h>

#include <algorithm>

#include "common.h"

namespace moe {
namespace {


constexpr int kSub = 32;                   // MFMA tile edge
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = kWaves * kSub;         // weight rows per N-tile
constexpr int kBlockHalfs = 64 * 8;        // one fragment block: 64 lanes x 8 fp16
constexpr int kBufferFlags = 0x00020000;   // buffer descriptor word 3 for raw dword access on gfx9
// Cost of a work item: kSubCost per live 32-row subtile plus kItemBase
// (weight streaming and per-group vector work do not shrink with the rows).
// Measured item durations grow about 11 us per subtile above a 17 us floor
// at the 4096-token shape, a base about 1.5 times the per-subtile cost.
constexpr int kSubCost = 2;
constexpr int kItemBase = 3;

// Groups per LDS stage: deeper for 32-row tiles, which stream weights with
// little arithmetic per byte, so more bytes must be in flight per wave.
template <bool GATE_UP, int MSUB>
struct StageCfg {
  static constexpr int kCopies = GATE_UP ? 1 : 2;   // A copies: x, or act hi + lo
  static constexpr int kKC = (GATE_UP ? 4 : 2) * (MSUB == 1 ? 2 : 1);
  // codes through LDS (stage 1; 1024 tokens: gate/up 304 us against 328 with
  // the lane-half loads and swaps; stage 2 kept the swaps: the LDS area cost
  // its 32-row kernel a workgroup per compute unit, 212 against 198 us)
  static constexpr bool kCodesLds = GATE_UP;
};

// Per-wave LDS copy of a stage's codes: 32 rows of KC groups (16 bytes each),
// row stride KC x 16 + 8 bytes, so that the 32 rows' 8-byte reads of one
// group fall on distinct banks (the stride in banks, 4 KC + 2, is twice an
// odd number).
template <int KC>
struct CodesLds {
  static constexpr int kStride = KC * 16 + 8;
  static constexpr int kWaveBytes = 32 * kStride;
};

struct PrefillArgs {
  const uint16_t* a_hi;        // stage 1: permuted x [T, H]; stage 2: act_hi [S, I]
  const uint16_t* a_lo;        // stage 2: act_lo [S, I]
  const int* sorted_slots;     // stage 1 row gather
  int T, top_k, E, H, I;
  const int* offsets;
  const int* tiles;
  const int* tile_count;
  const int* qw;
  const uint16_t* sc;
  const int* qz;
  uint16_t* act_hi;            // stage 1 outputs
  uint16_t* act_lo;
  float* y;                    // stage 2 output
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           kBufferFlags);
}

// Per-lane weight operands of one stage: codes of kKC / 2 group pairs (lane
// half h loads group 2p + h of pair p), one zero word per group and the
// group scales packed two per dword.
template <int KC>
struct BRegs {
  uint4 q[KC / 2];
  uint32_t z[KC];
  uint32_t s[(KC + 1) / 2];
  __device__ __forceinline__ uint32_t scale(int g) const { return (s[g >> 1] >> (16 * (g & 1))) & 0xFFFFu; }
};

struct BAddr {
  __amdgpu_buffer_rsrc_t rq, rs, rz;
  uint32_t q_rows[4];                 // codes: first byte of the row of load pp
  uint32_t qg;                        // codes: group of load pp, less 2 pp (lane swaps)
  uint32_t s_row, z_row;              // byte offsets of the first group of the lane's row
  uint32_t q_oob, s_oob, z_oob;       // offsets that read as zero
  int G;
};

// Loads of one stage's weight operands.  The whole byte offset of every load
// is in the vector offset (the scalar offset is 0), so the buffer's range
// check covers the full address: a lane past the matrix reads at or beyond
// the end of the buffer and gets zeros without touching memory.  Groups are
// clamped to the lane's own row: a stage past the end of K re-reads the row's
// last valid groups, which the compute skips.  VEC (the group count is a
// multiple of kKC): a stage's zero words and scales of one row are contiguous
// and aligned, and are read with one wide load each.
template <int KC, bool VEC, bool CODES_LDS>
__device__ __forceinline__ void load_b_stage(const BAddr& ba, int g0, BRegs<KC>& b) {
#pragma unroll
  for (int pp = 0; pp < KC / 2; ++pp) {
    // lane swaps: lane half h loads group g0 + 2 pp + h of its own row;
    // codes through LDS: group g0 + L % KC of row 64 / KC pp + L / KC
    const int gl = g0 + static_cast<int>(ba.qg) + (CODES_LDS ? 0 : 2 * pp);
    const uint32_t g = static_cast<uint32_t>(min(gl, ba.G - 1));
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(ba.rq, static_cast<int>(ba.q_rows[pp] + g * 16u), 0, 0);
    b.q[pp] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  if constexpr (VEC) {
    const uint32_t gs = static_cast<uint32_t>(min(g0, ba.G - KC));
    if constexpr (KC == 2) {
      const auto z = __builtin_amdgcn_raw_buffer_load_b64(ba.rz, static_cast<int>(ba.z_row + gs * 4u), 0, 0);
      b.z[0] = z[0];
      b.z[1] = z[1];
    } else {
#pragma unroll
      for (int i = 0; i < KC; i += 4) {
        const auto z = __builtin_amdgcn_raw_buffer_load_b128(
            ba.rz, static_cast<int>(ba.z_row + (gs + i) * 4u), 0, 0);
        for (int t = 0; t < 4; ++t) b.z[i + t] = z[t];
      }
    }
    const int so = static_cast<int>(ba.s_row + gs * 2u);
    if constexpr (KC == 8) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(ba.rs, so, 0, 0);
      for (int t = 0; t < 4; ++t) b.s[t] = v[t];
    } else if constexpr (KC == 4) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(ba.rs, so, 0, 0);
      b.s[0] = v[0];
      b.s[1] = v[1];
    } else {
      b.s[0] = __builtin_amdgcn_raw_buffer_load_b32(ba.rs, so, 0, 0);
    }
  } else {
    uint32_t sv[KC];
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const uint32_t g = static_cast<uint32_t>(min(g0 + i, ba.G - 1));
      b.z[i] = __builtin_amdgcn_raw_buffer_load_b32(ba.rz, static_cast<int>(ba.z_row + g * 4u), 0, 0);
      sv[i] = __builtin_amdgcn_raw_buffer_load_b16(ba.rs, static_cast<int>(ba.s_row + g * 2u), 0, 0);
    }
#pragma unroll
    for (int i = 0; i < KC; i += 2) b.s[i / 2] = sv[i] | (i + 1 < KC ? sv[i + 1] << 16 : 0u);
  }
}

// A staging.  8 threads share a row, so each load instruction reads 128
// contiguous bytes of 8 rows; a pass of the 256 threads covers one 32-row
// subtile, and each thread loads kCPP chunks of 16 bytes per pass.  A row's
// stage span is kCopies x kKC groups x 4 chunks.  Rows past the tile read
// past the end of the buffer (zeros, no traffic).
template <bool GATE_UP, int MSUB>
struct AStage {
  static constexpr int kKC = StageCfg<GATE_UP, MSUB>::kKC;
  static constexpr int kCopies = StageCfg<GATE_UP, MSUB>::kCopies;
  static constexpr int kBM = MSUB * kSub;
  static constexpr int kTPR = 8;                               // threads per row
  static constexpr int kCPR = kCopies * kKC * 4;               // chunks per row per stage
  static constexpr int kCPP = kCPR / kTPR;                     // chunks per thread per pass
  static constexpr int kStageHalfs = kCopies * kKC * MSUB * 2 * kBlockHalfs;
  static_assert(kThreads / kTPR == kSub, "one pass of the workgroup stages one subtile");
  static_assert(kCPR % kTPR == 0, "stage chunks must split evenly over a row's threads");
  uint4 v[MSUB][kCPP];
};

struct ASrc {
  __amdgpu_buffer_rsrc_t r[2];   // copy 0 (x or act_hi), copy 1 (act_lo)
  uint32_t row_off[4];           // byte offset of this thread's row of subtile i
};

// XOR applied to the 16-byte slot of a fragment block, so that the 8 threads
// staging one row (chunk c of groups 2m and 2m + 1) write 8 different bank
// groups, while the 8 lanes of any aligned octet still read distinct ones.
__device__ __forceinline__ int slot_xor(int g, int h, int t) { return ((g & 1) << 2) | (h << 1) | t; }

// The whole byte offset is in the vector offset, and a group past the end of
// K is clamped to the row's last group (the compute skips it), so every load
// stays inside the row it stages; rows past the tile start at or beyond the
// end of the buffer and read zeros.
template <bool GATE_UP, int MSUB, int NS>
__device__ __forceinline__ void load_a(uint32_t tid, const ASrc& src, int g0, int G,
                                       AStage<GATE_UP, MSUB>& a) {
  using S = AStage<GATE_UP, MSUB>;
  const int t8 = static_cast<int>(tid % S::kTPR);
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int k = 0; k < S::kCPP; ++k) {
      const int cc = k * S::kTPR + t8;
      const int cp = cc / (S::kKC * 4);
      const int g = (cc / 4) % S::kKC;
      const int c = cc % 4;
      const uint32_t ga = static_cast<uint32_t>(min(g0 + g, G - 1));
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(
          src.r[cp], static_cast<int>(src.row_off[i] + ga * (kGroup * 2) + c * 16), 0, 0);
      a.v[i][k] = make_uint4(v[0], v[1], v[2], v[3]);
    }
}

template <bool GATE_UP, int MSUB, int NS>
__device__ __forceinline__ void store_a(uint32_t tid, const AStage<GATE_UP, MSUB>& a, uint16_t* stage) {
  using S = AStage<GATE_UP, MSUB>;
  const int j = static_cast<int>(tid / S::kTPR) & (kSub - 1);
  const int t8 = static_cast<int>(tid % S::kTPR);
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int k = 0; k < S::kCPP; ++k) {
      const int cc = k * S::kTPR + t8;
      const int cp = cc / (S::kKC * 4);
      const int g = (cc / 4) % S::kKC;
      const int c = cc % 4;
      const int block = ((cp * S::kKC + g) * MSUB + i) * 2 + (c & 1);
      const int slot = (32 * (c >> 1) + j) ^ slot_xor(g, c >> 1, c & 1);
      *reinterpret_cast<uint4*>(stage + block * kBlockHalfs + slot * 8) = a.v[i][k];
    }
}

// A stage's codes (as loaded for CodesLds) into the wave's LDS area.
template <int KC>
__device__ __forceinline__ void write_codes(uint32_t tid, const BRegs<KC>& b, uint8_t* cw) {
  const int lane = static_cast<int>(tid & 63);
#pragma unroll
  for (int pp = 0; pp < KC / 2; ++pp) {
    uint8_t* d = cw + CodesLds<KC>::kStride * ((64 / KC) * pp + lane / KC) + 16 * (lane % KC);
    *reinterpret_cast<uint2*>(d) = make_uint2(b.q[pp].x, b.q[pp].y);
    *reinterpret_cast<uint2*>(d + 8) = make_uint2(b.q[pp].z, b.q[pp].w);
  }
}

// One stage of the main loop: NG groups (NG < kKC only in a tail stage) of a
// tile with NS live 32-row subtiles.  The scaling of each partial is issued
// after the next partial's MFMAs, so it does not wait on its own MFMA.
template <bool GATE_UP, int MSUB, int NS, int NG>
__device__ __forceinline__ void compute_stage(uint32_t tid, const uint16_t* stage,
                                              const BRegs<StageCfg<GATE_UP, MSUB>::kKC>& b,
                                              const uint8_t* cw, uint32_t zshift, uint32_t bias,
                                              float16v (&acc)[MSUB]) {
  constexpr int KC = StageCfg<GATE_UP, MSUB>::kKC;
  constexpr int kLoOff = KC * MSUB * 2 * kBlockHalfs;   // act_lo copy
  const int lane = static_cast<int>(tid & 63);
  float16v pend = {};
  float pend_s = 0.f;
#pragma unroll
  for (int pp = 0; pp < (NG + 1) / 2; ++pp) {
    // lane half h needs words 2 h and 2 h + 1 of groups 2 pp and 2 pp + 1
    // of its row
    uint32_t words[2][2];   // [group][MFMA]
    if constexpr (StageCfg<GATE_UP, MSUB>::kCodesLds) {
      const int jj = lane & 31, hh = lane >> 5;
      const uint8_t* r = cw + CodesLds<KC>::kStride * jj + 8 * hh;
      const uint2 w0 = *reinterpret_cast<const uint2*>(r + 16 * (2 * pp));
      const uint2 w1 = *reinterpret_cast<const uint2*>(r + 16 * (2 * pp + 1));
      words[0][0] = w0.x; words[0][1] = w0.y; words[1][0] = w1.x; words[1][1] = w1.y;
    } else {
      // lane half 0 holds group 2pp, half 1 group 2pp + 1; after the swaps
      // the lower half holds words 0 and 1 and the upper half words 2 and 3
      const auto sx = __builtin_amdgcn_permlane32_swap(b.q[pp].x, b.q[pp].z, false, false);
      const auto sy = __builtin_amdgcn_permlane32_swap(b.q[pp].y, b.q[pp].w, false, false);
      words[0][0] = sx[0]; words[0][1] = sy[0]; words[1][0] = sx[1]; words[1][1] = sy[1];
    }
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int g = 2 * pp + gi;
      if (g >= NG) break;
      const uint32_t zc = (b.z[g] >> zshift) & 0xFu;
      const h2 m1024 = __builtin_bit_cast(h2, (0xE400u | zc) * 0x00010001u);
      const h2 m64 = __builtin_bit_cast(h2, (0xD400u | (zc << 4)) * 0x00010001u);
      const half8 b0 = dequant_word(words[gi][0], bias, m1024, m64);
      const half8 b1 = dequant_word(words[gi][1], bias, m1024, m64);
      float sf = half_bits_to_float(static_cast<uint16_t>(b.scale(g)));
      // converted once here: left foldable, every scaling FMA below becomes a
      // v_fma_mix_f32 (fp16 operand), which issues slower than v_fma_f32
      asm volatile("" : "+v"(sf));
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const uint16_t* blk = stage + ((g * MSUB + i) * 2) * kBlockHalfs;
        const int s0 = (lane ^ slot_xor(g, lane >> 5, 0)) * 8;
        const int s1 = (lane ^ slot_xor(g, lane >> 5, 1)) * 8 + kBlockHalfs;
        const half8 a0 = *reinterpret_cast<const half8*>(blk + s0);
        const half8 a1 = *reinterpret_cast<const half8*>(blk + s1);
        const float16v zero = {};
        float16v pr = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, zero, 0, 0, 0);
        pr = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, pr, 0, 0, 0);
        if (!GATE_UP) {
          const half8 l0 = *reinterpret_cast<const half8*>(blk + kLoOff + s0);
          const half8 l1 = *reinterpret_cast<const half8*>(blk + kLoOff + s1);
          pr = __builtin_amdgcn_mfma_f32_32x32x16_f16(l0, b0, pr, 0, 0, 0);
          pr = __builtin_amdgcn_mfma_f32_32x32x16_f16(l1, b1, pr, 0, 0, 0);
        }
        if (g > 0 || i > 0) {
          const int pi = i > 0 ? i - 1 : NS - 1;
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[pi][v] = fmaf(pend_s, pend[v], acc[pi][v]);
        }
        pend = pr;
        pend_s = sf;
      }
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[NS - 1][v] = fmaf(pend_s, pend[v], acc[NS - 1][v]);
}

// Tail stage of NG < kKC groups, NG chosen at run time.
template <bool GATE_UP, int MSUB, int NS, int NG>
__device__ __forceinline__ void compute_tail(uint32_t tid, int ng, const uint16_t* stage,
                                             const BRegs<StageCfg<GATE_UP, MSUB>::kKC>& b,
                                             const uint8_t* cw, uint32_t zshift, uint32_t bias,
                                             float16v (&acc)[MSUB]) {
  if constexpr (NG >= 1) {
    if (ng == NG) compute_stage<GATE_UP, MSUB, NS, NG>(tid, stage, b, cw, zshift, bias, acc);
    else compute_tail<GATE_UP, MSUB, NS, NG - 1>(tid, ng, stage, b, cw, zshift, bias, acc);
  }
}

template <bool GATE_UP, int MSUB, int NS, bool VEC>
__device__ __forceinline__ void main_loop(uint32_t tid, const ASrc& asrc, uint16_t* lds,
                                          const BAddr& ba, uint32_t zshift,
                                          float16v (&acc)[MSUB]) {
  using S = AStage<GATE_UP, MSUB>;
  constexpr int KC = S::kKC;
  const int G = ba.G;
  uint32_t bias;   // kept in a vector register so each mask-and-insert is one v_and_or_b32
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(bias));
  constexpr bool CL = StageCfg<GATE_UP, MSUB>::kCodesLds;
  const int nfull = G / KC;
  BRegs<KC> bcur, bnxt;
  AStage<GATE_UP, MSUB> astage;
  // the wave's codes area (stage 1), after the two A stages
  uint8_t* const cw = reinterpret_cast<uint8_t*>(lds + 2 * S::kStageHalfs) +
                      (static_cast<int>(tid >> 6) & (kWaves - 1)) * CodesLds<KC>::kWaveBytes;
  load_b_stage<KC, VEC, CL>(ba, 0, bcur);
  load_a<GATE_UP, MSUB, NS>(tid, asrc, 0, G, astage);
  store_a<GATE_UP, MSUB, NS>(tid, astage, lds);
  if constexpr (CL) write_codes<KC>(tid, bcur, cw);
  __syncthreads();
  for (int s = 0; s < nfull; ++s) {
    const int g0 = s * KC;
    // The next stage's loads are issued unconditionally (past the end of K
    // they read zeros or the following row), so every wait below is exact.
    load_b_stage<KC, VEC, CL>(ba, g0 + KC, bnxt);
    load_a<GATE_UP, MSUB, NS>(tid, asrc, g0 + KC, G, astage);
    // keep the loads ahead of the compute that hides their latency
    __builtin_amdgcn_sched_barrier(0);
    compute_stage<GATE_UP, MSUB, NS, KC>(tid, lds + (s & 1) * S::kStageHalfs, bcur, cw, zshift,
                                         bias, acc);
    __builtin_amdgcn_sched_barrier(0);
    store_a<GATE_UP, MSUB, NS>(tid, astage, lds + ((s + 1) & 1) * S::kStageHalfs);
    // the same wave read this stage's codes above: its LDS operations stay
    // in order, so no barrier is needed before overwriting them
    if constexpr (CL) write_codes<KC>(tid, bnxt, cw);
    bcur = bnxt;
    __syncthreads();
  }
  // tail stage of G % KC groups, loaded by the last iteration
  compute_tail<GATE_UP, MSUB, NS, KC - 1>(tid, G - nfull * KC, lds + (nfull & 1) * S::kStageHalfs,
                                          bcur, cw, zshift, bias, acc);
}

// One work item: M-tile `slot` of the tile list against N-tile `nt`.
template <bool GATE_UP, int MSUB, bool VEC>
__device__ __forceinline__ void process_item(const PrefillArgs& p, int slot, int nt,
                                             uint16_t* lds) {
  using S = AStage<GATE_UP, MSUB>;
  const uint32_t tid = threadIdx.x;
  const int e = p.tiles[2 * slot];
  const int row0 = p.tiles[2 * slot + 1];
  const int rows = min(S::kBM, p.offsets[e + 1] - row0);
  const int nsub = (rows + kSub - 1) / kSub;
  const int K = GATE_UP ? p.H : p.I;
  const int N = GATE_UP ? 2 * p.I : p.H;
  const int G = K / kGroup;

  // A rows: stage 1 gathers x rows through the sorted slots; stage 2 reads
  // the tile's own act rows (buffers based at the tile's first row).
  ASrc asrc;
  {
    const int j = static_cast<int>(tid / S::kTPR) & (kSub - 1);
    if (GATE_UP) {
      const uint32_t bytes = static_cast<uint32_t>(p.T) * K * 2u;
      asrc.r[0] = make_rsrc(p.a_hi, bytes);
      asrc.r[1] = asrc.r[0];
#pragma unroll
      for (int i = 0; i < MSUB; ++i) {
        const int r = i * kSub + j;
        asrc.row_off[i] = r < rows ? static_cast<uint32_t>(p.sorted_slots[row0 + r] / p.top_k) * K * 2u
                                   : bytes;
      }
    } else {
      const uint32_t bytes = static_cast<uint32_t>(rows) * K * 2u;
      asrc.r[0] = make_rsrc(p.a_hi + static_cast<size_t>(row0) * K, bytes);
      asrc.r[1] = make_rsrc(p.a_lo + static_cast<size_t>(row0) * K, bytes);
#pragma unroll
      for (int i = 0; i < MSUB; ++i) asrc.row_off[i] = static_cast<uint32_t>(i * kSub + j) * K * 2u;
    }
  }

  const int lane = static_cast<int>(tid & 63);
  const int wave = static_cast<int>(tid >> 6) & (kWaves - 1);
  const int j = lane & 31;
  const int h = lane >> 5;
  // This lane's weight row.  Stage 1: lanes 0..15 take gate columns c0..,
  // lanes 16..31 the matching up columns.
  int c0, n;
  if (GATE_UP) {
    c0 = nt * (kBN / 2) + wave * 16;
    n = c0 < p.I ? (j < 16 ? c0 + j : p.I + c0 + j - 16) : N;
  } else {
    c0 = nt * kBN + wave * kSub;
    n = c0 < N ? c0 + j : N;
  }
  const size_t wbase = static_cast<size_t>(e) * N;
  const bool n_ok = n < N;
  BAddr ba;
  ba.G = G;
  ba.rq = make_rsrc(p.qw + wbase * (G * 4), static_cast<uint32_t>(N) * G * 16u);
  ba.rs = make_rsrc(p.sc + wbase * G, static_cast<uint32_t>(N) * G * 2u);
  ba.rz = make_rsrc(p.qz + (wbase / 8) * G, static_cast<uint32_t>(N / 8) * G * 4u);
  ba.q_oob = static_cast<uint32_t>(N) * G * 16u;
  ba.s_oob = static_cast<uint32_t>(N) * G * 2u;
  ba.z_oob = static_cast<uint32_t>(N / 8) * G * 4u;
  // a lane past the matrix reads from the end of the buffers: zeros
  {
    constexpr int KC = StageCfg<GATE_UP, MSUB>::kKC;
    if constexpr (StageCfg<GATE_UP, MSUB>::kCodesLds) {
      // load pp of lane L: group L % KC of the wave's row 64 / KC pp + L / KC
      ba.qg = static_cast<uint32_t>(lane % KC);
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const int jr = (64 / KC) * pp + lane / KC;
        const int nr = c0 < p.I ? (jr < 16 ? c0 + jr : p.I + c0 + jr - 16) : N;
        ba.q_rows[pp] = (pp < KC / 2 && nr < N) ? static_cast<uint32_t>(nr) * G * 16u : ba.q_oob;
      }
    } else {
      ba.qg = static_cast<uint32_t>(h);
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) ba.q_rows[pp] = n_ok ? static_cast<uint32_t>(n) * G * 16u : ba.q_oob;
    }
  }
  ba.s_row = n_ok ? static_cast<uint32_t>(n) * G * 2u : ba.s_oob;
  ba.z_row = n_ok ? static_cast<uint32_t>(n >> 3) * G * 4u : ba.z_oob;
  const uint32_t zshift = 4u * static_cast<uint32_t>(n & 7);

  float16v acc[MSUB];
#pragma unroll
  for (int i = 0; i < MSUB; ++i) acc[i] = float16v{};

  if (MSUB == 1 || nsub == 1)
    main_loop<GATE_UP, MSUB, 1, VEC>(tid, asrc, lds, ba, zshift, acc);
  else if (nsub == 2)
    main_loop<GATE_UP, MSUB, (MSUB >= 2 ? 2 : 1), VEC>(tid, asrc, lds, ba, zshift, acc);
  else if (nsub == 3)
    main_loop<GATE_UP, MSUB, (MSUB >= 3 ? 3 : 1), VEC>(tid, asrc, lds, ba, zshift, acc);
  else
    main_loop<GATE_UP, MSUB, MSUB, VEC>(tid, asrc, lds, ba, zshift, acc);

  // Epilogue: lane (h, j) holds rows 8 (v / 4) + 4 h + v % 4, column j of
  // every 32 x 32 subtile.
#pragma unroll
  for (int i = 0; i < MSUB; ++i) {
    if (i >= nsub) break;
    if (GATE_UP) {
      // Lanes j < 16 hold gate and lanes j + 16 the up value of the same
      // column; each lane of the pair finishes 8 of the 16 rows.
      const bool low = j < 16;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float send = low ? acc[i][u + 8] : acc[i][u];
        const float recv = __shfl_xor(send, 16, 64);
        const int v = low ? u : u + 8;
        const float gate = low ? acc[i][u] : recv;
        const float up = low ? recv : acc[i][u + 8];
        const int r = i * kSub + 8 * (v >> 2) + 4 * h + (v & 3);
        if (r < rows && c0 < p.I) {
          const float act = gate / (1.f + expf(-gate)) * up;
          const uint16_t hi = float_to_half_bits(act);
          const uint16_t lo = float_to_half_bits(act - half_bits_to_float(hi));
          const size_t idx = static_cast<size_t>(row0 + r) * p.I + slot_pos(c0 + (j & 15));
          p.act_hi[idx] = hi;
          p.act_lo[idx] = lo;
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = i * kSub + 8 * (v >> 2) + 4 * h + (v & 3);
        if (r < rows && n_ok) p.y[static_cast<size_t>(row0 + r) * p.H + n] = acc[i][v];
      }
    }
  }
}

// Work item i is (M-tile i / n_ntiles, N-tile i % n_ntiles).  The prep
// kernel cut the items into 8 contiguous ranges of equal estimated cost;
// workgroup b takes item b / 8 of range b % 8.  Workgroups are dealt to the
// XCDs round-robin, so each XCD walks its own run of experts in order and the
// workgroups running together share A rows and weights in their L2.  The grid
// covers the longest possible range; workgroups past the end of their range
// exit at once.
template <bool GATE_UP, int MSUB, bool VEC>
__global__ __launch_bounds__(kThreads) void ffn_mfma_kernel(PrefillArgs p, int n_ntiles,
                                                            const int* __restrict__ sched) {
  using S = AStage<GATE_UP, MSUB>;
  constexpr int kCodesBytes =
      StageCfg<GATE_UP, MSUB>::kCodesLds ? kWaves * CodesLds<S::kKC>::kWaveBytes : 0;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * S::kStageHalfs + kCodesBytes / 2];
  const int x = static_cast<int>(blockIdx.x & 7);
  const int item = sched[x] + static_cast<int>(blockIdx.x >> 3);
  if (item >= sched[x + 1]) return;
  const int slot = item / n_ntiles;
  process_item<GATE_UP, MSUB, VEC>(p, slot, item - slot * n_ntiles, lds);
}

// Exclusive scan over the 1024 threads of a block; returns the thread's
// exclusive prefix and stores the total in tot[16].
__device__ __forceinline__ int block_exclusive_scan(int v, int* tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  if (lane == 63) tot[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < 16 ? tot[lane] : 0;
    int winc = w;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(winc, d, 64);
      if (lane >= d) winc += o;
    }
    if (lane < 16) tot[lane] = winc - w;
    if (lane == 15) tot[16] = winc;
  }
  __syncthreads();
  const int r = tot[wave] + inc - v;
  __syncthreads();   // tot is reused by the next scan
  return r;
}

// Block 0: the tile list (for every active expert, ceil(rows / bm) entries
// (expert, first row), in active-expert order), and for each of the two
// GEMMs the bounds of its 8 work ranges.  Blocks 1..: x permuted to
// k-slot order within every 8-wide block.
__global__ __launch_bounds__(1024) void prefill_prep_kernel(
    const int* __restrict__ offsets, const int* __restrict__ active,
    const int* __restrict__ num_active, int bm, int sub_cost, int base, int nn_gate_up, int nn_down,
    int* __restrict__ tiles, int* __restrict__ tile_count, int* __restrict__ sched,
    const uint16_t* __restrict__ x, uint16_t* __restrict__ xp, int64_t chunks) {
  if (blockIdx.x > 0) {
    const int64_t c = static_cast<int64_t>(blockIdx.x - 1) * 1024 + threadIdx.x;
    if (c < chunks)
      reinterpret_cast<uint4*>(xp)[c] = permute8(reinterpret_cast<const uint4*>(x)[c]);
    return;
  }
  __shared__ int tot[17];
  __shared__ int tile0[kMaxExperts + 1];   // per active expert: first tile
  __shared__ int work0[kMaxExperts + 1];   // per active expert: subtiles before it
  constexpr int kPer = kMaxExperts / 1024;
  const int tid = threadIdx.x;
  const int na = *num_active;
  const int msub = bm / kSub;
  int cnt[kPer], wk[kPer];
  int csum = 0, wsum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int a = tid * kPer + i;
    cnt[i] = 0;
    wk[i] = 0;
    if (a < na) {
      const int e = active[a];
      const int rows = offsets[e + 1] - offsets[e];
      cnt[i] = (rows + bm - 1) / bm;
      wk[i] = sub_cost * ((rows + kSub - 1) / kSub) + base * cnt[i];
    }
    csum += cnt[i];
    wsum += wk[i];
  }
  int pos = block_exclusive_scan(csum, tot);
  const int total_tiles = tot[16];
  __syncthreads();
  int wpos = block_exclusive_scan(wsum, tot);
  const int total_work = tot[16];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int a = tid * kPer + i;
    if (a < na) {
      const int e = active[a];
      const int r0 = offsets[e];
      tile0[a] = pos;
      work0[a] = wpos;
      for (int t = 0; t < cnt[i]; ++t) {
        tiles[2 * (pos + t)] = e;
        tiles[2 * (pos + t) + 1] = r0 + t * bm;
      }
    }
    pos += cnt[i];
    wpos += wk[i];
  }
  if (tid == 0) {
    *tile_count = total_tiles;
    tile0[na] = total_tiles;
    work0[na] = total_work;
  }
  __syncthreads();
  if (tid < 16) {
    // first item of range xr of GEMM k: the first item whose cumulative work
    // reaches xr / 8 of the total
    const int k = tid >> 3, xr = tid & 7;
    const int nn = k ? nn_down : nn_gate_up;
    int* sc = sched + k * kSchedStride;
    const int64_t items = static_cast<int64_t>(total_tiles) * nn;
    const int64_t target = static_cast<int64_t>(total_work) * nn * xr / 8;
    int lo = 0, hi = na;   // last expert a with work0[a] * nn <= target
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (static_cast<int64_t>(work0[mid]) * nn <= target) lo = mid;
      else hi = mid;
    }
    const int64_t r = target - static_cast<int64_t>(work0[lo]) * nn;
    const int ntl = tile0[lo + 1] - tile0[lo];
    const int wa = work0[lo + 1] - work0[lo];
    const int wfull = sub_cost * msub + base;   // work of a full tile
    const int u = static_cast<int>(min<int64_t>(r / (static_cast<int64_t>(wfull) * nn), ntl - 1));
    const int w = min(wfull, wa - u * wfull);
    const int64_t r2 = r - static_cast<int64_t>(u) * wfull * nn;
    const int64_t first = static_cast<int64_t>(tile0[lo] + u) * nn + (r2 + w - 1) / w;
    sc[xr] = static_cast<int>(min(first, items));
    if (xr == 7) sc[8] = static_cast<int>(items);
  }
}

// Workgroups per range.  An item of s live subtiles costs
// c = kSubCost s + kItemBase, at least c1 = kSubCost + kItemBase and at most
// c1 s, so a range (1/8 of the cost) holds at most 1/8 of the items'
// subtiles plus one item.  The subtiles
// number at most one per 32 rows plus one per expert.
int64_t range_bound(int64_t S, int E, int n_ntiles) {
  const int64_t subtiles = (S + kSub - 1) / kSub + std::min<int64_t>(E, S);
  return (subtiles * n_ntiles + 7) / 8 + 1;
}

template <bool GATE_UP, int MSUB>
void launch_gemm(const PrefillArgs& p, int n_ntiles, const int* sched, hipStream_t stream) {
  const int64_t per_range = range_bound(static_cast<int64_t>(p.T) * p.top_k, p.E, n_ntiles);
  const dim3 grid(static_cast<unsigned>(8 * per_range));
  const int G = (GATE_UP ? p.H : p.I) / kGroup;
  if (G % StageCfg<GATE_UP, MSUB>::kKC == 0)
    hipLaunchKernelGGL((ffn_mfma_kernel<GATE_UP, MSUB, true>), grid, dim3(kThreads), 0, stream, p,
                       n_ntiles, sched);
  else
    hipLaunchKernelGGL((ffn_mfma_kernel<GATE_UP, MSUB, false>), grid, dim3(kThreads), 0, stream, p,
                       n_ntiles, sched);
}

int ntiles_gate_up(int I) { return (I + kBN / 2 - 1) / (kBN / 2); }
int ntiles_down(int H) { return (H + kBN - 1) / kBN; }

}  // namespace

int64_t prefill_max_items(int64_t S, int E, int H, int I) {
  return 8 * range_bound(S, E, std::max(ntiles_gate_up(I), ntiles_down(H)));
}

void launch_prefill_prep(const uint16_t* x, int T, int H, int I, const int* offsets,
                         const int* active, const int* num_active, int64_t S, int E, int msub,
                         const FfnWorkspace& ws, hipStream_t stream) {
  const int64_t chunks = static_cast<int64_t>(T) * H / 8;
  const unsigned blocks = 1 + static_cast<unsigned>((chunks + 1023) / 1024);
  hipLaunchKernelGGL(prefill_prep_kernel, dim3(blocks), dim3(1024), 0, stream, offsets, active,
                     num_active, msub * kSub, kSubCost, kItemBase, ntiles_gate_up(I),
                     ntiles_down(H), ws.tiles, ws.tile_count, ws.sched, x, ws.x_perm, chunks);
}

void launch_gate_up_prefill(const GateUpArgs& a, const FfnWorkspace& ws, hipStream_t stream) {
  PrefillArgs p{ws.x_perm, nullptr, a.sorted_slots, a.T, a.top_k, a.E, a.H, a.I, a.offsets,
                ws.tiles, ws.tile_count, a.qw, a.sc, a.qz, ws.act_hi, ws.act_lo, nullptr};
  if (a.msub == 4)  // the prep kernel's tiles are of a.msub subtiles too
    launch_gemm<true, 4>(p, ntiles_gate_up(a.I), ws.sched, stream);
  else
    launch_gemm<true, 1>(p, ntiles_gate_up(a.I), ws.sched, stream);
}

void launch_down_prefill(const DownArgs& a, const FfnWorkspace& ws, hipStream_t stream) {
  PrefillArgs p{ws.act_hi, ws.act_lo, nullptr, a.T, a.top_k, a.E, a.H, a.I, a.offsets,
                ws.tiles, ws.tile_count, a.qw, a.sc, a.qz, nullptr, nullptr, a.y};
  const int* sched = ws.sched + kSchedStride;
  if (a.msub == 4)
    launch_gemm<false, 4>(p, ntiles_down(a.H), sched, stream);
  else
    launch_gemm<false, 1>(p, ntiles_down(a.H), sched, stream);
}

}  // namespace moe
