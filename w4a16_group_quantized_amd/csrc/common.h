// Internal declarations shared by the HIP translation units of libmoe_w4a16.
// Not part of the public ABI (see include/moe_w4a16.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_w4a16.h"

namespace moe {

constexpr int kGroup = 32;          // quantisation group size along K
constexpr int kMaxExperts = 4096;   // E limit
constexpr int kMaxTopK = 64;        // top_k limit (one router round per lane)
constexpr int kMaxGroups = 512;     // K / 32 limit (K <= 16384)
constexpr int kPermBlockTokens = 64;  // tokens per permutation block (one 64-bit mask)
constexpr int kMaxDevices = 64;     // devices with cached attributes

// Compute-unit count and the LDS bytes one workgroup may use on the current
// device.  Read from the runtime once per device and kept in a per-device
// cache (a value never changes for a device, so threads racing on the cache
// store the same thing).
struct DeviceInfo {
  int cus;
  int lds;
};
DeviceInfo device_info();

// Kernel variant and tile profile (plan.hip): the default for given sizes,
// and whether an explicit plan is allowed for them (MOE_OK or an error code).
// top_k and E count the routed experts; shared = 1 adds a shared expert.
using Plan = moe_plan;
Plan default_plan(int64_t T, int top_k, int E, int shared, int H, int I);
int plan_check(const Plan& p, int64_t T, int top_k, int E, int shared, int H, int I);
// Whether a GEMV plan's kernels fit `lds_bytes` of LDS per workgroup.
bool gemv_fits(const Plan& p, int64_t T, int top_k, int E, int shared, int H, int I,
               size_t lds_bytes);

// ----------------------------------------------------------------------------
// Launchers (each enqueues on `stream`, returns nothing; the ABI layer checks
// hipGetLastError afterwards).
// ----------------------------------------------------------------------------
// shared = 1: ids/weights rows have top_k + 1 entries, the last the shared
// expert E with weight 1.
void launch_route(const float* logits, int T, int E, int top_k, int shared, int* ids,
                  float* weights, hipStream_t stream);

size_t permute_workspace_bytes(int64_t T, int E);
void launch_permute(const int* ids, int T, int top_k, int E, int* offsets,
                    int* sorted_slots, int* slot_rows, int* active,
                    int* num_active, void* workspace, hipStream_t stream);

// Router and permutation in one call: one launch when `one_launch` (T <= 64,
// E + shared <= 1024), else the router kernel and the permutation kernels.
// E is the logits' expert count; with shared = 1 the permutation covers
// E + 1 experts and top_k + 1 slots per token.
void launch_route_permute(const float* logits, int T, int E, int top_k, int shared, int* ids,
                          float* weights, int* offsets, int* sorted_slots, int* slot_rows,
                          int* active, int* num_active, void* workspace, bool one_launch,
                          hipStream_t stream);

// Router gate projection logits[T, E] = x[T, H] . Wg[E, H]^T (router_gate.hip):
// the GEMV variant when `gemv` (T <= 16, T * H * 2 <= 80 KiB), else the
// matrix-core one.
void launch_router_gate(const uint16_t* x, int T, int H, const uint16_t* gate_weight, int E,
                        float* logits, bool gemv, hipStream_t stream);

struct FfnWorkspace {
  uint16_t* act_hi;  // [S, I] fp16, high part of SiLU(gate)*up
  uint16_t* act_lo;  // [S, I] fp16, act - act_hi rounded to fp16
  int* tiles;        // matrix-core M-tile list (prefill variant)
  int* tile_count;   // number of valid entries of `tiles`
  int* sched;        // per GEMM (stride kSchedStride): bounds of its 8 work ranges
  uint16_t* x_perm;  // [T, H] x in k-slot order (prefill variant)
};
constexpr int kSchedStride = 16;    // ints per GEMM schedule (9 used)
size_t ffn_workspace_bytes(int64_t T, int top_k, int E, int H, int I);
FfnWorkspace ffn_workspace_carve(void* base, int64_t T, int top_k, int E, int H, int I);

struct GateUpArgs {
  const uint16_t* x;
  int T, top_k, E, H, I;
  int shared = 0;  // routing kernels only: top_k and E count a shared expert (index E - 1)
  int lanes = 0;          // GEMV: lanes per weight row (from the plan)
  int rows_per_pass = 0;  // GEMV: A rows of an expert per weight pass (from the plan)
  int cost_split = 0;     // GEMV: units shared out by cost (from the plan)
  int shared_mfma = 0;    // GEMV: the shared expert (the last expert) on the matrix cores
  int msub = 0;           // MFMA: 32-row subtiles per M-tile (from the plan)
  const int* offsets;
  const int* sorted_slots;
  const int* active;
  const int* num_active;
  const int* qw;
  const uint16_t* sc;
  const int* qz;
};
struct DownArgs {
  int T, top_k, E, H, I;
  int lanes = 0;  // as in GateUpArgs
  int rows_per_pass = 0;
  int cost_split = 0;
  int shared_mfma = 0;
  int msub = 0;
  const int* offsets;
  const int* active;
  const int* num_active;
  const int* qw;
  const uint16_t* sc;
  const int* qz;
  float* y;
  // the combine folded into the down GEMV (layer calls): out written from
  // the weights and slot rows of the routing
  int combine = 0;
  const float* c_weights = nullptr;
  const int* c_slot_rows = nullptr;
  uint16_t* out = nullptr;
};
void launch_gate_up_decode(const GateUpArgs& a, const FfnWorkspace& ws, hipStream_t stream);

// Stage 1 of the decode FFN that first routes the T tokens itself, from
// logits [T, E] (T <= 64, E <= 1024), and writes the routing out as
// moe_route_permute does.  The routing fields of `a` (offsets, sorted_slots,
// active, num_active) are not read.
struct RouteOut {
  int* ids;
  float* weights;
  int* offsets;
  int* sorted_slots;
  int* slot_rows;
  int* active;
  int* num_active;
};
void launch_route_gate_up_decode(const float* logits, const GateUpArgs& a, const RouteOut& r,
                                 const FfnWorkspace& ws, hipStream_t stream);
void launch_down_decode(const DownArgs& a, const FfnWorkspace& ws, hipStream_t stream);
// Gate/up (routing inside) and down in one persistent launch; a.lanes and
// d.lanes are the two stages' lanes per row, a.rows_per_pass the A rows per
// pass; no shared expert, even split.
void launch_one_launch_decode(const float* logits, const GateUpArgs& a, const DownArgs& d,
                              const RouteOut& r, const FfnWorkspace& ws, hipStream_t stream);

// Least LDS bytes one workgroup of a GEMV stage needs at these sizes and
// lanes per row (ffn_decode.hip); a plan whose GEMV needs more than the
// device gives a workgroup cannot run.
size_t gemv_min_lds(bool gate_up, bool route, int64_t T, int top_k, int E, int H, int I,
                    int lanes, bool cost_split);
// The down GEMV with the combine folded in (T <= 2): its LDS (every act row's
// fragments and one block of y rows), and whether it can run at these sizes
// (at most 8 steps per lane, LDS within lds_bytes).
size_t down_fold_lds(int64_t T, int top_k, int I, int lanes);
bool down_fold_ok(int64_t T, int top_k, int I, int lanes, size_t lds_bytes);
// Least LDS bytes of the one-launch FFN's workgroup (routing tables and the
// larger stage).
size_t one_launch_min_lds(int64_t T, int top_k, int E, int H, int I, int lanes_gate_up,
                          int lanes_down);
// LDS of the shared expert's matrix-core workgroups inside the GEMV launches
// (A rows of both stages and the K-split partial sums), T <= 32.
size_t shared_mfma_lds(int64_t T, int H, int I);
constexpr size_t kGfx950LdsBytes = 160 * 1024;   // LDS per workgroup on gfx950
// LDS a decode launch keeps beside its dynamic LDS (the kernels' static LDS,
// rounded up): every dynamic-size check leaves it free.
constexpr size_t kDecodeStaticLds = 256;

// Matrix-core variant: a prep kernel (tile list of M-tiles of msub 32-row
// subtiles built from the routing, x permuted to k-slot order, both into the
// FFN workspace) followed by the two grouped GEMMs, which take the same msub.
int64_t prefill_max_items(int64_t S, int E, int H, int I);   // grid of the larger GEMM
void launch_prefill_prep(const uint16_t* x, int T, int H, int I, const int* offsets,
                         const int* active, const int* num_active, int64_t S, int E, int msub,
                         const FfnWorkspace& ws, hipStream_t stream);
void launch_gate_up_prefill(const GateUpArgs& a, const FfnWorkspace& ws, hipStream_t stream);
void launch_down_prefill(const DownArgs& a, const FfnWorkspace& ws, hipStream_t stream);

void launch_combine(const float* y_sorted, const float* weights,
                    const int* slot_rows, int T, int top_k, int H,
                    uint16_t* out, hipStream_t stream);

// ----------------------------------------------------------------------------
// Device helpers
// ----------------------------------------------------------------------------
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

// v_dot2_f32_f16: a.lo*b.lo + a.hi*b.hi + c, fp16 products exact in fp32.
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a),
                                __builtin_bit_cast(h2_t, b), c, false);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// Round to nearest even (the default rounding mode of v_cvt_f16_f32).
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// ---- matrix-core operands (v_mfma_f32_32x32x16_f16) --------------------------
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

// Position of column c once its 8-wide block is permuted to k-slot order
// (0, 4, 1, 5, 2, 6, 3, 7).
__device__ __forceinline__ int slot_pos(int c) {
  return (c & ~7) | ((c & 3) << 1) | ((c >> 2) & 1);
}

// 8 consecutive fp16 (4 dwords: (a0,a1) (a2,a3) (a4,a5) (a6,a7)) reordered
// to the k-slot order (a0,a4) (a1,a5) (a2,a6) (a3,a7).
__device__ __forceinline__ uint4 permute8(uint4 d) {
  return make_uint4((d.x & 0xFFFFu) | (d.z << 16), (d.x >> 16) | (d.z & 0xFFFF0000u),
                    (d.y & 0xFFFFu) | (d.w << 16), (d.y >> 16) | (d.w & 0xFFFF0000u));
}

// (q - z) of one packed word as 8 fp16 in k-slot order, exactly.  m1024 holds
// -(1024 + z) and m64 holds -(64 + z) in both halves.
__device__ __forceinline__ half8 dequant_word(uint32_t w, uint32_t bias, h2 m1024, h2 m64) {
  const uint32_t w8 = w >> 8;
  const h2 pa = __builtin_bit_cast(h2, (w & 0x000F000Fu) | bias);   // 1024 + q0, 1024 + q4
  const h2 pb = __builtin_bit_cast(h2, (w & 0x00F000F0u) | bias);   // 1024 + 16 q1, ...
  const h2 pc = __builtin_bit_cast(h2, (w8 & 0x000F000Fu) | bias);  // 1024 + q2, 1024 + q6
  const h2 pd = __builtin_bit_cast(h2, (w8 & 0x00F000F0u) | bias);  // 1024 + 16 q3, ...
  const h2 sixteenth = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
  const h2 r0 = pa + m1024;              // q0 - z, q4 - z
  const h2 r1 = pb * sixteenth + m64;    // q1 - z, q5 - z
  const h2 r2 = pc + m1024;
  const h2 r3 = pd * sixteenth + m64;
  half8 out;
  out[0] = r0[0]; out[1] = r0[1]; out[2] = r1[0]; out[3] = r1[1];
  out[4] = r2[0]; out[5] = r2[1]; out[6] = r3[0]; out[7] = r3[1];
  return out;
}


// The two zero-point terms of dequant_word for zero code zc: -(1024 + z) and
// -(64 + z) (the latter for the nibbles read 16 times too large), in both
// halves.
__device__ __forceinline__ void zero_terms(uint32_t zc, h2& m1024, h2& m64) {
  m1024 = __builtin_bit_cast(h2, (0xE400u | zc) * 0x00010001u);
  m64 = __builtin_bit_cast(h2, (0xD400u | (zc << 4)) * 0x00010001u);
}

}  // namespace moe
