// Per-shape choice of kernel variant and tile profile: the one table every
// entry point takes its choices from ("[Perf][SM70] Narrow Qwen3.8 AWQ active
// grouped decode", section "Additional existing-autotune benefit
// (fresh-process pair)": tuned tiles per shape, there a W13 tile change from
// M64 x 128 x 32 to M8 x 256 x 64 at 4-8 tokens).  Host code only, a pure
// function of the sizes.  The entries below were chosen from a sweep of the
// layer on MI355X at T = 1 ... 4096 and I = 160 / 640 (bench.py --sweep),
// every plan timed on 16 weight copies.
#include "../../include/moe_w4a16.h"
#include "common.h"

namespace moe {

// The table.  Layer times at 512 experts, top-10, hidden 2560 from the
// sweep, in us: the fastest GEMV plan and the fastest matrix-core plan.
//   tokens          1     8     9    16    32    64   | I
//   GEMV          30.2  70.2  76.3 113.2 182.5 298.3  | 640
//   MFMA          45.0  88.2 102.9 141.1 212.3 307.4  | 640
//   GEMV          26.4  39.8  43.1  54.3  78.2 122.1  | 160
//   MFMA          39.2  51.0  52.2  65.2  83.9 116.3  | 160
// GEMV (one weight stream, A rows from LDS) up to 32 tokens, the matrix-core
// GEMMs above.
constexpr int64_t kGemvMaxT = 32;
// Routing inside the gate/up GEMV (every workgroup routes the T tokens
// itself) is the fastest GEMV form at every size swept.
constexpr int64_t kRouteInKernelMaxT = kGemvMaxT;
constexpr int kRouteInKernelMaxE = 1024;
// Router and permutation as one single-workgroup launch: faster than the two
// kernels up to 8 tokens only (its 16 waves route the tokens in turn).
constexpr int64_t kRouteOneLaunchMaxT = 8;
constexpr int kRouteOneLaunchMaxE = 1024;
// From 10 tokens some expert draws 3 or more rows: four A rows per weight
// pass and work shared out by cost (I = 640, 10 tokens: 119.8 us with two
// rows and an even split, 82.5 us with four and the cost split).
constexpr int64_t kRows4MinT = 10;
// 128-row M-tiles (4 subtiles) once an expert averages 64 rows or more
// (I = 640: 1024 tokens 529.9 us with 32-row tiles, 593.0 with 128;
// 4096 skewed tokens 1226.8 us with 128-row tiles, 1384.3 with 32).
constexpr int64_t kMsub4RowsPerExpert = 64;
// Router projection: GEMV up to 16 tokens (its kernel limit) while x
// (T x H fp16) is at most 80 KiB, a size the sweep covered at hidden 2560
// (block at 8 tokens, I = 640: 78.6 us with it, 94.4 us with MFMA); the
// matrix cores above.
constexpr int64_t kRouterGemvMaxT = 16;
constexpr int64_t kRouterGemvMaxXBytes = 80 * 1024;
// Shared expert on the matrix cores in extra workgroups of the GEMV launches
// from 3 tokens; below, as one more expert of the GEMV (block, graph of 16
// steps, us, matrix cores / GEMV): I = 640: 1 token 52.5 / 35.8, 2: 56.5 /
// 47.0, 3: 59.5 / 67.6, 4: 64.8 / 85.4, 16: 130.7 / 160.7; I = 160: 1 token
// 41.1 / 31.9, 2: 46.0 / 35.5, 3: 49.4 / 50.7.
constexpr int64_t kSharedMfmaMinT = 3;
// 16 lanes per w13 row up to 4 tokens (each wave's run of loads per block is
// half as long), 8 above (layer, us, 8 / 16 lanes: I = 160: 1 token 26.9 /
// 25.5, 2: 28.7 / 27.7, 4: 33.6 / 32.9, 8: 40.5 / 40.2, 16: 67.6 / 69.0;
// I = 640: 1 token 30.9 / 30.2, 4: 48.7 / 48.0, 8: 69.2 / 71.8).
constexpr int64_t kLanes16MaxT = 4;
// The combine folded into the down GEMV (one workgroup per block of output
// rows of every active expert) up to 2 tokens (layer, us, folded / separate
// combine: I = 160: 1 token 21.4 / 25.1, 2: 26.1 / 27.4; I = 640: 1 token
// 26.6 / 30.5, 2: 34.3 / 38.1).  A form for up to 4 rows per expert was
// slower from 3 tokens (4 tokens: I = 160 39.2 / 32.6, I = 640 51.0 / 48.5).
constexpr int64_t kCombineInDownMaxT = 2;

// Lanes per weight row of a GEMV over K = 32 G: the largest power of two
// <= cap that divides G (a lane takes every lanes-th group of the row).
static int gemv_lanes(int G, int cap) {
  int C = 1;
  while (C < cap && G % (2 * C) == 0) C *= 2;
  return C;
}

// Smallest power of two >= n, at most 8.
static int pow2_rows(int64_t n) {
  int r = 1;
  while (r < 8 && r < n) r *= 2;
  return r;
}

bool gemv_fits(const Plan& p, int64_t T, int top_k, int E, int shared, int H, int I,
               size_t lds_bytes);

Plan default_plan(int64_t T, int top_k, int E, int shared, int H, int I) {
  Plan p;
  const int kk = top_k + shared, EP = E + shared;  // slots per token, experts
  const int64_t S = T * static_cast<int64_t>(kk);
  p.ffn = T <= kGemvMaxT ? MOE_FFN_GEMV : MOE_FFN_MFMA;
  if (p.ffn == MOE_FFN_GEMV && T <= kRouteInKernelMaxT && EP <= kRouteInKernelMaxE)
    p.route = MOE_ROUTE_IN_GATE_UP;
  else if (T <= kRouteOneLaunchMaxT && EP <= kRouteOneLaunchMaxE)
    p.route = MOE_ROUTE_ONE_LAUNCH;
  else
    p.route = MOE_ROUTE_SEPARATE;
  p.msub = S >= kMsub4RowsPerExpert * static_cast<int64_t>(EP) ? 4 : 1;
  p.lanes_gate_up = gemv_lanes(H / kGroup, T <= kLanes16MaxT ? 16 : 8);
  p.lanes_down = gemv_lanes(I / kGroup, 8);
  // A shared expert with the GEMV runs on the matrix cores in extra
  // workgroups (the GEMV then holds the routed experts only) from 3 tokens,
  // where its A rows fit in LDS.
  p.shared_mfma = shared && p.ffn == MOE_FFN_GEMV && T >= kSharedMfmaMinT &&
                  shared_mfma_lds(T, H, I) + kDecodeStaticLds <= kGfx950LdsBytes;
  p.rows_per_pass = T >= kRows4MinT ? 4 : (T >= 2 ? 2 : 1);
  p.cost_split = T >= kRows4MinT;
  p.router_gemv = T <= kRouterGemvMaxT && T * static_cast<int64_t>(H) * 2 <= kRouterGemvMaxXBytes;
  // the one-launch FFN is slower than two launches at every size swept
  p.one_launch = 0;
  p.combine_in_down = p.ffn == MOE_FFN_GEMV && T <= kCombineInDownMaxT && !p.shared_mfma &&
                      down_fold_ok(T, kk, I, p.lanes_down, kGfx950LdsBytes);
  // A shared expert of 3 tokens or more whose A rows do not fit in LDS (23
  // and more at H = 2560): the matrix-core FFN, which takes its rows as one
  // more M-tile (block, us, GEMV with the shared expert in it / matrix
  // cores: I = 640: 23 tokens 259.3 / 203.6, 28: 293.1 / 222.5, 32: 297.5 /
  // 230.7; I = 160: 23 tokens 189.3 / 113.2, 32: 199.7 / 117.0).
  const bool shared_no_room =
      shared && p.ffn == MOE_FFN_GEMV && T >= kSharedMfmaMinT && !p.shared_mfma;
  // the GEMV's A fragments of a long K (I near 16384 for the down stage)
  // do not fit a workgroup's LDS: the matrix cores then take every size
  if (p.ffn == MOE_FFN_GEMV &&
      (shared_no_room || !gemv_fits(p, T, top_k, E, shared, H, I, kGfx950LdsBytes))) {
    p.ffn = MOE_FFN_MFMA;
    p.shared_mfma = 0;
    p.combine_in_down = 0;
    if (p.route == MOE_ROUTE_IN_GATE_UP)
      p.route = T <= kRouteOneLaunchMaxT && EP <= kRouteOneLaunchMaxE ? MOE_ROUTE_ONE_LAUNCH
                                                                      : MOE_ROUTE_SEPARATE;
  }
  return p;
}

bool gemv_fits(const Plan& p, int64_t T, int top_k, int E, int shared, int H, int I,
               size_t lds_bytes) {
  const int kk = top_k + shared, EP = E + shared;
  const bool route = p.route == MOE_ROUTE_IN_GATE_UP;
  if (p.shared_mfma && shared_mfma_lds(T, H, I) + kDecodeStaticLds > lds_bytes) return false;
  if (p.combine_in_down && !down_fold_ok(T, kk, I, p.lanes_down, lds_bytes)) return false;
  if (p.one_launch &&
      one_launch_min_lds(T, kk, EP, H, I, p.lanes_gate_up, p.lanes_down) > lds_bytes)
    return false;
  return gemv_min_lds(true, route, T, kk, EP, H, I, p.lanes_gate_up, p.cost_split) <= lds_bytes &&
         gemv_min_lds(false, false, T, kk, EP, H, I, p.lanes_down, p.cost_split) <= lds_bytes;
}

int plan_check(const Plan& p, int64_t T, int top_k, int E, int shared, int H, int I) {
  E += shared;
  if (p.ffn != MOE_FFN_GEMV && p.ffn != MOE_FFN_MFMA) return MOE_ERR_INVALID_ARG;
  if (p.rows_per_pass != 1 && p.rows_per_pass != 2 && p.rows_per_pass != 4 &&
      p.rows_per_pass != 8)
    return MOE_ERR_INVALID_ARG;
  if (p.cost_split != 0 && p.cost_split != 1) return MOE_ERR_INVALID_ARG;
  if (p.route < MOE_ROUTE_IN_GATE_UP || p.route > MOE_ROUTE_SEPARATE) return MOE_ERR_INVALID_ARG;
  if (p.msub != 1 && p.msub != 4) return MOE_ERR_INVALID_ARG;
  auto lanes_ok = [](int c, int G) {
    return (c == 1 || c == 2 || c == 4 || c == 8 || c == 16) && G % c == 0;
  };
  if (!lanes_ok(p.lanes_gate_up, H / kGroup) || !lanes_ok(p.lanes_down, I / kGroup))
    return MOE_ERR_INVALID_ARG;
  if (p.router_gemv != 0 && p.router_gemv != 1) return MOE_ERR_INVALID_ARG;
  if (p.shared_mfma != 0 && p.shared_mfma != 1) return MOE_ERR_INVALID_ARG;
  if (p.combine_in_down != 0 && p.combine_in_down != 1) return MOE_ERR_INVALID_ARG;
  // the folded combine: the GEMV, up to 2 tokens, no shared-expert
  // workgroups, its LDS and steps within the kernel's limits
  if (p.combine_in_down &&
      (p.ffn != MOE_FFN_GEMV || p.shared_mfma || !down_fold_ok(T, top_k + shared, I, p.lanes_down,
                                                                 kGfx950LdsBytes)))
    return MOE_ERR_UNSUPPORTED;
  if (p.one_launch != 0 && p.one_launch != 1) return MOE_ERR_INVALID_ARG;
  // the one-launch FFN: the GEMV routing inside gate/up, no shared expert, an
  // even split, a separate combine, both stages' LDS within the device's
  if (p.one_launch &&
      (p.ffn != MOE_FFN_GEMV || p.route != MOE_ROUTE_IN_GATE_UP || shared || p.cost_split ||
       p.combine_in_down ||
       one_launch_min_lds(T, top_k + shared, E, H, I, p.lanes_gate_up, p.lanes_down) >
           kGfx950LdsBytes))
    return MOE_ERR_UNSUPPORTED;
  if (p.shared_mfma && !shared) return MOE_ERR_INVALID_ARG;
  // the shared expert's matrix-core workgroups: with the GEMV, up to 32 rows
  // (one MFMA tile) whose A rows fit in LDS
  if (p.shared_mfma &&
      (p.ffn != MOE_FFN_GEMV || T > 32 ||
       shared_mfma_lds(T, H, I) + kDecodeStaticLds > kGfx950LdsBytes))
    return MOE_ERR_UNSUPPORTED;
  // what each variant supports (the table above picks within these limits)
  if (p.ffn == MOE_FFN_GEMV && T > kPermBlockTokens) return MOE_ERR_UNSUPPORTED;
  if (p.route == MOE_ROUTE_IN_GATE_UP &&
      (p.ffn != MOE_FFN_GEMV || T > kPermBlockTokens || E > kRouteInKernelMaxE))
    return MOE_ERR_UNSUPPORTED;
  if (p.route == MOE_ROUTE_ONE_LAUNCH && (T > kPermBlockTokens || E > kRouteOneLaunchMaxE))
    return MOE_ERR_UNSUPPORTED;
  if (p.router_gemv && T > kRouterGemvMaxT)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace moe
