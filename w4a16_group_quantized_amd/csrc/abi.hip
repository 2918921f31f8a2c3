// C ABI of libmoe_w4a16.so: argument validation, workspace sizing and kernel
// dispatch.  Declarations and the full contract are in include/moe_w4a16.h.
// Nothing here allocates, frees or synchronises.
#include <stdint.h>

#include <atomic>

#include "../../include/moe_w4a16.h"
#include "common.h"

namespace {

using namespace moe;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
inline size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

int check_launch() {
  const hipError_t err = hipGetLastError();
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// Routing sizes shared by every entry point.
int check_routing(int64_t T, int32_t top_k, int32_t E) {
  if (T < 0 || E < 1 || top_k < 1 || top_k > E) return MOE_ERR_INVALID_ARG;
  if (E > kMaxExperts || top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (T * static_cast<int64_t>(top_k) > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// A GEMV plan must fit the device's LDS per workgroup (checked before
// anything is enqueued).
int check_gemv(const Plan& pl, int64_t T, int32_t top_k, int32_t E, int32_t shared, int32_t H,
               int32_t I) {
  if (pl.ffn != MOE_FFN_GEMV) return MOE_OK;
  const size_t lds = static_cast<size_t>(device_info().lds);
  return gemv_fits(pl, T, top_k, E, shared, H, I, lds) ? MOE_OK : MOE_ERR_UNSUPPORTED;
}

// The matrix-core variant addresses x with 32-bit byte offsets and numbers
// its work items with int.
int check_mfma(const Plan& pl, int64_t T, int32_t top_k, int32_t E, int32_t H, int32_t I) {
  if (pl.ffn != MOE_FFN_MFMA) return MOE_OK;
  if (T * static_cast<int64_t>(H) >= (static_cast<int64_t>(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (prefill_max_items(T * top_k, E, H, I) >= (static_cast<int64_t>(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The projection addresses x and Wg with 32-bit byte offsets.
int check_router_gate(int64_t T, int32_t H, int32_t E) {
  if (T < 0 || E < 1 || H <= 0 || H % kGroup) return MOE_ERR_INVALID_ARG;
  if (E > kMaxExperts || H / kGroup > kMaxGroups) return MOE_ERR_UNSUPPORTED;
  if (T * static_cast<int64_t>(H) * 2 >= (static_cast<int64_t>(1) << 32)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_dims(int32_t H, int32_t I, int32_t group_size) {
  if (group_size != kGroup) return MOE_ERR_UNSUPPORTED;
  if (H <= 0 || I <= 0 || H % kGroup || I % kGroup) return MOE_ERR_INVALID_ARG;
  if (H / kGroup > kMaxGroups || I / kGroup > kMaxGroups) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Enqueue the two halves of the FFN with the plan's variant (arguments
// already validated).  Both halves of one FFN take the same plan: the
// matrix-core down GEMM reads the tile list the gate/up call built.
void run_gate_up(GateUpArgs a, const Plan& pl, void* workspace, hipStream_t st) {
  const FfnWorkspace ws = ffn_workspace_carve(workspace, a.T, a.top_k, a.E, a.H, a.I);
  a.lanes = pl.lanes_gate_up;
  a.rows_per_pass = pl.rows_per_pass;
  a.cost_split = pl.cost_split;
  a.shared_mfma = pl.shared_mfma;
  a.msub = pl.msub;
  if (pl.ffn == MOE_FFN_GEMV) {
    launch_gate_up_decode(a, ws, st);
  } else {
    launch_prefill_prep(a.x, a.T, a.H, a.I, a.offsets, a.active, a.num_active,
                        static_cast<int64_t>(a.T) * a.top_k, a.E, pl.msub, ws, st);
    launch_gate_up_prefill(a, ws, st);
  }
}

void run_down(DownArgs d, const Plan& pl, void* workspace, hipStream_t st) {
  const FfnWorkspace ws = ffn_workspace_carve(workspace, d.T, d.top_k, d.E, d.H, d.I);
  d.lanes = pl.lanes_down;
  d.rows_per_pass = pl.rows_per_pass;
  d.cost_split = pl.cost_split;
  d.shared_mfma = pl.shared_mfma;
  d.msub = pl.msub;
  if (pl.ffn == MOE_FFN_GEMV)
    launch_down_decode(d, ws, st);
  else
    launch_down_prefill(d, ws, st);  // tile list from gate_up
}

}  // namespace

namespace moe {

DeviceInfo device_info() {
  static std::atomic<uint64_t> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  if (dev >= 0) {
    const uint64_t v = cache[dev].load(std::memory_order_relaxed);
    if (v) return {static_cast<int>(v >> 32), static_cast<int>(v & 0xFFFFFFFFu)};
  }
  int cus = 0, lds = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) !=
          hipSuccess ||
      cus < 1)
    cus = 256;
  // without a device to ask (host-side checks on a machine with no GPU), the
  // gfx950 value the library is built for
  if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev < 0 ? 0 : dev) !=
          hipSuccess ||
      lds < 1)
    lds = static_cast<int>(kGfx950LdsBytes);
  if (dev >= 0)
    cache[dev].store((static_cast<uint64_t>(cus) << 32) | static_cast<uint32_t>(lds),
                     std::memory_order_relaxed);
  return {cus, lds};
}

// Layout: act_hi | act_lo | tile list | tile count | permuted x, each part
// 256-byte aligned.  The tile list holds at most S + E entries (every tile
// but one per expert is full).
size_t ffn_workspace_bytes(int64_t T, int top_k, int E, int H, int I) {
  const size_t S = static_cast<size_t>(T) * top_k;
  const size_t act = align256(S * I * sizeof(uint16_t));
  const size_t tiles = align256((S + E + 1) * 2 * sizeof(int));
  const size_t xp = align256(static_cast<size_t>(T) * H * sizeof(uint16_t));
  return 2 * act + tiles + 256 + xp;
}

FfnWorkspace ffn_workspace_carve(void* base, int64_t T, int top_k, int E, int H, int I) {
  char* p = static_cast<char*>(base);
  const size_t S = static_cast<size_t>(T) * top_k;
  const size_t act = align256(S * I * sizeof(uint16_t));
  const size_t tiles = align256((S + E + 1) * 2 * sizeof(int));
  FfnWorkspace ws;
  ws.act_hi = reinterpret_cast<uint16_t*>(p);
  ws.act_lo = reinterpret_cast<uint16_t*>(p + act);
  ws.tiles = reinterpret_cast<int*>(p + 2 * act);
  ws.tile_count = reinterpret_cast<int*>(p + 2 * act + tiles);
  ws.sched = ws.tile_count + 8;
  ws.x_perm = reinterpret_cast<uint16_t*>(p + 2 * act + tiles + 256);
  (void)H;
  return ws;
}

}  // namespace moe

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size)";
    case MOE_ERR_UNSUPPORTED: return "unsupported size or group size";
    case MOE_ERR_WORKSPACE: return "workspace smaller than the size query requires";
    case MOE_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int moe_abi_version(void) { return 102; }

int moe_route(const float* logits, int64_t T, int32_t E, int32_t top_k, int32_t* topk_ids,
              float* topk_weights, void* stream) {
  if (int st = check_routing(T, top_k, E)) return st;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(logits) || !ok_ptr(topk_ids) || !ok_ptr(topk_weights)) return MOE_ERR_INVALID_ARG;
  launch_route(logits, static_cast<int>(T), E, top_k, 0, topk_ids, topk_weights,
               static_cast<hipStream_t>(stream));
  return check_launch();
}

int moe_route_shared(const float* logits, int64_t T, int32_t E, int32_t top_k, int32_t* topk_ids,
                     float* topk_weights, void* stream) {
  if (int st = check_routing(T, top_k, E)) return st;
  if (int st = check_routing(T, top_k + 1, E + 1)) return st;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(logits) || !ok_ptr(topk_ids) || !ok_ptr(topk_weights)) return MOE_ERR_INVALID_ARG;
  launch_route(logits, static_cast<int>(T), E, top_k, 1, topk_ids, topk_weights,
               static_cast<hipStream_t>(stream));
  return check_launch();
}

int moe_router_gate(const uint16_t* x, int64_t T, int32_t H, const uint16_t* gate_weight,
                    int32_t E, float* logits, void* stream) {
  if (int st = check_router_gate(T, H, E)) return st;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(x) || !ok_ptr(gate_weight) || !ok_ptr(logits)) return MOE_ERR_INVALID_ARG;
  launch_router_gate(x, static_cast<int>(T), H, gate_weight, E, logits,
                     default_plan(T, 1, E, 0, H, kGroup).router_gemv != 0,
                     static_cast<hipStream_t>(stream));
  return check_launch();
}

size_t moe_permute_workspace_bytes(int64_t T, int32_t top_k, int32_t E) {
  if (check_routing(T, top_k, E) != MOE_OK) return 0;
  return permute_workspace_bytes(T, E);
}

int moe_permute(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t E,
                int32_t* expert_offsets, int32_t* sorted_slots, int32_t* slot_rows,
                int32_t* active_experts, int32_t* num_active, void* workspace,
                size_t workspace_bytes, void* stream) {
  if (int st = check_routing(T, top_k, E)) return st;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(topk_ids) || !ok_ptr(expert_offsets) || !ok_ptr(sorted_slots) ||
      !ok_ptr(slot_rows) || !ok_ptr(active_experts) || !ok_ptr(num_active))
    return MOE_ERR_INVALID_ARG;
  const size_t need = permute_workspace_bytes(T, E);
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE;
  if (need > 0 && !ok_ptr(workspace)) return MOE_ERR_INVALID_ARG;
  launch_permute(topk_ids, static_cast<int>(T), top_k, E, expert_offsets, sorted_slots,
                 slot_rows, active_experts, num_active, workspace,
                 static_cast<hipStream_t>(stream));
  return check_launch();
}

int moe_route_permute(const float* logits, int64_t T, int32_t E, int32_t top_k,
                      int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                      int32_t* sorted_slots, int32_t* slot_rows, int32_t* active_experts,
                      int32_t* num_active, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (int st = check_routing(T, top_k, E)) return st;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(logits) || !ok_ptr(topk_ids) || !ok_ptr(topk_weights) || !ok_ptr(expert_offsets) ||
      !ok_ptr(sorted_slots) || !ok_ptr(slot_rows) || !ok_ptr(active_experts) ||
      !ok_ptr(num_active))
    return MOE_ERR_INVALID_ARG;
  const size_t need = permute_workspace_bytes(T, E);
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE;
  if (need > 0 && !ok_ptr(workspace)) return MOE_ERR_INVALID_ARG;
  const bool one_launch =
      default_plan(T, top_k, E, 0, kGroup, kGroup).route != MOE_ROUTE_SEPARATE;
  launch_route_permute(logits, static_cast<int>(T), E, top_k, 0, topk_ids, topk_weights,
                       expert_offsets, sorted_slots, slot_rows, active_experts, num_active,
                       workspace, one_launch, static_cast<hipStream_t>(stream));
  return check_launch();
}

size_t moe_ffn_workspace_bytes(int64_t T, int32_t top_k, int32_t E, int32_t H, int32_t I) {
  if (check_routing(T, top_k, E) != MOE_OK || check_dims(H, I, kGroup) != MOE_OK) return 0;
  return ffn_workspace_bytes(T, top_k, E, H, I);
}

int moe_w4a16_gate_up(const uint16_t* x, int64_t T, int32_t top_k, const int32_t* expert_offsets,
                      const int32_t* sorted_slots, const int32_t* active_experts,
                      const int32_t* num_active, const int32_t* w13_qweight,
                      const uint16_t* w13_scales, const int32_t* w13_qzeros, int32_t E, int32_t H,
                      int32_t I, int32_t group_size, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (int st = check_routing(T, top_k, E)) return st;
  if (int st = check_dims(H, I, group_size)) return st;
  const Plan pl = default_plan(T, top_k, E, 0, H, I);
  if (int st = check_mfma(pl, T, top_k, E, H, I)) return st;
  if (int st = check_gemv(pl, T, top_k, E, 0, H, I)) return st;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(x) || !ok_ptr(expert_offsets) || !ok_ptr(sorted_slots) || !ok_ptr(active_experts) ||
      !ok_ptr(num_active) || !ok_ptr(w13_qweight) || !ok_ptr(w13_scales) || !ok_ptr(w13_qzeros) ||
      !ok_ptr(workspace))
    return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < ffn_workspace_bytes(T, top_k, E, H, I)) return MOE_ERR_WORKSPACE;
  GateUpArgs a;
  a.x = x;
  a.T = static_cast<int>(T);
  a.top_k = top_k;
  a.E = E;
  a.H = H;
  a.I = I;
  a.offsets = expert_offsets;
  a.sorted_slots = sorted_slots;
  a.active = active_experts;
  a.num_active = num_active;
  a.qw = w13_qweight;
  a.sc = w13_scales;
  a.qz = w13_qzeros;
  run_gate_up(a, pl, workspace, static_cast<hipStream_t>(stream));
  return check_launch();
}

int moe_route_gate_up(const float* logits, const uint16_t* x, int64_t T, int32_t E, int32_t top_k,
                      const int32_t* w13_qweight, const uint16_t* w13_scales,
                      const int32_t* w13_qzeros, int32_t H, int32_t I, int32_t group_size,
                      int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                      int32_t* sorted_slots, int32_t* slot_rows, int32_t* active_experts,
                      int32_t* num_active, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (int st = check_routing(T, top_k, E)) return st;
  if (int st = check_dims(H, I, group_size)) return st;
  Plan pl = default_plan(T, top_k, E, 0, H, I);
  pl.ffn = MOE_FFN_GEMV;
  pl.route = MOE_ROUTE_IN_GATE_UP;
  if (plan_check(pl, T, top_k, E, 0, H, I) != MOE_OK) return MOE_ERR_UNSUPPORTED;
  if (int st = check_gemv(pl, T, top_k, E, 0, H, I)) return st;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(logits) || !ok_ptr(x) || !ok_ptr(w13_qweight) || !ok_ptr(w13_scales) ||
      !ok_ptr(w13_qzeros) || !ok_ptr(topk_ids) || !ok_ptr(topk_weights) ||
      !ok_ptr(expert_offsets) || !ok_ptr(sorted_slots) || !ok_ptr(slot_rows) ||
      !ok_ptr(active_experts) || !ok_ptr(num_active) || !ok_ptr(workspace))
    return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < ffn_workspace_bytes(T, top_k, E, H, I)) return MOE_ERR_WORKSPACE;
  const FfnWorkspace ws = ffn_workspace_carve(workspace, T, top_k, E, H, I);
  GateUpArgs a{};
  a.x = x;
  a.T = static_cast<int>(T);
  a.top_k = top_k;
  a.E = E;
  a.H = H;
  a.I = I;
  a.qw = w13_qweight;
  a.sc = w13_scales;
  a.qz = w13_qzeros;
  a.lanes = pl.lanes_gate_up;
  a.rows_per_pass = pl.rows_per_pass;
  a.cost_split = pl.cost_split;
  const RouteOut r{topk_ids, topk_weights, expert_offsets, sorted_slots, slot_rows,
                   active_experts, num_active};
  launch_route_gate_up_decode(logits, a, r, ws, static_cast<hipStream_t>(stream));
  return check_launch();
}

int moe_w4a16_down(int64_t T, int32_t top_k, const int32_t* expert_offsets,
                   const int32_t* active_experts, const int32_t* num_active,
                   const int32_t* w2_qweight, const uint16_t* w2_scales, const int32_t* w2_qzeros,
                   int32_t E, int32_t H, int32_t I, int32_t group_size, float* y_sorted,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (int st = check_routing(T, top_k, E)) return st;
  if (int st = check_dims(H, I, group_size)) return st;
  const Plan pl = default_plan(T, top_k, E, 0, H, I);
  if (int st = check_mfma(pl, T, top_k, E, H, I)) return st;
  if (int st = check_gemv(pl, T, top_k, E, 0, H, I)) return st;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(expert_offsets) || !ok_ptr(active_experts) || !ok_ptr(num_active) ||
      !ok_ptr(w2_qweight) || !ok_ptr(w2_scales) || !ok_ptr(w2_qzeros) || !ok_ptr(y_sorted) ||
      !ok_ptr(workspace))
    return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < ffn_workspace_bytes(T, top_k, E, H, I)) return MOE_ERR_WORKSPACE;
  DownArgs a;
  a.T = static_cast<int>(T);
  a.top_k = top_k;
  a.E = E;
  a.H = H;
  a.I = I;
  a.offsets = expert_offsets;
  a.active = active_experts;
  a.num_active = num_active;
  a.qw = w2_qweight;
  a.sc = w2_scales;
  a.qz = w2_qzeros;
  a.y = y_sorted;
  run_down(a, pl, workspace, static_cast<hipStream_t>(stream));
  return check_launch();
}

int moe_w4a16_grouped_ffn(const uint16_t* x, int64_t T, int32_t top_k,
                          const int32_t* expert_offsets, const int32_t* sorted_slots,
                          const int32_t* active_experts, const int32_t* num_active,
                          const int32_t* w13_qweight, const uint16_t* w13_scales,
                          const int32_t* w13_qzeros, const int32_t* w2_qweight,
                          const uint16_t* w2_scales, const int32_t* w2_qzeros, int32_t E,
                          int32_t H, int32_t I, int32_t group_size, float* y_sorted,
                          void* workspace, size_t workspace_bytes, void* stream) {
  // Validate everything before enqueuing either half.
  if (int st = check_routing(T, top_k, E)) return st;
  if (int st = check_dims(H, I, group_size)) return st;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(w2_qweight) || !ok_ptr(w2_scales) || !ok_ptr(w2_qzeros) || !ok_ptr(y_sorted))
    return MOE_ERR_INVALID_ARG;
  if (int st = moe_w4a16_gate_up(x, T, top_k, expert_offsets, sorted_slots, active_experts,
                                 num_active, w13_qweight, w13_scales, w13_qzeros, E, H, I,
                                 group_size, workspace, workspace_bytes, stream))
    return st;
  return moe_w4a16_down(T, top_k, expert_offsets, active_experts, num_active, w2_qweight,
                        w2_scales, w2_qzeros, E, H, I, group_size, y_sorted, workspace,
                        workspace_bytes, stream);
}

int moe_combine(const float* y_sorted, const float* topk_weights, const int32_t* slot_rows,
                int64_t T, int32_t top_k, int32_t H, uint16_t* out, void* stream) {
  if (T < 0 || top_k < 1 || top_k > kMaxTopK) return top_k > kMaxTopK ? MOE_ERR_UNSUPPORTED
                                                                        : MOE_ERR_INVALID_ARG;
  if (T * static_cast<int64_t>(top_k) > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (H <= 0 || H % kGroup) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(y_sorted) || !ok_ptr(topk_weights) || !ok_ptr(slot_rows) || !ok_ptr(out))
    return MOE_ERR_INVALID_ARG;
  launch_combine(y_sorted, topk_weights, slot_rows, static_cast<int>(T), top_k, H, out,
                 static_cast<hipStream_t>(stream));
  return check_launch();
}

// ---- the whole layer ---------------------------------------------------------
// Workspace: the routing arrays (ids, weights, offsets, sorted slots, slot
// rows, active list, active count), the permutation and FFN workspaces and
// y_sorted, each 256-byte aligned.
struct LayerWs {
  int32_t* ids;
  float* weights;
  int32_t* offsets;
  int32_t* sorted;
  int32_t* slot_rows;
  int32_t* active;
  int32_t* num_active;
  void* perm;
  size_t perm_bytes;
  void* ffn;
  size_t ffn_bytes;
  float* y;
  size_t total;
};

static LayerWs layer_ws(void* base, int64_t T, int32_t top_k, int32_t E, int32_t H, int32_t I) {
  const size_t S = static_cast<size_t>(T) * top_k;
  char* p = static_cast<char*>(base);
  size_t at = 0;
  auto take = [&](size_t n) {
    char* q = p ? p + at : nullptr;
    at += align256(n);
    return q;
  };
  LayerWs w;
  w.ids = reinterpret_cast<int32_t*>(take(4 * S));
  w.weights = reinterpret_cast<float*>(take(4 * S));
  w.offsets = reinterpret_cast<int32_t*>(take(4 * (static_cast<size_t>(E) + 1)));
  w.sorted = reinterpret_cast<int32_t*>(take(4 * S));
  w.slot_rows = reinterpret_cast<int32_t*>(take(4 * S));
  w.active = reinterpret_cast<int32_t*>(take(4 * static_cast<size_t>(E)));
  w.num_active = reinterpret_cast<int32_t*>(take(4));
  w.perm_bytes = permute_workspace_bytes(T, E);
  w.perm = take(w.perm_bytes);
  w.ffn_bytes = ffn_workspace_bytes(T, top_k, E, H, I);
  w.ffn = take(w.ffn_bytes);
  w.y = reinterpret_cast<float*>(take(4 * S * static_cast<size_t>(H)));
  w.total = at;
  return w;
}

size_t moe_layer_workspace_bytes(int64_t T, int32_t top_k, int32_t E, int32_t H, int32_t I) {
  if (check_routing(T, top_k, E) != MOE_OK || check_dims(H, I, kGroup) != MOE_OK) return 0;
  return layer_ws(nullptr, T, top_k, E, H, I).total;
}

// Sizes, plan and pointers of a layer call (the shared expert, when `shared`
// is 1, adds one slot per token and one expert); MOE_OK or the error to
// return.  `pl` is the plan for top_k + shared slots and E + shared experts.
static int layer_check(const float* logits, const uint16_t* x, int64_t T, int32_t E,
                       int32_t top_k, int32_t shared, const int32_t* w13_qweight,
                       const uint16_t* w13_scales, const int32_t* w13_qzeros,
                       const int32_t* w2_qweight, const uint16_t* w2_scales,
                       const int32_t* w2_qzeros, int32_t H, int32_t I, int32_t group_size,
                       const uint16_t* out, const void* workspace, size_t workspace_bytes,
                       const Plan& pl) {
  if (shared != 0 && shared != 1) return MOE_ERR_INVALID_ARG;
  if (int st = check_routing(T, top_k, E)) return st;
  if (int st = check_routing(T, top_k + shared, E + shared)) return st;
  if (int st = check_dims(H, I, group_size)) return st;
  if (int st = plan_check(pl, T, top_k, E, shared, H, I)) return st;
  if (int st = check_mfma(pl, T, top_k + shared, E + shared, H, I)) return st;
  if (int st = check_gemv(pl, T, top_k, E, shared, H, I)) return st;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(logits) || !ok_ptr(x) || !ok_ptr(w13_qweight) || !ok_ptr(w13_scales) ||
      !ok_ptr(w13_qzeros) || !ok_ptr(w2_qweight) || !ok_ptr(w2_scales) || !ok_ptr(w2_qzeros) ||
      !ok_ptr(out) || !ok_ptr(workspace))
    return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < layer_ws(nullptr, T, top_k + shared, E + shared, H, I).total)
    return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// Enqueues a layer call that layer_check accepted.  With the shared expert
// the routing gives every token one more slot, (expert E, weight 1), and the
// permutation, the FFN and the combine run over E + 1 experts and top_k + 1
// slots, so the shared expert's rows go through the same launches as the
// routed experts' rows (its default plan takes all its T rows in one pass
// and shares the GEMV work out by cost).
static int layer_run(const float* logits, const uint16_t* x, int64_t T, int32_t E, int32_t top_k,
                     int32_t shared, const int32_t* w13_qweight, const uint16_t* w13_scales,
                     const int32_t* w13_qzeros, const int32_t* w2_qweight,
                     const uint16_t* w2_scales, const int32_t* w2_qzeros, int32_t H, int32_t I,
                     uint16_t* out, void* workspace, const Plan& pl, void* stream) {
  if (T == 0) return MOE_OK;
  const int32_t kk = top_k + shared, EP = E + shared;
  const LayerWs w = layer_ws(workspace, T, kk, EP, H, I);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  GateUpArgs a{};
  a.x = x;
  a.T = static_cast<int>(T);
  a.top_k = kk;
  a.E = EP;
  a.shared = shared;
  a.H = H;
  a.I = I;
  a.offsets = w.offsets;
  a.sorted_slots = w.sorted;
  a.active = w.active;
  a.num_active = w.num_active;
  a.qw = w13_qweight;
  a.sc = w13_scales;
  a.qz = w13_qzeros;
  DownArgs d{};
  d.T = static_cast<int>(T);
  d.top_k = kk;
  d.E = EP;
  d.H = H;
  d.I = I;
  d.offsets = w.offsets;
  d.active = w.active;
  d.num_active = w.num_active;
  d.qw = w2_qweight;
  d.sc = w2_scales;
  d.qz = w2_qzeros;
  d.y = w.y;
  if (pl.one_launch) {
    // routing, gate/up and down in one launch, then the combine
    const FfnWorkspace fws = ffn_workspace_carve(w.ffn, T, kk, EP, H, I);
    a.lanes = pl.lanes_gate_up;
    a.rows_per_pass = pl.rows_per_pass;
    d.lanes = pl.lanes_down;
    const RouteOut r{w.ids, w.weights, w.offsets, w.sorted, w.slot_rows, w.active, w.num_active};
    launch_one_launch_decode(logits, a, d, r, fws, st);
    launch_combine(w.y, w.weights, w.slot_rows, static_cast<int>(T), kk, H, out, st);
    return check_launch();
  }
  if (pl.route == MOE_ROUTE_IN_GATE_UP) {
    // the gate/up GEMV routes the tokens itself
    const FfnWorkspace fws = ffn_workspace_carve(w.ffn, T, kk, EP, H, I);
    a.lanes = pl.lanes_gate_up;
    a.rows_per_pass = pl.rows_per_pass;
    a.cost_split = pl.cost_split;
    a.shared_mfma = pl.shared_mfma;
    const RouteOut r{w.ids, w.weights, w.offsets, w.sorted, w.slot_rows, w.active, w.num_active};
    launch_route_gate_up_decode(logits, a, r, fws, st);
  } else {
    launch_route_permute(logits, static_cast<int>(T), E, top_k, shared, w.ids, w.weights,
                         w.offsets, w.sorted, w.slot_rows, w.active, w.num_active, w.perm,
                         pl.route == MOE_ROUTE_ONE_LAUNCH, st);
    run_gate_up(a, pl, w.ffn, st);
  }
  if (pl.combine_in_down) {  // the down GEMV writes out itself
    d.combine = 1;
    d.c_weights = w.weights;
    d.c_slot_rows = w.slot_rows;
    d.out = out;
  }
  run_down(d, pl, w.ffn, st);
  if (!pl.combine_in_down)
    launch_combine(w.y, w.weights, w.slot_rows, static_cast<int>(T), kk, H, out, st);
  return check_launch();
}

// The plan to use: the caller's, or the default for the layer's sizes.
static Plan layer_plan(const moe_plan* plan, int64_t T, int32_t top_k, int32_t E, int32_t shared,
                       int32_t H, int32_t I) {
  return plan ? *plan : default_plan(T, top_k, E, shared, H, I);
}

static int layer_forward(const float* logits, const uint16_t* x, int64_t T, int32_t E,
                         int32_t top_k, int32_t shared, const int32_t* w13_qweight,
                         const uint16_t* w13_scales, const int32_t* w13_qzeros,
                         const int32_t* w2_qweight, const uint16_t* w2_scales,
                         const int32_t* w2_qzeros, int32_t H, int32_t I, int32_t group_size,
                         uint16_t* out, void* workspace, size_t workspace_bytes,
                         const moe_plan* plan, void* stream) {
  const Plan pl = layer_plan(plan, T, top_k, E, shared, H, I);
  if (int st = layer_check(logits, x, T, E, top_k, shared, w13_qweight, w13_scales, w13_qzeros,
                           w2_qweight, w2_scales, w2_qzeros, H, I, group_size, out, workspace,
                           workspace_bytes, pl))
    return st;
  return layer_run(logits, x, T, E, top_k, shared, w13_qweight, w13_scales, w13_qzeros,
                   w2_qweight, w2_scales, w2_qzeros, H, I, out, workspace, pl, stream);
}

int moe_plan_default(int64_t T, int32_t top_k, int32_t E, int32_t shared, int32_t H, int32_t I,
                     moe_plan* plan) {
  if (shared != 0 && shared != 1) return MOE_ERR_INVALID_ARG;
  if (int st = check_routing(T, top_k, E)) return st;
  if (int st = check_routing(T, top_k + shared, E + shared)) return st;
  if (int st = check_dims(H, I, kGroup)) return st;
  if (plan == nullptr) return MOE_ERR_INVALID_ARG;
  *plan = default_plan(T, top_k, E, shared, H, I);
  return MOE_OK;
}

int moe_layer_forward(const float* logits, const uint16_t* x, int64_t T, int32_t E, int32_t top_k,
                      const int32_t* w13_qweight, const uint16_t* w13_scales,
                      const int32_t* w13_qzeros, const int32_t* w2_qweight,
                      const uint16_t* w2_scales, const int32_t* w2_qzeros, int32_t H, int32_t I,
                      int32_t group_size, uint16_t* out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return layer_forward(logits, x, T, E, top_k, 0, w13_qweight, w13_scales, w13_qzeros,
                       w2_qweight, w2_scales, w2_qzeros, H, I, group_size, out, workspace,
                       workspace_bytes, nullptr, stream);
}

int moe_layer_forward_plan(const float* logits, const uint16_t* x, int64_t T, int32_t E,
                           int32_t top_k, const int32_t* w13_qweight, const uint16_t* w13_scales,
                           const int32_t* w13_qzeros, const int32_t* w2_qweight,
                           const uint16_t* w2_scales, const int32_t* w2_qzeros, int32_t H,
                           int32_t I, int32_t group_size, uint16_t* out, void* workspace,
                           size_t workspace_bytes, const moe_plan* plan, void* stream) {
  return layer_forward(logits, x, T, E, top_k, 0, w13_qweight, w13_scales, w13_qzeros,
                       w2_qweight, w2_scales, w2_qzeros, H, I, group_size, out, workspace,
                       workspace_bytes, plan, stream);
}

size_t moe_block_workspace_bytes(int64_t T, int32_t top_k, int32_t E, int32_t shared, int32_t H,
                                 int32_t I) {
  if (shared != 0 && shared != 1) return 0;
  if (check_routing(T, top_k, E) != MOE_OK || check_routing(T, top_k + shared, E + shared) != MOE_OK ||
      check_dims(H, I, kGroup) != MOE_OK)
    return 0;
  return layer_ws(nullptr, T, top_k + shared, E + shared, H, I).total;
}

int moe_block_forward_plan(const uint16_t* x, int64_t T, const uint16_t* gate_weight, int32_t E,
                           int32_t top_k, int32_t shared, const int32_t* w13_qweight,
                           const uint16_t* w13_scales, const int32_t* w13_qzeros,
                           const int32_t* w2_qweight, const uint16_t* w2_scales,
                           const int32_t* w2_qzeros, int32_t H, int32_t I, int32_t group_size,
                           float* logits, uint16_t* out, void* workspace, size_t workspace_bytes,
                           const moe_plan* plan, void* stream) {
  // everything is checked before the projection is enqueued
  if (int st = check_router_gate(T, H, E)) return st;
  const Plan pl = layer_plan(plan, T, top_k, E, shared, H, I);
  if (int st = layer_check(logits, x, T, E, top_k, shared, w13_qweight, w13_scales, w13_qzeros,
                           w2_qweight, w2_scales, w2_qzeros, H, I, group_size, out, workspace,
                           workspace_bytes, pl))
    return st;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(gate_weight)) return MOE_ERR_INVALID_ARG;
  launch_router_gate(x, static_cast<int>(T), H, gate_weight, E, logits, pl.router_gemv != 0,
                     static_cast<hipStream_t>(stream));
  if (int e = check_launch()) return e;
  return layer_run(logits, x, T, E, top_k, shared, w13_qweight, w13_scales, w13_qzeros,
                   w2_qweight, w2_scales, w2_qzeros, H, I, out, workspace, pl, stream);
}

int moe_block_forward(const uint16_t* x, int64_t T, const uint16_t* gate_weight, int32_t E,
                      int32_t top_k, int32_t shared, const int32_t* w13_qweight,
                      const uint16_t* w13_scales, const int32_t* w13_qzeros,
                      const int32_t* w2_qweight, const uint16_t* w2_scales,
                      const int32_t* w2_qzeros, int32_t H, int32_t I, int32_t group_size,
                      float* logits, uint16_t* out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return moe_block_forward_plan(x, T, gate_weight, E, top_k, shared, w13_qweight, w13_scales,
                                w13_qzeros, w2_qweight, w2_scales, w2_qzeros, H, I, group_size,
                                logits, out, workspace, workspace_bytes, nullptr, stream);
}

}  // extern "C"

// ---- the whole layer without a workspace argument ----------------------------
// The scratch of moe_layer_forward_noalloc: one array per device, held from
// module load to process end.  In host code `scratch` only names the symbol;
// its device address (different on every device) comes from
// hipGetSymbolAddress with that device current, and only that address is
// passed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

std::atomic<void*> scratch_ptr[moe::kMaxDevices];

// The current device's address of `scratch` (looked up once per device), or
// nullptr with *err set when the runtime call fails.
void* device_scratch(int* err) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= moe::kMaxDevices) {
    *err = MOE_ERR_HIP;
    return nullptr;
  }
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      *err = MOE_ERR_HIP;
      return nullptr;
    }
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" int moe_layer_forward_noalloc(const float* logits, const uint16_t* x, int64_t T,
                                         int32_t E, int32_t top_k, const int32_t* w13_qweight,
                                         const uint16_t* w13_scales, const int32_t* w13_qzeros,
                                         const int32_t* w2_qweight, const uint16_t* w2_scales,
                                         const int32_t* w2_qzeros, int32_t H, int32_t I,
                                         int32_t group_size, uint16_t* out, void* stream) {
  // sizes first: nothing is looked up or enqueued for a call that cannot run
  if (int st = check_routing(T, top_k, E)) return st;
  if (int st = check_dims(H, I, group_size)) return st;
  if (T == 0) return MOE_OK;
  if (layer_ws(nullptr, T, top_k, E, H, I).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  int err = MOE_OK;
  void* ws = device_scratch(&err);
  if (ws == nullptr) return err;
  return layer_forward(logits, x, T, E, top_k, 0, w13_qweight, w13_scales, w13_qzeros,
                       w2_qweight, w2_scales, w2_qzeros, H, I, group_size, out, ws,
                       MOE_NOALLOC_SCRATCH_BYTES, nullptr, stream);
}
