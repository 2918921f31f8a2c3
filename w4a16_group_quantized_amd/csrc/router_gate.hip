// Router gate projection: logits[t, e] = sum_h x[t, h] * Wg[e, h], fp16 x
// [T, H] and fp16 Wg [E, H], fp32 logits [T, E].  The hidden -> expert
// projection in front of the router ("[Perf][SM70] Narrow Qwen3.8 AWQ active
// grouped decode", section "Capacity, startup, and remaining limit", names the
// shared projection among the remaining decode costs; 512 experts over hidden
// 2560 as in "[Model][SM70] Adapt Qwen3.8 Flash Next NVFP4", section
// "Implemented route").
//
// Few tokens (T <= 16, decode): the work is reading Wg once (2.6 MB at
// 512 x 2560), so it is a GEMV bound by HBM.  One wave per expert row: lane l
// takes the row's 16-byte chunks l, l + 64, ... and the same chunks of every
// token's x row (x stays in L2); v_dot2_f32_f16 multiplies fp16 pairs
// exactly and accumulates in fp32; the 64 lanes' sums are added by DPP and
// two shuffles in a fixed order.
//
// More tokens: a dense GEMM on v_mfma_f32_32x32x16_f16.  A workgroup computes
// a 64-token x 64-expert tile with four waves of 32 x 32; per K step of 64 it
// stages both operand tiles in LDS (double buffered, next step loaded into
// registers while the current one is multiplied).  Tiles are numbered
// token-tile-major and every XCD takes a contiguous run of them, so the
// workgroups of one XCD share each token tile in their L2 (Wg, 2.6 MB, stays
// in every XCD's L2).
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kBufferFlags = 0x00020000;  // buffer descriptor word 3 for raw dword access on gfx9
constexpr int kGemvMaxT = 16;             // tokens of the GEMV variant
constexpr int kGemvWin = 4;               // 16-byte weight chunks per lane and window
constexpr int kGemvHalf = kGemvMaxT / 2;  // tokens whose x loads go out together
constexpr int kXcds = 8;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           kBufferFlags);
}

__device__ __forceinline__ uint4 load_b128(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(byte_off), 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false);
  return v + __builtin_bit_cast(float, moved);
}

// Sum over the 64 lanes, the same value in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);  // row_half_mirror
  v = dpp_add<0x140>(v);  // row_mirror
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ float dot8(const uint4 a, const uint4 b, float c) {
  c = dot2_f16(a.x, b.x, c);
  c = dot2_f16(a.y, b.y, c);
  c = dot2_f16(a.z, b.z, c);
  return dot2_f16(a.w, b.w, c);
}

// ---- few tokens: one wave per expert row -------------------------------------
// A workgroup of one wave per expert row (E workgroups: every compute unit
// takes some).  Lane l takes the row's 16-byte chunks l, l + 64, ... in
// windows of kGemvWin; for each chunk it loads the matching chunk of every
// token's x row straight from global memory (x, T x H fp16, is read by every
// row and stays in L2), so nothing waits on a staging pass or a barrier.
__global__ __launch_bounds__(64) void router_gemv_kernel(const uint16_t* __restrict__ x, int T,
                                                         int H, const uint16_t* __restrict__ wg,
                                                         int E, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x;
  const int nch = H / 8;  // 16-byte chunks per row
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wg + static_cast<size_t>(e) * H, static_cast<uint32_t>(H) * 2u);
  const uint32_t x_end = static_cast<uint32_t>(T) * H * 2u;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, x_end);

  float acc[kGemvMaxT];
#pragma unroll
  for (int t = 0; t < kGemvMaxT; ++t) acc[t] = 0.f;
  for (int base = 0; base < nch; base += 64 * kGemvWin) {
    // chunks past the row read zeros (offsets at or past the buffer's end)
    int c[kGemvWin];
    uint4 w[kGemvWin];
#pragma unroll
    for (int i = 0; i < kGemvWin; ++i) {
      c[i] = base + i * 64 + lane;
      w[i] = load_b128(rw, c[i] < nch ? static_cast<uint32_t>(c[i]) * 16u : static_cast<uint32_t>(H) * 2u);
    }
    // tokens in halves of kGemvHalf: all of a half's x loads go out before
    // its dot products
    auto half = [&](auto t0_tag) {
      constexpr int T0 = decltype(t0_tag)::value;
      uint4 xv[kGemvHalf][kGemvWin];
#pragma unroll
      for (int tt = 0; tt < kGemvHalf; ++tt)
#pragma unroll
        for (int i = 0; i < kGemvWin; ++i) {
          const bool in = T0 + tt < T && c[i] < nch;
          xv[tt][i] = load_b128(rx, in ? (static_cast<uint32_t>(T0 + tt) * nch + c[i]) * 16u : x_end);
        }
#pragma unroll
      for (int tt = 0; tt < kGemvHalf; ++tt)
#pragma unroll
        for (int i = 0; i < kGemvWin; ++i) acc[T0 + tt] = dot8(w[i], xv[tt][i], acc[T0 + tt]);
    };
    half(std::integral_constant<int, 0>{});
    if (T > kGemvHalf) half(std::integral_constant<int, kGemvHalf>{});
  }
#pragma unroll
  for (int t = 0; t < kGemvMaxT; ++t) {
    if (t < T) {
      const float v = wave_sum(acc[t]);
      if (lane == t) logits[static_cast<size_t>(t) * E + e] = v;
    }
  }
}

// ---- more tokens: 64 x 64 tiles on the matrix cores ---------------------------
constexpr int kTile = 64;               // tokens and experts per workgroup tile
constexpr int kKs = 64;                 // K per step
constexpr int kRowPad = kKs + 8;        // LDS row stride in halves (144 bytes: reads spread over banks)
constexpr int kMmThreads = 256;
constexpr int kLoadsPerThread = kTile * kKs / 8 / kMmThreads;  // 16-byte chunks per operand per thread (2)

__global__ __launch_bounds__(kMmThreads) void router_mfma_kernel(
    const uint16_t* __restrict__ x, int T, int H, const uint16_t* __restrict__ wg, int E,
    float* __restrict__ logits, int n_mtiles, int n_ntiles) {
  __shared__ __align__(16) uint16_t sa[2][kTile * kRowPad];
  __shared__ __align__(16) uint16_t sb[2][kTile * kRowPad];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int j = lane & 31, h = lane >> 5;

  // tile of this workgroup: XCD x (blocks x, x + 8, ...) takes a contiguous
  // run of the token-tile-major order
  const int total = n_mtiles * n_ntiles;
  const int id = blockIdx.x;
  const int item = (total % kXcds == 0) ? (id % kXcds) * (total / kXcds) + id / kXcds : id;
  const int mt = item / n_ntiles, nt = item - mt * n_ntiles;
  const int m0 = mt * kTile, n0 = nt * kTile;

  // operand rows past T or E read zeros (offsets at or past the buffer end)
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(x, static_cast<uint32_t>(T) * H * 2u);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(wg, static_cast<uint32_t>(E) * H * 2u);
  const uint32_t a_end = static_cast<uint32_t>(T) * H * 2u, b_end = static_cast<uint32_t>(E) * H * 2u;
  uint32_t a_off[kLoadsPerThread], b_off[kLoadsPerThread];
  int s_at[kLoadsPerThread], k_at[kLoadsPerThread];
#pragma unroll
  for (int i = 0; i < kLoadsPerThread; ++i) {
    const int c = tid + i * kMmThreads;  // chunk of the tile: row c / 8, 8-half column c % 8
    const int r = c >> 3, col = (c & 7) * 8;
    a_off[i] = m0 + r < T ? (static_cast<uint32_t>(m0 + r) * H + col) * 2u : a_end;
    b_off[i] = n0 + r < E ? (static_cast<uint32_t>(n0 + r) * H + col) * 2u : b_end;
    s_at[i] = r * kRowPad + col;
    k_at[i] = col;
  }
  uint4 ga[kLoadsPerThread], gb[kLoadsPerThread];
  // K step from k0; the columns past H of a last half step read zeros
  auto load_step = [&](int k0) {
    const uint32_t kb = static_cast<uint32_t>(k0) * 2u;
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      const bool kin = k0 + k_at[i] < H;
      ga[i] = load_b128(ra, a_off[i] == a_end || !kin ? a_end : a_off[i] + kb);
      gb[i] = load_b128(rb, b_off[i] == b_end || !kin ? b_end : b_off[i] + kb);
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      *reinterpret_cast<uint4*>(&sa[buf][s_at[i]]) = ga[i];
      *reinterpret_cast<uint4*>(&sb[buf][s_at[i]]) = gb[i];
    }
  };

  float16v acc = float16v{};
  const int nks = (H + kKs - 1) / kKs;  // H is a multiple of 32
  load_step(0);
  store_step(0);
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nks) load_step((ks + 1) * kKs);
    const uint16_t* pa = &sa[buf][(wm * 32 + j) * kRowPad + 8 * h];
    const uint16_t* pb = &sb[buf][(wn * 32 + j) * kRowPad + 8 * h];
#pragma unroll
    for (int t = 0; t < kKs / 16; ++t) {
      // lane (h, j): row j of each operand, k block 16 t + 8 h (the same k for both)
      const half8 a = *reinterpret_cast<const half8*>(pa + 16 * t);
      const half8 b = *reinterpret_cast<const half8*>(pb + 16 * t);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
    }
    if (ks + 1 < nks) store_step(buf ^ 1);
    __syncthreads();
  }

  // lane (h, j) holds tokens 8 (v / 4) + 4 h + v % 4 of the wave's 32, expert j
  const int col = n0 + wn * 32 + j;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = m0 + wm * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
    if (row < T && col < E) logits[static_cast<size_t>(row) * E + col] = acc[v];
  }
}

}  // namespace

void launch_router_gate(const uint16_t* x, int T, int H, const uint16_t* gate_weight, int E,
                        float* logits, bool gemv, hipStream_t stream) {
  if (gemv) {  // T <= kGemvMaxT (the plan checks it)
    hipLaunchKernelGGL(router_gemv_kernel, dim3(E), dim3(64), 0, stream, x, T, H, gate_weight, E,
                       logits);
    return;
  }
  const int n_m = (T + kTile - 1) / kTile, n_n = (E + kTile - 1) / kTile;
  hipLaunchKernelGGL(router_mfma_kernel, dim3(n_m * n_n), dim3(kMmThreads), 0, stream, x, T, H,
                     gate_weight, E, logits, n_m, n_n);
}

}  // namespace moe
