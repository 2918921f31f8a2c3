/*
 * moe_w4a16.h - C ABI of libmoe_w4a16.so, a routed-expert mixture-of-experts
 * layer with W4A16 group-32 expert weights for AMD Instinct MI355X (gfx950).
 *
 * The layer is the one tuned across a 512-expert, top-10, hidden-2560 model on
 * the pages "[Model][SM70] Adapt Qwen3.8 Flash Next NVFP4" (section
 * "Implemented route": the (2560, 640, 512, top-10) routed-expert geometry) and
 * "[Perf][SM70] Narrow Qwen3.8 AWQ active grouped decode" (section "Purpose":
 * AWQ W4A16 with effective group size 32, a grouped operator over active
 * experts, multi-row active-expert segments with offsets-based scheduling, and
 * scratch buffers the operator mutates).  One layer call is, in order:
 *
 *   moe_route              softmax over expert logits, top-k, renormalise
 *   moe_permute            token->expert permutation: segments and offsets
 *   moe_w4a16_grouped_ffn  dequant-fused gate/up GEMM, SiLU(gate)*up, down GEMM
 *   moe_combine            router-weighted sum back to token order
 *
 * Around it (the MoE block): moe_router_gate makes the logits from the
 * activations, and a shared expert runs on every token beside the routed
 * ones (moe_route_shared, moe_block_forward).
 *
 * Conventions for every entry point
 *   - Pointers to tensors are DEVICE pointers unless stated otherwise; fp16
 *     tensors are passed as uint16_t bit patterns.  Every non-null tensor
 *     pointer must be 16-byte aligned.  All tensors are dense, row-major.
 *   - Ownership: the caller allocates and frees every buffer, including the
 *     workspaces.  The library never allocates or frees memory and never
 *     synchronises.  Its only state is a per-device cache of two device
 *     attributes (compute-unit count, LDS bytes per workgroup) read from the
 *     runtime on first use, the per-device scratch array of
 *     moe_layer_forward_noalloc with its address cache, and the per-device
 *     completion counts of the one-launch FFN plan (moe_plan.one_launch),
 *     which every such call leaves at zero.  Entry points other than
 *     moe_layer_forward_noalloc, and plans other than one_launch, may be
 *     called from several host threads at once.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream) and runs asynchronously.  A call that returns MOE_OK has
 *     only enqueued its kernels.
 *   - Errors: arguments are validated on the host before anything is enqueued;
 *     on a non-OK return nothing was enqueued, except MOE_ERR_HIP, which
 *     reports a failed launch (the library reads and clears hipGetLastError,
 *     so a pending error left by earlier unrelated work is reported too).
 *   - T == 0 is valid: the call returns MOE_OK, enqueues nothing and writes
 *     nothing; tensor pointers may then be NULL.
 *   - Device-side preconditions that are documented but not checked: logits
 *     are finite; expert ids are in [0, E) and distinct within a token (what
 *     moe_route produces); routing tensors passed to a later call are the
 *     unmodified outputs of the earlier calls of the same layer.
 *   - Results are deterministic: no step depends on the order in which
 *     threads or workgroups run, so a repeated call gives identical bits.
 *
 * Shapes.  T tokens, E experts, top_k experts per token, S = T * top_k slots
 * (slot s = t * top_k + j is the j-th choice of token t), hidden size H,
 * intermediate size I, group size 32 along the reduction dim K.
 *
 * Weight layout (N = output rows, K = reduction dim, G = K / 32):
 *   qweight int32 [E, N, K/8]   nibble j (bits 4j..4j+3) of word w is k = 8w+j
 *   scales  fp16  [E, N, G]
 *   qzeros  int32 [E, N/8, G]   nibble j of word w is row n = 8w+j
 *   dequantised weight  W[e, n, k] = (q - z[e, n, k/32]) * scales[e, n, k/32]
 * w13 has N = 2I, K = H (rows [0, I) gate, [I, 2I) up); w2 has N = H, K = I.
 *
 * Limits: 1 <= E <= 4096; 1 <= top_k <= min(E, 64); S < 2^31; group_size == 32;
 * H and I multiples of 32 with 32 <= H, I <= 16384; T * H < 2^31 (x is
 * addressed with 32-bit byte offsets).
 */
#ifndef MOE_W4A16_H_
#define MOE_W4A16_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes of every entry point. */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG 1 /* null/misaligned pointer, bad shape or count   */
#define MOE_ERR_UNSUPPORTED 2 /* valid but outside the limits (group_size...)  */
#define MOE_ERR_WORKSPACE 3   /* workspace_bytes below the size query's result */
#define MOE_ERR_HIP 4         /* a kernel launch failed                        */

/* Static, NUL-terminated description of a return code (host only). */
const char* moe_status_string(int status);

/* Library ABI version, MAJOR * 100 + MINOR (1.02: moe_plan gained one_launch). */
int moe_abi_version(void);

/*
 * moe_route - router softmax, top-k and renormalisation.
 *
 * For every token t: p = softmax(logits[t, :]); the top_k experts with the
 * largest logits are chosen in rank order (equal logits: lower expert index
 * first); weights[t, j] = p[id_j] / sum_j' p[id_j'].  Ranking is done on the
 * fp32 logits themselves, so the ids are exact.  The full-softmax denominator
 * cancels in the renormalisation and is not formed.
 * Source: the routed-expert top-10 geometry on "[Model][SM70] Adapt Qwen3.8
 * Flash Next NVFP4", section "Implemented route".
 *
 *   logits        in   fp32  [T, E]
 *   topk_ids      out  int32 [T, top_k]   expert ids in rank order
 *   topk_weights  out  fp32  [T, top_k]   sum to 1 per token
 */
int moe_route(const float* logits, int64_t T, int32_t E, int32_t top_k,
              int32_t* topk_ids, float* topk_weights, void* stream);

/*
 * moe_router_gate - the router's gate projection in front of moe_route:
 * logits[t, e] = sum_h x[t, h] * gate_weight[e, h], fp16 inputs, products
 * exact, sums in fp32.  "[Perf][SM70] Narrow Qwen3.8 AWQ active grouped
 * decode", section "Capacity, startup, and remaining limit", names this
 * projection among the costs beside the routed experts; the pages give no
 * formula, so this is the plain linear map without bias, with an unquantised
 * fp16 weight.  T <= 16: one GEMV launch bound by reading gate_weight; more
 * tokens: a matrix-core GEMM.  The order of every sum is fixed.
 *
 *   x            in   fp16 [T, H]
 *   gate_weight  in   fp16 [E, H]
 *   logits       out  fp32 [T, E]
 *
 * Limits: 1 <= E <= 4096; H a multiple of 32, <= 16384; T * H < 2^31.
 */
int moe_router_gate(const uint16_t* x, int64_t T, int32_t H,
                    const uint16_t* gate_weight, int32_t E, float* logits,
                    void* stream);

/*
 * moe_route_shared - moe_route for a layer with a shared expert: row t of
 * the outputs holds top_k + 1 entries, the top_k routed choices exactly as
 * moe_route gives them, then the shared expert, id E, with weight 1.  The
 * shared expert runs on every token with weight 1 beside the routed ones
 * ("[Perf][SM70] Narrow Qwen3.8 AWQ active grouped decode", section
 * "New-base bounded integration acceptance (r2)", names the shared overlap);
 * with these rows the permutation, the FFN and the combine treat it as expert
 * E of E + 1 experts, whose weights follow the routed experts' in the weight
 * arrays.
 *
 *   logits        in   fp32  [T, E]
 *   topk_ids      out  int32 [T, top_k + 1]
 *   topk_weights  out  fp32  [T, top_k + 1]
 *
 * Limits: as moe_route with top_k + 1 <= 64 and E + 1 <= 4096.
 */
int moe_route_shared(const float* logits, int64_t T, int32_t E, int32_t top_k,
                     int32_t* topk_ids, float* topk_weights, void* stream);

/* Workspace bytes moe_permute needs for these sizes (0 when T <= 64). */
size_t moe_permute_workspace_bytes(int64_t T, int32_t top_k, int32_t E);

/*
 * moe_permute - stable token-to-expert permutation: active-expert segments and
 * their offsets ("multi-row active-expert segments and offsets-based
 * scheduling", "[Perf][SM70] Narrow Qwen3.8 AWQ active grouped decode",
 * section "Purpose").
 *
 * Sorted row r belongs to expert e iff expert_offsets[e] <= r <
 * expert_offsets[e+1]; the rows of one expert are its slots in ascending slot
 * order.
 *
 *   topk_ids        in   int32 [T, top_k]
 *   expert_offsets  out  int32 [E + 1]   offsets[0] = 0, offsets[E] = S
 *   sorted_slots    out  int32 [S]       slot held by sorted row r
 *   slot_rows       out  int32 [S]       sorted row of slot s (inverse)
 *   active_experts  out  int32 [E]       experts with >= 1 row, ascending,
 *                                        then -1 up to E
 *   num_active      out  int32 [1]       number of active experts
 *   workspace       scratch, device, >= moe_permute_workspace_bytes(...)
 *                   bytes (may be NULL when that size is 0); contents on
 *                   entry are ignored.
 */
int moe_permute(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t E,
                int32_t* expert_offsets, int32_t* sorted_slots,
                int32_t* slot_rows, int32_t* active_experts,
                int32_t* num_active, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * moe_route_permute - moe_route followed by moe_permute, in one call: the
 * outputs of both, bit for bit identical to calling them in turn (routing of
 * "[Model][SM70] Adapt Qwen3.8 Flash Next NVFP4", section "Implemented route";
 * segments and offsets of "[Perf][SM70] Narrow Qwen3.8 AWQ active grouped
 * decode", section "Purpose").  For T <= 64 and E <= 1024 it is one kernel
 * launch (the decode path); otherwise it issues the two calls' kernels.
 *
 *   logits                                   in   fp32 [T, E], as moe_route
 *   topk_ids, topk_weights                   out  as moe_route
 *   expert_offsets, sorted_slots, slot_rows,
 *   active_experts, num_active               out  as moe_permute
 *   workspace       scratch, device, >= moe_permute_workspace_bytes(T,
 *                   top_k, E) bytes (0 when T <= 64; may then be NULL);
 *                   contents on entry are ignored.
 *
 * Errors as moe_route and moe_permute; nothing is enqueued on an error.
 */
int moe_route_permute(const float* logits, int64_t T, int32_t E, int32_t top_k,
                      int32_t* topk_ids, float* topk_weights,
                      int32_t* expert_offsets, int32_t* sorted_slots,
                      int32_t* slot_rows, int32_t* active_experts,
                      int32_t* num_active, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Workspace bytes the expert FFN entry points need for these sizes. */
size_t moe_ffn_workspace_bytes(int64_t T, int32_t top_k, int32_t E, int32_t H,
                               int32_t I);

/*
 * moe_w4a16_grouped_ffn - dequant-fused grouped expert FFN over the active
 * experts (the AWQ "active-stage" grouped W4A16 operator of "[Perf][SM70]
 * Narrow Qwen3.8 AWQ active grouped decode", section "Purpose"; W4A16 group
 * size 32 per "[Model][SM70] Support Qwen3.8 Flash Next with PLE offload",
 * section "SM70 QSA prefill tuning").
 *
 * For every sorted row r of expert e, with token t = sorted_slots[r] / top_k:
 *   h = x[t, :] . W13[e]^T                (2I values)
 *   a = SiLU(h[0:I]) * h[I:2I]            (I values, SiLU(v) = v / (1 + e^-v))
 *   y_sorted[r, :] = a . W2[e]^T          (H values)
 * Weights are dequantised exactly as (q - z) and scaled per 32-wide group in
 * fp32; x . W is accumulated in fp32 and a is carried to the down product at
 * about 22 bits of precision.  The kernel variant (bandwidth-bound decode
 * GEMV for T <= 8, matrix-core grouped GEMM otherwise) is chosen from T.
 *
 *   x                 in   fp16  [T, H]
 *   expert_offsets, sorted_slots, active_experts, num_active: moe_permute's
 *                     outputs for the same routing
 *   w13_qweight/scales/qzeros   in  W13 [E, 2I, H] in the layout above
 *   w2_qweight/scales/qzeros    in  W2  [E, H, I]  in the layout above
 *   group_size        must be 32
 *   y_sorted          out  fp32  [S, H]  per-row expert outputs, sorted order
 *   workspace         scratch, device, >= moe_ffn_workspace_bytes(...) bytes;
 *                     contents on entry are ignored.  Two calls that overlap
 *                     in time must not share a workspace.
 */
int moe_w4a16_grouped_ffn(
    const uint16_t* x, int64_t T, int32_t top_k, const int32_t* expert_offsets,
    const int32_t* sorted_slots, const int32_t* active_experts,
    const int32_t* num_active, const int32_t* w13_qweight,
    const uint16_t* w13_scales, const int32_t* w13_qzeros,
    const int32_t* w2_qweight, const uint16_t* w2_scales,
    const int32_t* w2_qzeros, int32_t E, int32_t H, int32_t I,
    int32_t group_size, float* y_sorted, void* workspace,
    size_t workspace_bytes, void* stream);

/*
 * moe_w4a16_gate_up / moe_w4a16_down - the two halves of
 * moe_w4a16_grouped_ffn, for callers that schedule or time them apart.
 * moe_w4a16_gate_up computes a = SiLU(h[0:I]) * h[I:2I] for every sorted row
 * into the workspace; moe_w4a16_down reads it and writes y_sorted.  A down
 * call must follow a gate_up call with the same routing, sizes and workspace,
 * on the same stream.  Arguments are as for moe_w4a16_grouped_ffn.
 */
int moe_w4a16_gate_up(const uint16_t* x, int64_t T, int32_t top_k,
                      const int32_t* expert_offsets,
                      const int32_t* sorted_slots,
                      const int32_t* active_experts,
                      const int32_t* num_active, const int32_t* w13_qweight,
                      const uint16_t* w13_scales, const int32_t* w13_qzeros,
                      int32_t E, int32_t H, int32_t I, int32_t group_size,
                      void* workspace, size_t workspace_bytes, void* stream);

int moe_w4a16_down(int64_t T, int32_t top_k, const int32_t* expert_offsets,
                   const int32_t* active_experts, const int32_t* num_active,
                   const int32_t* w2_qweight, const uint16_t* w2_scales,
                   const int32_t* w2_qzeros, int32_t E, int32_t H, int32_t I,
                   int32_t group_size, float* y_sorted, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * moe_route_gate_up - the first launch of moe_layer_forward at decode sizes:
 * the router, the permutation and the gate/up half of the FFN as one kernel
 * (every workgroup routes the tokens itself, so none waits for another;
 * workgroup 0 writes the routing out).  Its outputs equal those of
 * moe_route_permute followed by moe_w4a16_gate_up, bit for bit, and feed
 * moe_w4a16_down and moe_combine.  "[Perf][SM70] Narrow Qwen3.8 AWQ active
 * grouped decode", section "Capacity, startup, and remaining limit", names
 * each format's MoE preparation among the remaining decode costs; this takes
 * the preparation's launch out of the step.
 *
 *   logits, x        in   as moe_layer_forward
 *   w13_*            in   as moe_w4a16_grouped_ffn
 *   topk_ids ... num_active   out  as moe_route_permute
 *   workspace        FFN workspace (moe_ffn_workspace_bytes); holds act for
 *                    moe_w4a16_down afterwards
 *
 * MOE_ERR_UNSUPPORTED unless T <= 64 and E <= 1024 (moe_layer_forward uses
 * it up to 8 tokens, the default plan); other errors as the calls it stands
 * for.
 */
int moe_route_gate_up(const float* logits, const uint16_t* x, int64_t T,
                      int32_t E, int32_t top_k, const int32_t* w13_qweight,
                      const uint16_t* w13_scales, const int32_t* w13_qzeros,
                      int32_t H, int32_t I, int32_t group_size,
                      int32_t* topk_ids, float* topk_weights,
                      int32_t* expert_offsets, int32_t* sorted_slots,
                      int32_t* slot_rows, int32_t* active_experts,
                      int32_t* num_active, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * moe_combine - router-weighted combine back to token order.
 *
 *   out[t, h] = fp16_rne( sum_{j = 0..top_k-1} topk_weights[t, j] *
 *                          y_sorted[slot_rows[t * top_k + j], h] )
 * summed in fp32 in ascending j, rounded to fp16 once (round to nearest
 * even).  A gather without atomics.
 *
 *   y_sorted      in   fp32  [S, H]
 *   topk_weights  in   fp32  [T, top_k]
 *   slot_rows     in   int32 [S]
 *   out           out  fp16  [T, H]
 */
int moe_combine(const float* y_sorted, const float* topk_weights,
                const int32_t* slot_rows, int64_t T, int32_t top_k, int32_t H,
                uint16_t* out, void* stream);

/* Workspace bytes moe_layer_forward needs for these sizes. */
size_t moe_layer_workspace_bytes(int64_t T, int32_t top_k, int32_t E, int32_t H,
                                 int32_t I);

/*
 * moe_layer_forward - the whole routed-expert layer in one call:
 * moe_route_permute, moe_w4a16_grouped_ffn and moe_combine on the same
 * arguments, with the routing, the FFN scratch and y_sorted kept in the
 * workspace; out is what the four calls produce, bit for bit (the sections
 * cited above for each step).  For T <= 8 and E <= 1024 (decode) the gate/up
 * kernel routes the tokens itself, every workgroup the same way, which saves
 * the router/permutation launch.
 *
 *   logits      in   fp32 [T, E]
 *   x           in   fp16 [T, H]
 *   w13_*, w2_* in   as moe_w4a16_grouped_ffn
 *   group_size  must be 32
 *   out         out  fp16 [T, H]
 *   workspace   scratch, device, >= moe_layer_workspace_bytes(...) bytes;
 *               contents on entry are ignored.  After the call it holds, in
 *               order and each 256-byte aligned: topk_ids [S], topk_weights
 *               [S], expert_offsets [E+1], sorted_slots [S], slot_rows [S],
 *               active_experts [E], num_active [1], the permutation
 *               workspace, the FFN workspace and y_sorted [S, H].
 *
 * Errors as the calls it stands for; nothing is enqueued on an error.
 */
int moe_layer_forward(const float* logits, const uint16_t* x, int64_t T,
                      int32_t E, int32_t top_k, const int32_t* w13_qweight,
                      const uint16_t* w13_scales, const int32_t* w13_qzeros,
                      const int32_t* w2_qweight, const uint16_t* w2_scales,
                      const int32_t* w2_qzeros, int32_t H, int32_t I,
                      int32_t group_size, uint16_t* out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Workspace bytes moe_block_forward needs for these sizes (0: invalid sizes). */
size_t moe_block_workspace_bytes(int64_t T, int32_t top_k, int32_t E,
                                 int32_t shared, int32_t H, int32_t I);

/*
 * moe_block_forward - the MoE block: moe_router_gate, then the routed layer,
 * plus the shared expert when shared == 1.  With shared == 0 it is
 * moe_router_gate followed by moe_layer_forward; with shared == 1 it is
 * moe_router_gate, moe_route_shared, then moe_permute, moe_w4a16_grouped_ffn
 * and moe_combine over E + 1 experts and top_k + 1 slots per token, so the
 * shared expert's rows run in the same launches as the routed experts' rows
 * and its output (weight 1) joins the fp32 sum before the one rounding to
 * fp16.  out is what those calls produce, bit for bit, when the plan keeps
 * the shared expert in the FFN's kernels (shared_mfma = 0); the default at
 * GEMV sizes from 3 tokens runs its rows on the matrix cores in extra
 * workgroups of the same launches (shared_mfma = 1), which changes the order
 * of its fp32 sums only, and where those rows do not fit in LDS (23 to 32
 * tokens at H = 2560) takes the matrix-core FFN instead.  Sections as moe_router_gate and moe_route_shared.
 *
 *   x            in   fp16 [T, H]
 *   gate_weight  in   fp16 [E, H]
 *   shared       0 or 1
 *   w13_*, w2_*  in   as moe_w4a16_grouped_ffn, for E + shared experts
 *                     (the shared expert is expert E)
 *   group_size   must be 32
 *   logits       out  fp32 [T, E]
 *   out          out  fp16 [T, H]
 *   workspace    scratch, device, >= moe_block_workspace_bytes(...) bytes;
 *                contents on entry are ignored.  After the call it holds the
 *                layout of moe_layer_forward's workspace for top_k + shared
 *                slots per token and E + shared experts.
 *
 * Errors as the calls it stands for; nothing is enqueued on an error.
 */
int moe_block_forward(const uint16_t* x, int64_t T, const uint16_t* gate_weight,
                      int32_t E, int32_t top_k, int32_t shared,
                      const int32_t* w13_qweight, const uint16_t* w13_scales,
                      const int32_t* w13_qzeros, const int32_t* w2_qweight,
                      const uint16_t* w2_scales, const int32_t* w2_qzeros,
                      int32_t H, int32_t I, int32_t group_size, float* logits,
                      uint16_t* out, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Kernel variant and tile profile of a layer call.  Every entry point takes
 * its choices from moe_plan_default for its sizes; the _plan entry points
 * below take an explicit one (for measuring the alternatives).  The defaults
 * were chosen from a sweep on MI355X ("[Perf][SM70] Narrow Qwen3.8 AWQ
 * active grouped decode", section "Additional existing-autotune benefit
 * (fresh-process pair)": the tuned tile per shape, there a W13 tile change
 * from M64 x 128 x 32 to M8 x 256 x 64 at 4-8 tokens).
 */
#define MOE_FFN_GEMV 0            /* one weight stream per expert, A rows from LDS  */
#define MOE_FFN_MFMA 1            /* matrix-core grouped GEMMs                      */
#define MOE_ROUTE_IN_GATE_UP 0    /* the gate/up GEMV routes the tokens itself      */
#define MOE_ROUTE_ONE_LAUNCH 1    /* router and permutation in one launch           */
#define MOE_ROUTE_SEPARATE 2      /* router kernel, then the permutation kernels    */
typedef struct moe_plan {
  int32_t ffn;            /* MOE_FFN_GEMV or MOE_FFN_MFMA                            */
  int32_t route;          /* MOE_ROUTE_*                                              */
  int32_t msub;           /* MFMA: 32-row subtiles per M-tile, 1 or 4                 */
  int32_t lanes_gate_up;  /* GEMV: lanes per w13 row, 1/2/4/8/16 dividing H/32        */
  int32_t lanes_down;     /* GEMV: lanes per w2 row, 1/2/4/8/16 dividing I/32         */
  int32_t rows_per_pass;  /* GEMV: A rows of an expert per weight pass, 1/2/4/8
                             (the down stage takes at most 4)                         */
  int32_t cost_split;     /* GEMV: 1 share work out by cost (rows per expert), 0 evenly */
  int32_t router_gemv;    /* gate projection: 1 GEMV, 0 matrix cores                  */
  int32_t shared_mfma;    /* GEMV with a shared expert: 1 its rows on the matrix cores
                             in extra workgroups of the same launches (T <= 32, with
                             T x H and 2 T x I fp16 A rows and their K-split partial
                             sums in one workgroup's LDS: T <= 22 at H = 2560),
                             0 in the GEMV with the routed experts                    */
  int32_t combine_in_down; /* layer and block calls with the GEMV, up to 2 tokens: 1
                             the down launch also writes out (each workgroup takes
                             one block of output rows of every active expert and
                             combines it; needs shared_mfma = 0, I/32/lanes_down
                             <= 8 and every act row's fragments in LDS), 0 a
                             separate combine launch; the output is the same bit
                             for bit                                                  */
  int32_t one_launch;     /* GEMV with routing in gate/up, no shared expert, even split
                             (cost_split = 0), combine_in_down = 0: 1 gate/up and down
                             in one persistent launch (one workgroup per compute unit;
                             a workgroup's down share waits, bounded, for the gate/up
                             units of its experts, on per-device completion counts),
                             0 two launches; the output is the same bit for bit.
                             Calls with it that overlap in time on one device share
                             those counts and must not be issued                      */
} moe_plan;

/*
 * moe_plan_default - the plan every entry point uses for these sizes (pure
 * host function; `plan` is a HOST pointer).  top_k and E count the routed
 * experts; shared = 1 for a layer with a shared expert (one more slot per
 * token, one more expert, which holds all T rows).  MOE_ERR_INVALID_ARG /
 * UNSUPPORTED for sizes the layer rejects.
 */
int moe_plan_default(int64_t T, int32_t top_k, int32_t E, int32_t shared, int32_t H,
                     int32_t I, moe_plan* plan);

/*
 * moe_layer_forward_plan / moe_block_forward_plan - moe_layer_forward and
 * moe_block_forward with an explicit plan (HOST pointer; NULL = the default).
 * Every plan computes the same sums and the same routing; the order of the
 * fp32 additions inside the FFN differs between GEMV and MFMA and with the
 * lanes per row, so outputs may differ in the last bits.  Limits of a plan:
 * GEMV and
 * routing in gate/up or in one launch need T <= 64; routing in gate/up needs
 * the GEMV and E (with the shared expert) <= 1024, and so does the one-launch
 * router; the projection GEMV needs T <= 16.
 * MOE_ERR_INVALID_ARG for a malformed plan, MOE_ERR_UNSUPPORTED for one these
 * sizes do not allow; nothing is enqueued then.
 */
int moe_layer_forward_plan(const float* logits, const uint16_t* x, int64_t T,
                           int32_t E, int32_t top_k, const int32_t* w13_qweight,
                           const uint16_t* w13_scales, const int32_t* w13_qzeros,
                           const int32_t* w2_qweight, const uint16_t* w2_scales,
                           const int32_t* w2_qzeros, int32_t H, int32_t I,
                           int32_t group_size, uint16_t* out, void* workspace,
                           size_t workspace_bytes, const moe_plan* plan,
                           void* stream);
int moe_block_forward_plan(const uint16_t* x, int64_t T, const uint16_t* gate_weight,
                           int32_t E, int32_t top_k, int32_t shared,
                           const int32_t* w13_qweight, const uint16_t* w13_scales,
                           const int32_t* w13_qzeros, const int32_t* w2_qweight,
                           const uint16_t* w2_scales, const int32_t* w2_qzeros,
                           int32_t H, int32_t I, int32_t group_size, float* logits,
                           uint16_t* out, void* workspace, size_t workspace_bytes,
                           const moe_plan* plan, void* stream);

/* Scratch bytes of moe_layer_forward_noalloc (per device). */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * moe_layer_forward_noalloc - moe_layer_forward for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same layer on
 * the same kernels, with the workspace taken from a scratch array that the
 * library holds on every device it runs on (MOE_NOALLOC_SCRATCH_BYTES, from
 * module load to process end).  out is what moe_layer_forward returns, bit
 * for bit.  The call allocates nothing (no hipMalloc/hipFree, no allocating
 * library routine); on its first call on a device it looks up that device's
 * scratch address once.
 *
 *   arguments   as moe_layer_forward, without workspace / workspace_bytes
 *
 * Errors as moe_layer_forward; MOE_ERR_WORKSPACE when moe_layer_workspace_bytes
 * for these sizes exceeds MOE_NOALLOC_SCRATCH_BYTES (at the 512-expert,
 * top-10, H 2560, I 640 geometry that is above about 240 tokens), and
 * MOE_ERR_HIP when the scratch address cannot be looked up; nothing is
 * enqueued then.  Every call on one device shares that device's scratch:
 * calls that overlap in time on one device (other streams, other threads)
 * race and must not be issued.  The scratch keeps the last call's contents;
 * a call reads nothing from it that it did not write itself.
 */
int moe_layer_forward_noalloc(const float* logits, const uint16_t* x, int64_t T,
                              int32_t E, int32_t top_k,
                              const int32_t* w13_qweight,
                              const uint16_t* w13_scales,
                              const int32_t* w13_qzeros,
                              const int32_t* w2_qweight,
                              const uint16_t* w2_scales,
                              const int32_t* w2_qzeros, int32_t H, int32_t I,
                              int32_t group_size, uint16_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H_ */
