/*
 * moe_w4a16.h -- C ABI of the NVFP4 weight-only (W4A16) routed-expert MoE
 * layer for AMD Instinct MI355X (gfx950).
 *
 * The layer (pages: "GLM-5.3-Flash-NVFP4-h -- W4A16 dense-side quantization",
 * intro and "Config expectations"; "GLM-5.3-Flash on Blackwell", "The
 * quantization" and "The model loaded, served an API, and produced garbage";
 * "GLM-5.3-Flash NVFP4 W4A16 for 2x RTX PRO 6000 Blackwell", intro):
 *
 *   - every routed expert has gate, up and down projections, each stored as
 *     its own NVFP4 weight-only tensor: 4-bit E2M1 codes in groups of 16
 *     along K, one E4M3 scale per group, one FP32 scale per tensor;
 *   - activations are bf16 and the layer takes NO activation scale: a
 *     weight-only checkpoint has none, and a layer that reads one computes
 *     with an uninitialised value;
 *   - the W4A16 route dequantises weights to bf16 for the matrix units;
 *   - a missing or unset global scale is refused loudly, never computed.
 *
 *   out[t] = sum_j w[t,j] * down_e( silu(gate_e(x[t])) * up_e(x[t]) ),
 *   e = ids[t,j], with (ids, w) the top-k of the router logits and a softmax
 *   over the selected k.
 *
 * Conventions for every entry point:
 *   - Pointers named d_* (and every pointer inside moe_nvfp4_tensor) are
 *     DEVICE pointers; everything else is host memory.  The caller allocates
 *     and owns all of them, the workspace included.  Device pointers must be
 *     16-byte aligned.
 *   - Work is enqueued on `stream` and returns before it completes, except
 *     where a function says it synchronises.  Nothing on the hot path
 *     (moe_route_topk, moe_w4a16_forward) allocates, frees, synchronises or
 *     issues a memset, so both may be captured into a HIP graph.
 *   - Argument, shape and alignment errors are detected on the host before
 *     anything is enqueued; the call then has no effect.  Launch failures
 *     return MOE_ERR_HIP.  A device fault surfaces at the caller's next
 *     synchronisation, as usual for HIP.
 *   - The entry points keep no state between calls and may be called from
 *     several threads at once (on different streams, or ordered on one).
 *     The only process-wide state is the benchmarking switches at the end
 *     of this header (the grouped-GEMM kernel choice and per-kernel
 *     profiling): a call reads them atomically when it starts, so changing
 *     them while other threads run forwards is safe and affects only calls
 *     made afterwards.
 *
 * Limits: 1 <= E <= 1024, 1 <= k <= min(E, 32); quantize_pack needs
 * K % 32 == 0; the forward needs H % 256 == 0 and I % 128 == 0.
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
#define MOE_OK                  0
#define MOE_ERR_INVALID_ARG   (-1)  /* null pointer, aliasing, bad enum            */
#define MOE_ERR_SHAPE         (-2)  /* dimension out of range or not a multiple    */
#define MOE_ERR_ALIGN         (-3)  /* device pointer not 16-byte aligned          */
#define MOE_ERR_UNSUPPORTED   (-4)  /* E or k beyond the compiled limits           */
#define MOE_ERR_NONFINITE     (-5)  /* validate: non-finite global scale           */
#define MOE_ERR_BAD_SCALE     (-6)  /* validate: global scale <= 0, or a NaN E4M3  */
#define MOE_ERR_WORKSPACE     (-7)  /* workspace null or smaller than required     */
#define MOE_ERR_HIP           (-8)  /* a HIP runtime call failed                   */

#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK    32

/*
 * One NVFP4 weight-only tensor stack: E experts of an [N, K] projection
 * (output features N, input features K), canonical layout:
 *   codes        [E][N][K/2]  byte i of a row = code(2i) | code(2i+1) << 4
 *                             (even k in the low nibble), E2M1 codes
 *   scales       [E][N][K/16] E4M3 ("FN") bit patterns, one per 16 k
 *   global_scale [E]          fp32, finite and > 0
 * Weight value: (E2M1(code) * E4M3(scale)) * global_scale, in fp32.
 * The struct itself lives in host memory; its pointers are device pointers.
 */
typedef struct {
    int32_t E, N, K;
    uint8_t *codes;
    uint8_t *scales;
    float *global_scale;
} moe_nvfp4_tensor;

/* Human-readable name of a status code (static storage; never NULL). */
const char *moe_status_string(moe_status status);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t moe_w4a16_version(void);

/*
 * Quantize fp32 master weights to NVFP4 (load time, not the hot path).
 * Follows the weight-only, calibration-free conversion the pages describe
 * ("GLM-5.3-Flash NVFP4 W4A16 for 2x RTX PRO 6000 Blackwell", intro;
 * "GLM-5.3-Flash-NVFP4-h", "Config expectations": group size 16 and a FP32
 * second-level scale per tensor).  Per expert e, all in fp32 with correctly
 * rounded operations in this order:
 *   g = amax|W_e| / 2688, or 1 if that is 0;
 *   per 16-group: s = E4M3_rne_saturating((amax_group / 6) / g);
 *   code = E2M1_rne_saturating(W / (E4M3(s) * g)), sign kept, ties to even
 *   (a group whose E4M3(s) * g is 0 gets magnitude-0 codes with the sign bit
 *   of each weight).
 * d_w: fp32 [E][N][K] row-major.  out->E/N/K must equal E/N/K; out's buffers
 * are written (out->global_scale is also used as scratch during the call).
 * Results are bit-identical to the reference definition above for finite
 * input; non-finite masters give unspecified (but memory-safe) output.
 */
moe_status moe_w4a16_quantize_pack(const float *d_w, int32_t E, int32_t N, int32_t K,
                                   const moe_nvfp4_tensor *out, hipStream_t stream);

/*
 * Test hook: dequantize a whole tensor stack to fp32 [E][N][K] with the same
 * device decode routines the forward uses ((E2M1 * E4M3) * g in fp32).
 */
moe_status moe_w4a16_dequantize(const moe_nvfp4_tensor *t, float *d_w_out, hipStream_t stream);

/*
 * Check a tensor stack before use.  SYNCHRONISES `stream`.  Returns
 * MOE_ERR_NONFINITE if a global scale is NaN/Inf, MOE_ERR_BAD_SCALE if one is
 * <= 0 (the unset-scale fault: "GLM-5.3-Flash on Blackwell", "The model
 * loaded, served an API, and produced garbage"; the static check for a
 * missing weight_scale_2 before load: "GLM-5.3-Flash-NVFP4-h", "Config
 * expectations") or if a group scale byte is an E4M3 NaN (0x7F / 0xFF).
 *   d_flag  a caller-owned device word (4 bytes, 16-byte aligned) that the
 *           call clears and the check kernel sets; its value afterwards is
 *           unspecified.  Must not overlap the tensor.  NULL gives
 *           MOE_ERR_WORKSPACE.  The call allocates nothing.
 */
moe_status moe_w4a16_validate(const moe_nvfp4_tensor *t, void *d_flag, hipStream_t stream);

/* Workspace bytes moe_route_topk needs for T tokens (0 is a valid answer). */
size_t moe_route_workspace_size(int32_t T, int32_t E, int32_t k);

/*
 * Router top-k + softmax, and the expert-sorted permutation.  The pages keep
 * every router in BF16 and never quantize it ("GLM-5.3-Flash on Blackwell",
 * "The quantization"; "GLM-5.3-Flash-NVFP4-h", "Config expectations", the
 * ignore list) but print no scoring rule.  Reading taken: the k largest
 * logits, ties to the lower expert index, then a softmax over the k selected
 * logits (equal to a softmax over all E renormalised over the k); no bias
 * correction, grouped top-k or routed scaling factor.
 *   d_logits       fp32 [T][E] router logits (finite)
 *   d_topk_ids     int32 [T][k] out: per token, experts by descending logit,
 *                  ties to the lower index
 *   d_topk_w       fp32 [T][k] out: softmax over the k selected logits
 *   d_counts       int32 [E]   out: (token, slot) pairs per expert
 *   d_offsets      int32 [E+1] out: exclusive prefix sum, d_offsets[E] = T*k
 *   d_sorted_slots int32 [T*k] out: flat slot indices t*k+j grouped by expert,
 *                  ascending flat index inside each expert (stable)
 *   d_slot_pos     int32 [T*k] out: inverse of d_sorted_slots
 *   d_ws           workspace of moe_route_workspace_size(T, E, k) bytes
 * Deterministic: identical inputs give identical bits.  T == 0 is a no-op.
 */
moe_status moe_route_topk(const float *d_logits, int32_t T, int32_t E, int32_t k,
                          int32_t *d_topk_ids, float *d_topk_w,
                          int32_t *d_counts, int32_t *d_offsets,
                          int32_t *d_sorted_slots, int32_t *d_slot_pos,
                          void *d_ws, size_t ws_bytes, hipStream_t stream);

/*
 * Workspace bytes moe_w4a16_forward and moe_w4a16_route_forward need (no
 * initialisation: every call writes what it reads).
 */
size_t moe_w4a16_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k);

/*
 * The routed-expert layer: out = sum_j w[t,j] * SwiGLU-FFN_{ids[t,j]}(x[t]).
 *   d_x     bf16 [T][H] activations (uint16 bit patterns); no activation scale
 *   gate,up NVFP4 stacks with N = I, K = H;  down: N = H, K = I;  all with E
 *   routing arrays exactly as moe_route_topk produces them
 *   d_out   bf16 [T][H] out (must not overlap d_x)
 *   d_ws    workspace of moe_w4a16_workspace_size(T, H, I, E, k) bytes
 * Arithmetic: weights decode exactly to bf16 (E2M1 * E4M3 has at most 6
 * significant bits), products accumulate in fp32, the global scale is
 * applied in fp32 after the K reduction, SwiGLU in fp32, the SwiGLU output is
 * rounded once to bf16, the down projection accumulates in fp32 and the
 * routing-weighted combine runs in fp32 before one rounding to bf16.  Shapes
 * beyond the decode kernels round each expert's down-projection row to bf16
 * before the combine (it goes through memory; half the bytes of fp32).
 * Deterministic: no floating-point atomics.  T == 0 is a no-op.
 */
moe_status moe_w4a16_forward(const uint16_t *d_x, int32_t T, int32_t H, int32_t I,
                             int32_t E, int32_t k,
                             const moe_nvfp4_tensor *gate, const moe_nvfp4_tensor *up,
                             const moe_nvfp4_tensor *down,
                             const int32_t *d_topk_ids, const float *d_topk_w,
                             const int32_t *d_counts, const int32_t *d_offsets,
                             const int32_t *d_sorted_slots, const int32_t *d_slot_pos,
                             uint16_t *d_out, void *d_ws, size_t ws_bytes,
                             hipStream_t stream);

/*
 * Route and layer in one call (the pages treat routing and the expert FFN as
 * one MoE layer): moe_route_topk on d_logits (fp32 [T][E]), storing every
 * routing output exactly as moe_route_topk does, followed by
 * moe_w4a16_forward on that routing.  Decode shapes (1 <= T <= 8, T*k <= 64,
 * H % 1024 == 0, H <= 8192, I % 512 == 0, I <= 2048): with one token the
 * gate/up kernel routes itself (two launches in all), with more tokens a
 * single-workgroup route launch precedes the two decode kernels; other shapes
 * run the route kernels followed by the forward kernels.  Same workspace as
 * moe_w4a16_forward.
 */
moe_status moe_w4a16_route_forward(const float *d_logits, const uint16_t *d_x,
                                   int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                   const moe_nvfp4_tensor *gate, const moe_nvfp4_tensor *up,
                                   const moe_nvfp4_tensor *down,
                                   int32_t *d_topk_ids, float *d_topk_w,
                                   int32_t *d_counts, int32_t *d_offsets,
                                   int32_t *d_sorted_slots, int32_t *d_slot_pos,
                                   uint16_t *d_out, void *d_ws, size_t ws_bytes,
                                   hipStream_t stream);

/*
 * The W4A4 NVFP4 variant: the stock routed experts of the NVIDIA release keep
 * W4A4 NVFP4 -- activations quantized to NVFP4 as well -- with a per-tensor
 * activation scale (input_scale) in the checkpoint ("GLM-5.3-Flash-NVFP4-h --
 * W4A16 dense-side quantization", its opening; "GLM-5.3-Flash · 512k + MTP +
 * vision ...", "Input-scales provenance").  The pages print no formula; the
 * reading taken: an activation row is quantized exactly like a weight row --
 * per 16-group s = E4M3((amax / 6) / input_scale), code =
 * E2M1(v / (E4M3(s) * input_scale)), correctly rounded fp32 steps -- with a
 * static FP32 input scale for the gate/up input x and one for the down input
 * h (h quantized from its fp32 value).  A missing scale read as 0 zeroes every
 * expert output ("GLM-5.3-Flash on Blackwell", "The model loaded, served an
 * API, and produced garbage"), so every call below refuses an input scale
 * that is not finite (MOE_ERR_NONFINITE) or not > 0 (MOE_ERR_BAD_SCALE)
 * before anything else, even with T == 0.
 *
 * moe_nvfp4_quantize_activations: bf16 activations [T][K] (K % 32 == 0) ->
 *   d_codes u8 [T][K/2] (byte i = code(2i) | code(2i+1) << 4) and d_scales u8
 *   [T][K/16] (E4M3 bytes), bit-identical to the definition above.  The
 *   three buffers must not overlap.  Asynchronous; allocates nothing.
 *
 * moe_w4a4_forward: as moe_w4a16_forward (same routing arrays, same output,
 *   same shape rules) with x and h passed through that quantization: the
 *   matrix units see the exact values E2M1 * E4M3 of both operands (exact in
 *   bf16) and the input scale multiplies the weight's global scale in each
 *   epilogue; products accumulate in fp32.  d_ws of moe_w4a4_workspace_size
 *   bytes (no initialisation).  Deterministic; graph-capturable.
 *
 * moe_w4a4_route_forward: moe_route_topk on d_logits (fp32 [T][E]) and
 *   moe_w4a4_forward in one call, as moe_w4a16_route_forward is for the
 *   W4A16 layer: the routing outputs are stored exactly as moe_route_topk
 *   stores them and the output is exactly moe_w4a4_forward's on them; with one
 *   token the gate/up kernel routes itself (no route launch).  Same workspace
 *   and errors as moe_w4a4_forward, plus MOE_ERR_INVALID_ARG for a null
 *   d_logits.
 */
moe_status moe_nvfp4_quantize_activations(const uint16_t *d_x, int32_t T, int32_t K, float input_scale,
                                          uint8_t *d_codes, uint8_t *d_scales, hipStream_t stream);
size_t moe_w4a4_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k);
moe_status moe_w4a4_forward(const uint16_t *d_x, int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                            const moe_nvfp4_tensor *gate, const moe_nvfp4_tensor *up,
                            const moe_nvfp4_tensor *down, float input_scale_x, float input_scale_h,
                            const int32_t *d_topk_ids, const float *d_topk_w,
                            const int32_t *d_counts, const int32_t *d_offsets,
                            const int32_t *d_sorted_slots, const int32_t *d_slot_pos,
                            uint16_t *d_out, void *d_ws, size_t ws_bytes, hipStream_t stream);
moe_status moe_w4a4_route_forward(const float *d_logits, const uint16_t *d_x, int32_t T, int32_t H, int32_t I,
                                  int32_t E, int32_t k, const moe_nvfp4_tensor *gate,
                                  const moe_nvfp4_tensor *up, const moe_nvfp4_tensor *down,
                                  float input_scale_x, float input_scale_h, int32_t *d_topk_ids,
                                  float *d_topk_w, int32_t *d_counts, int32_t *d_offsets,
                                  int32_t *d_sorted_slots, int32_t *d_slot_pos, uint16_t *d_out,
                                  void *d_ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_w4a16_route_forward for callers that cannot allocate -- code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation: the
 * same call, kernels and results, without a workspace argument.  Its
 * workspace is a device array owned by the library, MOE_NOALLOC_SCRATCH_BYTES
 * on every GPU the library runs on, held until the process ends; its device
 * address is looked up (hipGetSymbolAddress) on the first call on each
 * device.  The call allocates and frees nothing.  Shapes whose workspace
 * (moe_w4a16_workspace_size) exceeds MOE_NOALLOC_SCRATCH_BYTES are refused
 * with MOE_ERR_WORKSPACE: every decode shape fits, and prefill up to about
 * 2500 (token, expert) pairs at hidden 5120 / intermediate 1536.  The array
 * keeps the last call's contents and nothing in it needs to start at zero.
 * All calls on one GPU share the array: calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race and
 * give undefined results; order them on one stream.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_w4a16_route_forward_noalloc(const float *d_logits, const uint16_t *d_x,
                                           int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                           const moe_nvfp4_tensor *gate, const moe_nvfp4_tensor *up,
                                           const moe_nvfp4_tensor *down,
                                           int32_t *d_topk_ids, float *d_topk_w,
                                           int32_t *d_counts, int32_t *d_offsets,
                                           int32_t *d_sorted_slots, int32_t *d_slot_pos,
                                           uint16_t *d_out, hipStream_t stream);

/*
 * Router logits, the step in front of moe_route_topk: the BF16 gate of the
 * layer, logits[t][e] = sum_i x[t][i] * Wr[e][i], accumulated in fp32 (the
 * routers stay BF16 and are never quantized: "GLM-5.3-Flash on Blackwell",
 * "The quantization"; the pages print no router formula, the plain linear
 * gate without bias is the reading taken).
 *   d_x       bf16 [T][H] activations (caller-owned, read only)
 *   d_wr      bf16 [E][H] router weight, row e = expert e (read only)
 *   d_logits  fp32 [T][E] out, ready for moe_route_topk /
 *             moe_w4a16_route_forward; must not overlap d_x or d_wr
 *   H % 64 == 0, E >= 1, T >= 0 (T == 0 is a no-op); all pointers 16-byte
 *   aligned.  1-8 tokens run a one-pass GEMV over Wr, more tokens bf16 MFMA
 *   tiles; both sum in a fixed order (deterministic), no workspace, no
 *   allocation, graph-capturable.
 */
moe_status moe_router_logits(const uint16_t *d_x, int32_t T, int32_t H,
                             const uint16_t *d_wr, int32_t E, float *d_logits,
                             hipStream_t stream);

/*
 * The router GEMM and the route in one call: moe_router_logits followed by
 * moe_route_topk, with identical outputs (the logits too), for the BF16 gate
 * in front of the top-k (routers stay BF16: "GLM-5.3-Flash on Blackwell",
 * "The quantization"; the scoring rule is moe_route_topk's reading).  For
 * decode token counts (1-8 tokens, T * k <= 64) it is ONE launch: every
 * workgroup computes its expert's logits and takes a ticket, and the
 * workgroup that takes the last one routes all tokens; other shapes run the
 * router kernels and then the route kernels.
 *   arguments as moe_router_logits (d_x, T, H, d_wr, E, d_logits) and
 *   moe_route_topk (k and the six routing outputs)
 *   d_ws   moe_router_route_workspace_size(T, E, k) bytes.  Its first 4 bytes
 *          are the ticket counter: they must be ZERO before the first call on
 *          a workspace (allocate it zero-filled), and every call leaves them
 *          zero.  Calls that share a workspace must be ordered on one stream.
 * Deterministic; graph-capturable (no memset, no allocation).
 */
size_t moe_router_route_workspace_size(int32_t T, int32_t E, int32_t k);
moe_status moe_router_route_topk(const uint16_t *d_x, int32_t T, int32_t H, const uint16_t *d_wr,
                                 int32_t E, int32_t k, float *d_logits,
                                 int32_t *d_topk_ids, float *d_topk_w,
                                 int32_t *d_counts, int32_t *d_offsets,
                                 int32_t *d_sorted_slots, int32_t *d_slot_pos,
                                 void *d_ws, size_t ws_bytes, hipStream_t stream);

/*
 * Dense NVFP4 weight-only projection of T tokens: out = bf16(g * x . Wd^T),
 * Wd the dequantized [N][K] weight (E2M1 code * E4M3 group scale), g its
 * FP32 global scale, products accumulated in fp32 and rounded once (the dense
 * linears -- attention projections, shared experts, lm_head -- quantized to
 * W4A16 NVFP4 like the routed experts: "GLM-5.3-Flash-NVFP4-h -- W4A16
 * dense-side quantization", its opening).
 *   d_x    bf16 [T][K];  w  an NVFP4 tensor with E = 1, N rows, K columns
 *   d_out  bf16 [T][N] (must not overlap d_x or the workspace)
 *   d_ws   workspace of moe_w4a16_linear_workspace_size(T, K, N) bytes
 * Shapes: 1-8 tokens with K % 1024 == 0, K <= 8192 stream the weights once
 * (the decode gate/up kernel with one stack); otherwise N % 256 == 0 and
 * K % 128 == 0 (the grouped down GEMM with one expert, then the combine).
 * MOE_ERR_SHAPE for other shapes.  T == 0 is a no-op.
 */
size_t moe_w4a16_linear_workspace_size(int32_t T, int32_t K, int32_t N);
moe_status moe_w4a16_linear(const uint16_t *d_x, int32_t T, int32_t K, int32_t N,
                            const moe_nvfp4_tensor *w, uint16_t *d_out,
                            void *d_ws, size_t ws_bytes, hipStream_t stream);

/*
 * The shared expert: one always-on SwiGLU FFN applied to every token,
 * out = bf16( g_d * h . Dd^T ), h = bf16( silu(g_g * x . Gd^T) * (g_u * x . Ud^T) )
 * -- moe_w4a16_forward with E = 1, k = 1 and routing weight 1, with the same
 * arithmetic (the model's single shared expert runs for every token beside
 * the routed experts: "GLM-5.3-Flash on Blackwell", "The model loaded, served
 * an API, and produced garbage"; quantized as in "GLM-5.3-Flash-NVFP4-h --
 * W4A16 dense-side quantization"; the caller adds the two outputs).
 *   gate, up  NVFP4 with E = 1, N = I, K = H;  down  E = 1, N = H, K = I
 *   same shape rules as moe_w4a16_forward; d_ws of
 *   moe_w4a16_shared_expert_workspace_size(T, H, I) bytes (no initialization
 *   needed).  T == 0 is a no-op.  With 1-8 tokens the decode kernels run in a
 *   one-expert mode that reads no routing arrays (two launches); with more,
 *   an identity routing is written to d_ws first and the prefill kernels run.
 */
size_t moe_w4a16_shared_expert_workspace_size(int32_t T, int32_t H, int32_t I);
moe_status moe_w4a16_shared_expert(const uint16_t *d_x, int32_t T, int32_t H, int32_t I,
                                   const moe_nvfp4_tensor *gate, const moe_nvfp4_tensor *up,
                                   const moe_nvfp4_tensor *down, uint16_t *d_out,
                                   void *d_ws, size_t ws_bytes, hipStream_t stream);

/*
 * Benchmarking and test hook: which grouped-GEMM kernels run the shapes the
 * decode kernels do not take.  0: operands staged through registers, one
 * K stage in flight, for both products; 1: operands streamed to LDS by DMA
 * through a four-stage ring (128 x 512 output tiles), for both products;
 * 2 (default): the LDS-streamed kernels when the mean rows per touched
 * expert (T * k / min(E, T * k)) is at least 256, the register-staged
 * kernels otherwise.  All give results within the forward's
 * tolerance of each other; each is deterministic.  Shapes the LDS-streamed
 * kernel does not cover (H % 512 or I % 256 nonzero) use 0.  Process-wide,
 * stored atomically; a call made afterwards on any thread uses the new
 * value.  Returns MOE_ERR_INVALID_ARG for other values.
 */
moe_status moe_debug_set_prefill_variant(int32_t variant);

/*
 * A plain streaming read of `bytes` bytes from d_src, for benchmarks: the
 * rate at which a kernel that only reads (16-byte non-temporal loads, all of
 * a thread's loads issued before any is used, as in the decode kernels)
 * streams a buffer of that size on this GPU -- the achievable reference that
 * bench.py reports beside the spec HBM peak.  Not part of the layer.  d_src:
 * device, 16-byte aligned, `bytes` a multiple of 16; d_sink: one device
 * uint32 that the kernel writes only if its reduction of the data equals a
 * fixed magic value (it exists so that the loads are kept).  bytes == 0 is a
 * no-op.  Errors: MOE_ERR_INVALID_ARG (null pointer), MOE_ERR_SHAPE (bytes
 * not a multiple of 16), MOE_ERR_ALIGN, MOE_ERR_HIP.  Asynchronous on
 * `stream`; allocates nothing.
 */
moe_status moe_bench_stream_read(const void *d_src, size_t bytes, uint32_t *d_sink, hipStream_t stream);

/*
 * Per-kernel timing for benchmarks.  moe_profile_begin(n) makes the calls that
 * follow (on any stream) launch each kernel with a pair of HIP timing events
 * that the launch stamps with the kernel's own start and end
 * (hipExtLaunchKernel), for up to n kernels; do not profile while a stream is
 * being captured.  moe_profile_end() synchronises on the events and writes, for each
 * distinct kernel name (up to `max`), its launch count and total milliseconds.
 * Returns the number of names written.  The switch is process-wide: launches
 * on every thread are timed while it is on.  Call begin and end from one
 * thread; for benchmarks only.
 */
moe_status moe_profile_begin(int32_t max_launches);
int32_t moe_profile_end(char (*names)[64], int32_t *counts, double *total_ms, int32_t max);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H */
