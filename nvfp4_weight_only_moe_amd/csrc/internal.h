// Host-side interface between the C ABI (abi.cpp) and the kernel launchers
// (*.hip).  Not part of the public API.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_w4a16.h"

namespace moe {

// ---- per-kernel timing (moe_profile_begin / moe_profile_end)
// While profiling is on, returns true and a pair of timing events that the
// launch itself stamps with the kernel's start and end (hipExtLaunchKernel),
// so the interval is the kernel's execution, not the gap between markers.
bool prof_events(const char* name, hipEvent_t* start, hipEvent_t* stop);

// Launch helper: timed launch when profiling is on; reports launch errors.
#define MOE_LAUNCH(name, kern, grid, block, shmem, stream, ...)                          \
    do {                                                                                 \
        hipEvent_t moe_ev0_ = nullptr, moe_ev1_ = nullptr;                               \
        if (::moe::prof_events(name, &moe_ev0_, &moe_ev1_))                              \
            hipExtLaunchKernelGGL(kern, grid, block, shmem, stream, moe_ev0_, moe_ev1_, 0, \
                                  __VA_ARGS__);                                          \
        else                                                                             \
            hipLaunchKernelGGL(kern, grid, block, shmem, stream, __VA_ARGS__);           \
        if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;                         \
    } while (0)

// Allow `bytes` of dynamic LDS for `kernel` (HIP needs an explicit opt-in
// above 64 KB).  Cached per kernel; host-side only, never captured.
moe_status allow_dynamic_lds(const void* kernel, size_t bytes);

// ---- quantize.hip
moe_status launch_quantize_pack(const float* w, int E, int N, int K, const moe_nvfp4_tensor* out,
                                hipStream_t s);
moe_status launch_dequantize(const moe_nvfp4_tensor* t, float* w_out, hipStream_t s);
moe_status launch_validate(const moe_nvfp4_tensor* t, uint32_t* d_flag, hipStream_t s);
// W4A4 activations: rows x K (bf16, or fp32 when in_f32) quantized to NVFP4
// with a static input scale; either packed (codes/scales non-null) or the
// unscaled values E2M1 * E4M3 as bf16 into deq
moe_status launch_quant_act(const void* in, bool in_f32, int64_t rows, int K, float input_scale, uint8_t* codes,
                            uint8_t* scales, uint16_t* deq, hipStream_t s);
// n words set to zero by a fill kernel (graph-safe: no memset node)
moe_status launch_zero_words(uint32_t* p, int n, hipStream_t s);

// ---- route.hip
size_t route_workspace_bytes(int T, int E, int k);
moe_status launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_slots,
                        int32_t* slot_pos, void* ws, hipStream_t s);
// ---- router logits (router.hip): logits = x . W^T, bf16 in, fp32 out
bool router_shape_supported(int T, int H, int E);
moe_status launch_router_logits(const uint16_t* x, int T, int H, const uint16_t* w, int E, float* logits,
                                hipStream_t s);
// router logits and the route in one launch (decode token counts: 1-8
// tokens, T * k <= 64); ticket: a device word that is zero on entry and is
// left zero
bool router_route_fused_supported(int T, int H, int E, int k);
moe_status launch_router_route(const uint16_t* x, int T, int H, const uint16_t* w, int E, int k, float* logits,
                               uint32_t* ticket, int32_t* ids, float* wts, int32_t* counts, int32_t* offsets,
                               int32_t* sorted_slots, int32_t* slot_pos, hipStream_t s);
// routing of one always-on expert (E = 1, k = 1, weight 1; sorted order = token order)
moe_status launch_route_identity(int T, int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                                 int32_t* sorted_slots, int32_t* slot_pos, hipStream_t s);

// ---- forward (moe_decode.hip / moe_prefill.hip)
struct FwdArgs {
    const uint16_t* x;
    int T, H, I, E, k;
    const moe_nvfp4_tensor *gate, *up, *down;
    const int32_t* ids;
    const float* topk_w;
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* sorted_slots;
    const int32_t* slot_pos;
    uint16_t* out;
    uint16_t* h;  // workspace: [T*k][I] bf16, expert-sorted rows (the down GEMM's input)
    uint16_t* y;  // workspace: [T*k][H] bf16, expert-sorted rows (prefill only)
    // W4A4: the activations' static input scales multiply the weights' global
    // scales in the epilogues (x: gate/up, h: down; 1 for W4A16), and the
    // gate/up output goes as fp32 to hf (when set) for the NVFP4 quantization
    // of h instead of as bf16 to h
    float xs = 1.0f;
    float hs = 1.0f;
    float* hf = nullptr;
    // W4A4 on the decode path: when > 0, the decode gate/up kernel quantizes
    // its own output groups of h under this input scale (h gets the groups'
    // NVFP4 values as bf16) and no hf round trip is made
    float hq = 0.0f;
};

size_t forward_workspace_bytes(int T, int H, int I, int E, int k);
bool decode_path_supported(int T, int k, int H, int I);
moe_status launch_forward_decode(const FwdArgs& a, hipStream_t s);
// its two halves (gate/up + SwiGLU, down + combine) as separate calls
moe_status launch_forward_decode_gateup(const FwdArgs& a, hipStream_t s);
moe_status launch_forward_decode_down(const FwdArgs& a, hipStream_t s);
// the gate/up half routing a single token itself (stores the routing outputs)
moe_status launch_forward_decode_gateup_routed(const FwdArgs& a, const float* logits, int32_t* ids, float* w,
                                               int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* pos,
                                               hipStream_t s);
// the same kernels for one always-on expert (E = 1, k = 1, weight 1, tokens
// in order): no routing arrays are read
moe_status launch_forward_decode_one(const FwdArgs& a, hipStream_t s);
// the same two kernels with the routing computed by the gate/up kernel from
// the logits (it stores the routing outputs, which the down kernel reads);
// one token only (MOE_ERR_UNSUPPORTED otherwise)
moe_status launch_forward_decode_routed(const FwdArgs& a, const float* logits, int32_t* ids, float* w,
                                        int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* pos,
                                        hipStream_t s);
// a dense projection out = bf16(g * x . W^T) of a few tokens by the gate/up
// kernel's streaming with one weight stack (a.gate, E = 1, tokens in order --
// no routing arrays are read -- K = a.H, N = a.I, out written through a.h)
bool linear_decode_supported(int T, int K, int N);
moe_status launch_linear_decode(const FwdArgs& a, hipStream_t s);

// Plain streaming read of `bytes` (a multiple of 16) for benchmarks (probe.hip).
moe_status launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);
// moe_prefill.hip: register-staged grouped GEMMs and the combine
moe_status launch_gateup_grouped(const FwdArgs& a, hipStream_t s);
moe_status launch_down_grouped(const FwdArgs& a, hipStream_t s);
moe_status launch_combine(const FwdArgs& a, hipStream_t s);
// moe_prefill_pipe.hip: LDS-pipelined grouped GEMMs
bool prefill_pipe_supported(int64_t T, int k, int H, int I);
moe_status launch_gateup_pipe(const FwdArgs& a, hipStream_t s);
moe_status launch_down_pipe(const FwdArgs& a, hipStream_t s);

}  // namespace moe
