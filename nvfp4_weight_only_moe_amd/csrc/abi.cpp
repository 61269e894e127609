// C ABI of libmoe_w4a16: argument checking, workspace layout and dispatch.
// Every check runs on the host before anything is enqueued, so a refused
// call has no effect on the device.  See include/moe_w4a16.h for the
// contract of each entry point.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace moe {
namespace {

constexpr size_t kAlign = 256;

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_tensor(const moe_nvfp4_tensor* t, int E, int N, int K) {
    if (!t || !t->codes || !t->scales || !t->global_scale) return MOE_ERR_INVALID_ARG;
    if (t->E != E || t->N != N || t->K != K) return MOE_ERR_SHAPE;
    if (!aligned16(t->codes) || !aligned16(t->scales) || !aligned16(t->global_scale)) return MOE_ERR_ALIGN;
    return MOE_OK;
}

moe_status check_tensor_self(const moe_nvfp4_tensor* t) {
    if (!t) return MOE_ERR_INVALID_ARG;
    if (t->E < 1 || t->N < 1 || t->K < 32 || t->K % 32) return MOE_ERR_SHAPE;
    if (t->E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
    return check_tensor(t, t->E, t->N, t->K);
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// ---- profiling state (benchmarks only)
struct ProfRec {
    std::string name;
    hipEvent_t start, stop;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};   // read without the mutex by every launch
int g_prof_max = 0;
std::vector<ProfRec> g_prof;

}  // namespace

bool prof_events(const char* name, hipEvent_t* start, hipEvent_t* stop) {
    if (!g_prof_on.load(std::memory_order_relaxed)) return false;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if ((int)g_prof.size() >= g_prof_max) return false;
    ProfRec r{name, nullptr, nullptr};
    if (hipEventCreate(&r.start) != hipSuccess) return false;
    if (hipEventCreate(&r.stop) != hipSuccess) {
        (void)hipEventDestroy(r.start);
        return false;
    }
    g_prof.push_back(r);
    *start = r.start;
    *stop = r.stop;
    return true;
}

moe_status allow_dynamic_lds(const void* kernel, size_t bytes) {
    static std::mutex mu;
    static std::vector<std::pair<const void*, size_t>> done;
    std::lock_guard<std::mutex> lk(mu);
    for (auto& d : done)
        if (d.first == kernel && d.second >= bytes) return MOE_OK;
    if (bytes > 64 * 1024 &&
        hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) != hipSuccess)
        return MOE_ERR_HIP;
    done.emplace_back(kernel, bytes);
    return MOE_OK;
}

// Forward workspace: [h (bf16 [T*k][I]) | y (bf16 [T*k][H]) | route scratch].
size_t forward_workspace_bytes(int T, int H, int I, int E, int k) {
    const size_t slots = (size_t)T * k;
    return round_up(slots * I * sizeof(uint16_t), kAlign) + round_up(slots * H * sizeof(uint16_t), kAlign) +
           round_up(route_workspace_bytes(T, E, k), kAlign);
}

struct WsLayout {
    uint16_t* h;
    uint16_t* y;
    void* route;
};

WsLayout ws_layout(void* d_ws, int T, int H, int I, int k) {
    uint8_t* ws = static_cast<uint8_t*>(d_ws);
    const size_t slots = (size_t)T * k;
    const size_t hb = round_up(slots * I * sizeof(uint16_t), kAlign);
    const size_t yb = round_up(slots * H * sizeof(uint16_t), kAlign);
    return WsLayout{reinterpret_cast<uint16_t*>(ws), reinterpret_cast<uint16_t*>(ws + hb), ws + hb + yb};
}

// Grouped-GEMM kernels for larger T: 0 = register-staged (k_grouped_gemm)
// for both products, 1 = LDS-pipelined (k_gemm_pipe) for both, 2 = chosen
// from the mean rows per touched expert (the default).  The pipelined
// kernel's 128-row tiles pay off once experts hold a few hundred rows (16K
// tokens, top-8 of 256 on MI355X: gate/up 4.6 ms against 7.3, down 2.5 ms
// against 4.1); with few rows per expert (1K tokens: about 32) its padding
// costs more than it saves.  Chosen by moe_debug_set_prefill_variant; a
// forward reads it once, atomically, when it is called.
std::atomic<int> g_prefill_variant{2};
constexpr int64_t kPipeMinRowsPerExpert = 256;

bool use_pipe(const FwdArgs& a);

moe_status launch_prefill(const FwdArgs& a, hipStream_t stream) {
    const bool pipe = use_pipe(a);
    moe_status st = pipe ? launch_gateup_pipe(a, stream) : launch_gateup_grouped(a, stream);
    if (st != MOE_OK) return st;
    st = pipe ? launch_down_pipe(a, stream) : launch_down_grouped(a, stream);
    if (st != MOE_OK) return st;
    return launch_combine(a, stream);
}

moe_status launch_decode_forward(const FwdArgs& a, hipStream_t stream) {
    if (decode_path_supported(a.T, a.k, a.H, a.I)) return launch_forward_decode(a, stream);
    return launch_prefill(a, stream);
}

// Checks shared by moe_w4a16_forward and moe_w4a16_route_forward.
moe_status check_forward(const uint16_t* d_x, int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                         const moe_nvfp4_tensor* gate, const moe_nvfp4_tensor* up, const moe_nvfp4_tensor* down,
                         const void* const* ptrs, int nptrs, const uint16_t* d_out, void* d_ws, size_t ws_bytes,
                         size_t need_override = 0) {
    if (T < 0 || E < 1 || k < 1 || H < 1 || I < 1) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || k > E) return MOE_ERR_UNSUPPORTED;
    if (H % 256 || I % 128) return MOE_ERR_SHAPE;
    if ((int64_t)T * k > (int64_t)INT32_MAX / 2) return MOE_ERR_SHAPE;
    if (!gate || !up || !down) return MOE_ERR_INVALID_ARG;
    moe_status st;
    if ((st = check_tensor(gate, E, I, H)) != MOE_OK) return st;
    if ((st = check_tensor(up, E, I, H)) != MOE_OK) return st;
    if ((st = check_tensor(down, E, H, I)) != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    for (int i = 0; i < nptrs; ++i) {
        if (!ptrs[i]) return MOE_ERR_INVALID_ARG;
        if (!aligned16(ptrs[i])) return MOE_ERR_ALIGN;
    }
    if (!d_x || !d_out) return MOE_ERR_INVALID_ARG;
    if (!aligned16(d_x) || !aligned16(d_out)) return MOE_ERR_ALIGN;
    if (!d_ws) return MOE_ERR_WORKSPACE;
    if (!aligned16(d_ws)) return MOE_ERR_ALIGN;
    const size_t xbytes = (size_t)T * H * sizeof(uint16_t);
    if (ranges_overlap(d_x, xbytes, d_out, xbytes)) return MOE_ERR_INVALID_ARG;
    const size_t need = need_override ? need_override : forward_workspace_bytes(T, H, I, E, k);
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (ranges_overlap(d_ws, need, d_out, xbytes) || ranges_overlap(d_ws, need, d_x, xbytes))
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

FwdArgs make_args(const uint16_t* d_x, int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                  const moe_nvfp4_tensor* gate, const moe_nvfp4_tensor* up, const moe_nvfp4_tensor* down,
                  const int32_t* ids, const float* w, const int32_t* counts, const int32_t* offsets,
                  const int32_t* sorted, const int32_t* pos, uint16_t* d_out, const WsLayout& L) {
    FwdArgs a{};
    a.x = d_x;
    a.T = T; a.H = H; a.I = I; a.E = E; a.k = k;
    a.gate = gate; a.up = up; a.down = down;
    a.ids = ids;
    a.topk_w = w;
    a.counts = counts;
    a.offsets = offsets;
    a.sorted_slots = sorted;
    a.slot_pos = pos;
    a.out = d_out;
    a.h = L.h;
    a.y = L.y;
    return a;
}

// Single-expert entry points (dense linear, shared expert): the workspace
// starts with the identity routing of T tokens (ids, weights, sorted slots
// and slot positions: T each; counts and offsets: 1 and 2), then what the
// chosen path needs.
struct IdRoute {
    int32_t* ids;
    float* w;
    int32_t* counts;
    int32_t* offsets;
    int32_t* sorted;
    int32_t* pos;
    uint8_t* rest;
};

size_t id_route_bytes(int T) { return 4 * round_up((size_t)T * 4, kAlign) + kAlign; }

IdRoute id_route_layout(void* d_ws, int T) {
    uint8_t* p = static_cast<uint8_t*>(d_ws);
    const size_t tb = round_up((size_t)T * 4, kAlign);
    IdRoute r;
    r.ids = reinterpret_cast<int32_t*>(p);
    r.w = reinterpret_cast<float*>(p + tb);
    r.sorted = reinterpret_cast<int32_t*>(p + 2 * tb);
    r.pos = reinterpret_cast<int32_t*>(p + 3 * tb);
    r.counts = reinterpret_cast<int32_t*>(p + 4 * tb);
    r.offsets = r.counts + 4;
    r.rest = p + 4 * tb + kAlign;
    return r;
}

size_t linear_workspace_bytes(int T, int K, int N) {
    (void)K;
    return id_route_bytes(T) + round_up((size_t)T * N * sizeof(uint16_t), kAlign);
}

size_t shared_workspace_bytes(int T, int H, int I) { return id_route_bytes(T) + forward_workspace_bytes(T, H, I, 1, 1); }

// W4A4 forward workspace: [x as NVFP4 values (bf16 [T][H]) | SwiGLU output
// (fp32 [T*k][I]) | the W4A16 forward workspace (h as NVFP4 values, y, ...)].
size_t w4a4_workspace_bytes(int T, int H, int I, int E, int k) {
    const size_t slots = (size_t)T * k;
    return round_up((size_t)T * H * sizeof(uint16_t), kAlign) + round_up(slots * I * sizeof(float), kAlign) +
           forward_workspace_bytes(T, H, I, E, k);
}

// A static input scale must be a finite number > 0: a missing scale read as
// 0.0 multiplies every expert output by zero ("GLM-5.3-Flash on Blackwell",
// "The model loaded, served an API, and produced garbage").
moe_status check_input_scale(float s) {
    if (!std::isfinite(s)) return MOE_ERR_NONFINITE;
    if (!(s > 0.0f)) return MOE_ERR_BAD_SCALE;
    return MOE_OK;
}

bool use_pipe(const FwdArgs& a) {
    const int64_t slots = (int64_t)a.T * a.k;
    const int64_t per_expert = slots / std::max<int64_t>(1, std::min<int64_t>(a.E, slots));
    const int variant = g_prefill_variant.load(std::memory_order_relaxed);
    return prefill_pipe_supported(a.T, a.k, a.H, a.I) &&
           (variant == 1 || (variant == 2 && per_expert >= kPipeMinRowsPerExpert));
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(moe_status st) {
    switch (st) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: null pointer, aliasing or bad argument";
        case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: dimension out of range or not a required multiple";
        case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: device pointer not 16-byte aligned";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: E or k beyond the compiled limits";
        case MOE_ERR_NONFINITE: return "MOE_ERR_NONFINITE: a global scale is NaN or infinite";
        case MOE_ERR_BAD_SCALE: return "MOE_ERR_BAD_SCALE: a global scale is <= 0 or a group scale is an E4M3 NaN";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP runtime call failed";
        default: return "MOE_ERR_UNKNOWN";
    }
}

int32_t moe_w4a16_version(void) { return 100; }

moe_status moe_w4a16_quantize_pack(const float* d_w, int32_t E, int32_t N, int32_t K, const moe_nvfp4_tensor* out,
                                   hipStream_t stream) {
    if (!d_w || !out) return MOE_ERR_INVALID_ARG;
    if (E < 1 || N < 1 || K < 32 || K % 32) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
    moe_status st = check_tensor(out, E, N, K);
    if (st != MOE_OK) return st;
    if (!aligned16(d_w)) return MOE_ERR_ALIGN;
    const size_t wbytes = (size_t)E * N * K * sizeof(float);
    if (ranges_overlap(d_w, wbytes, out->codes, (size_t)E * N * K / 2) ||
        ranges_overlap(d_w, wbytes, out->scales, (size_t)E * N * K / 16) ||
        ranges_overlap(d_w, wbytes, out->global_scale, (size_t)E * sizeof(float)))
        return MOE_ERR_INVALID_ARG;
    return launch_quantize_pack(d_w, E, N, K, out, stream);
}

moe_status moe_w4a16_dequantize(const moe_nvfp4_tensor* t, float* d_w_out, hipStream_t stream) {
    moe_status st = check_tensor_self(t);
    if (st != MOE_OK) return st;
    if (!d_w_out) return MOE_ERR_INVALID_ARG;
    if (!aligned16(d_w_out)) return MOE_ERR_ALIGN;
    return launch_dequantize(t, d_w_out, stream);
}

moe_status moe_w4a16_validate(const moe_nvfp4_tensor* t, void* d_flag, hipStream_t stream) {
    moe_status st = check_tensor_self(t);
    if (st != MOE_OK) return st;
    if (!d_flag) return MOE_ERR_WORKSPACE;
    if (!aligned16(d_flag)) return MOE_ERR_ALIGN;
    uint32_t* flag_d = static_cast<uint32_t*>(d_flag);
    if (ranges_overlap(d_flag, sizeof(uint32_t), t->codes, (size_t)t->E * t->N * t->K / 2) ||
        ranges_overlap(d_flag, sizeof(uint32_t), t->scales, (size_t)t->E * t->N * t->K / 16) ||
        ranges_overlap(d_flag, sizeof(uint32_t), t->global_scale, (size_t)t->E * sizeof(float)))
        return MOE_ERR_INVALID_ARG;
    st = launch_zero_words(flag_d, 1, stream);
    if (st == MOE_OK) st = launch_validate(t, flag_d, stream);
    uint32_t flag = 0;
    if (st == MOE_OK && hipMemcpyAsync(&flag, flag_d, sizeof(flag), hipMemcpyDeviceToHost, stream) != hipSuccess)
        st = MOE_ERR_HIP;
    if (st == MOE_OK && hipStreamSynchronize(stream) != hipSuccess) st = MOE_ERR_HIP;
    if (st != MOE_OK) return st;
    if (flag & 1u) return MOE_ERR_NONFINITE;
    if (flag & 6u) return MOE_ERR_BAD_SCALE;
    return MOE_OK;
}

size_t moe_route_workspace_size(int32_t T, int32_t E, int32_t k) {
    if (T <= 0 || E < 1 || k < 1) return 0;
    return route_workspace_bytes(T, E, k);
}

moe_status moe_route_topk(const float* d_logits, int32_t T, int32_t E, int32_t k, int32_t* d_topk_ids,
                          float* d_topk_w, int32_t* d_counts, int32_t* d_offsets, int32_t* d_sorted_slots,
                          int32_t* d_slot_pos, void* d_ws, size_t ws_bytes, hipStream_t stream) {
    if (T < 0 || E < 1 || k < 1) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || k > E) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)T * k > (int64_t)INT32_MAX / 2) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    const void* ptrs[] = {d_logits, d_topk_ids, d_topk_w, d_counts, d_offsets, d_sorted_slots, d_slot_pos};
    for (const void* p : ptrs) {
        if (!p) return MOE_ERR_INVALID_ARG;
        if (!aligned16(p)) return MOE_ERR_ALIGN;
    }
    const size_t need = route_workspace_bytes(T, E, k);
    if (need > 0) {
        if (!d_ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
        if (!aligned16(d_ws)) return MOE_ERR_ALIGN;
    }
    return launch_route(d_logits, T, E, k, d_topk_ids, d_topk_w, d_counts, d_offsets, d_sorted_slots, d_slot_pos,
                        d_ws, stream);
}

size_t moe_w4a16_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k) {
    if (T <= 0 || H <= 0 || I <= 0 || k <= 0) return 0;
    return forward_workspace_bytes(T, H, I, E, k);
}

moe_status moe_w4a16_forward(const uint16_t* d_x, int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                             const moe_nvfp4_tensor* gate, const moe_nvfp4_tensor* up, const moe_nvfp4_tensor* down,
                             const int32_t* d_topk_ids, const float* d_topk_w, const int32_t* d_counts,
                             const int32_t* d_offsets, const int32_t* d_sorted_slots, const int32_t* d_slot_pos,
                             uint16_t* d_out, void* d_ws, size_t ws_bytes, hipStream_t stream) {
    const void* ptrs[] = {d_topk_ids, d_topk_w, d_counts, d_offsets, d_sorted_slots, d_slot_pos};
    moe_status st = check_forward(d_x, T, H, I, E, k, gate, up, down, ptrs, 6, d_out, d_ws, ws_bytes);
    if (st != MOE_OK || T == 0) return st;
    const WsLayout L = ws_layout(d_ws, T, H, I, k);
    const FwdArgs a = make_args(d_x, T, H, I, E, k, gate, up, down, d_topk_ids, d_topk_w, d_counts, d_offsets,
                                d_sorted_slots, d_slot_pos, d_out, L);
    return launch_decode_forward(a, stream);
}

moe_status moe_w4a16_route_forward(const float* d_logits, const uint16_t* d_x, int32_t T, int32_t H, int32_t I,
                                   int32_t E, int32_t k, const moe_nvfp4_tensor* gate, const moe_nvfp4_tensor* up,
                                   const moe_nvfp4_tensor* down, int32_t* d_topk_ids, float* d_topk_w,
                                   int32_t* d_counts, int32_t* d_offsets, int32_t* d_sorted_slots,
                                   int32_t* d_slot_pos, uint16_t* d_out, void* d_ws, size_t ws_bytes,
                                   hipStream_t stream) {
    const void* ptrs[] = {d_logits, d_topk_ids, d_topk_w, d_counts, d_offsets, d_sorted_slots, d_slot_pos};
    moe_status st = check_forward(d_x, T, H, I, E, k, gate, up, down, ptrs, 7, d_out, d_ws, ws_bytes);
    if (st != MOE_OK || T == 0) return st;
    const WsLayout L = ws_layout(d_ws, T, H, I, k);
    const FwdArgs a = make_args(d_x, T, H, I, E, k, gate, up, down, d_topk_ids, d_topk_w, d_counts, d_offsets,
                                d_sorted_slots, d_slot_pos, d_out, L);
    if (T == 1 && decode_path_supported(T, k, H, I))
        return launch_forward_decode_routed(a, d_logits, d_topk_ids, d_topk_w, d_counts, d_offsets, d_sorted_slots,
                                            d_slot_pos, stream);
    st = launch_route(d_logits, T, E, k, d_topk_ids, d_topk_w, d_counts, d_offsets, d_sorted_slots, d_slot_pos,
                      L.route, stream);
    if (st != MOE_OK) return st;
    return launch_decode_forward(a, stream);
}

size_t moe_w4a4_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k) {
    if (T <= 0 || H <= 0 || I <= 0 || k <= 0) return 0;
    return w4a4_workspace_bytes(T, H, I, E, k);
}

moe_status moe_nvfp4_quantize_activations(const uint16_t* d_x, int32_t T, int32_t K, float input_scale,
                                          uint8_t* d_codes, uint8_t* d_scales, hipStream_t stream) {
    moe_status st = check_input_scale(input_scale);
    if (st != MOE_OK) return st;
    if (T < 0 || K < 32 || K % 32) return MOE_ERR_SHAPE;
    if ((int64_t)T * K > (int64_t)INT32_MAX * 16) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!d_x || !d_codes || !d_scales) return MOE_ERR_INVALID_ARG;
    if (!aligned16(d_x) || !aligned16(d_codes) || !aligned16(d_scales)) return MOE_ERR_ALIGN;
    const size_t xb = (size_t)T * K * 2, cb = (size_t)T * K / 2, sb = (size_t)T * K / 16;
    if (ranges_overlap(d_x, xb, d_codes, cb) || ranges_overlap(d_x, xb, d_scales, sb) ||
        ranges_overlap(d_codes, cb, d_scales, sb))
        return MOE_ERR_INVALID_ARG;
    return launch_quant_act(d_x, false, T, K, input_scale, d_codes, d_scales, nullptr, stream);
}

namespace {

// The W4A4 layer after the argument checks: x -> NVFP4 values; gate/up +
// SwiGLU in fp32; h -> NVFP4 values; down.  With one token the decode gate/up
// kernel quantizes its own groups of h (and, given R, routes itself).
moe_status w4a4_run(const uint16_t* d_x, int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                    const moe_nvfp4_tensor* gate, const moe_nvfp4_tensor* up, const moe_nvfp4_tensor* down,
                    float input_scale_x, float input_scale_h, const float* d_logits, int32_t* d_topk_ids,
                    float* d_topk_w, int32_t* d_counts, int32_t* d_offsets, int32_t* d_sorted_slots,
                    int32_t* d_slot_pos, uint16_t* d_out, void* d_ws, hipStream_t stream) {
    uint8_t* ws = static_cast<uint8_t*>(d_ws);
    const size_t slots = (size_t)T * k;
    uint16_t* xq = reinterpret_cast<uint16_t*>(ws);
    float* hf = reinterpret_cast<float*>(ws + round_up((size_t)T * H * sizeof(uint16_t), kAlign));
    void* fws = ws + round_up((size_t)T * H * sizeof(uint16_t), kAlign) + round_up(slots * I * sizeof(float), kAlign);
    const WsLayout L = ws_layout(fws, T, H, I, k);
    FwdArgs a = make_args(xq, T, H, I, E, k, gate, up, down, d_topk_ids, d_topk_w, d_counts, d_offsets,
                          d_sorted_slots, d_slot_pos, d_out, L);
    a.xs = input_scale_x;
    a.hs = input_scale_h;
    a.hf = hf;
    const bool decode = decode_path_supported(T, k, H, I);
    moe_status st;
    if (d_logits && !(decode && T == 1)) {
        st = launch_route(d_logits, T, E, k, d_topk_ids, d_topk_w, d_counts, d_offsets, d_sorted_slots, d_slot_pos,
                          L.route, stream);
        if (st != MOE_OK) return st;
    }
    if ((st = launch_quant_act(d_x, false, T, H, input_scale_x, nullptr, nullptr, xq, stream)) != MOE_OK) return st;
    if (decode && T == 1) {
        a.hf = nullptr;
        a.hq = input_scale_h;
        st = d_logits ? launch_forward_decode_gateup_routed(a, d_logits, d_topk_ids, d_topk_w, d_counts, d_offsets,
                                                            d_sorted_slots, d_slot_pos, stream)
                      : launch_forward_decode_gateup(a, stream);
        if (st != MOE_OK) return st;
        return launch_forward_decode_down(a, stream);
    }
    const bool pipe = !decode && use_pipe(a);
    st = decode ? launch_forward_decode_gateup(a, stream)
                : (pipe ? launch_gateup_pipe(a, stream) : launch_gateup_grouped(a, stream));
    if (st != MOE_OK) return st;
    if ((st = launch_quant_act(hf, true, (int64_t)slots, I, input_scale_h, nullptr, nullptr, L.h, stream)) != MOE_OK)
        return st;
    if (decode) return launch_forward_decode_down(a, stream);
    st = pipe ? launch_down_pipe(a, stream) : launch_down_grouped(a, stream);
    if (st != MOE_OK) return st;
    return launch_combine(a, stream);
}

}  // namespace

moe_status moe_w4a4_forward(const uint16_t* d_x, int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                            const moe_nvfp4_tensor* gate, const moe_nvfp4_tensor* up, const moe_nvfp4_tensor* down,
                            float input_scale_x, float input_scale_h, const int32_t* d_topk_ids,
                            const float* d_topk_w, const int32_t* d_counts, const int32_t* d_offsets,
                            const int32_t* d_sorted_slots, const int32_t* d_slot_pos, uint16_t* d_out, void* d_ws,
                            size_t ws_bytes, hipStream_t stream) {
    moe_status st = check_input_scale(input_scale_x);
    if (st != MOE_OK) return st;
    if ((st = check_input_scale(input_scale_h)) != MOE_OK) return st;
    const void* ptrs[] = {d_topk_ids, d_topk_w, d_counts, d_offsets, d_sorted_slots, d_slot_pos};
    const size_t need = T > 0 && k > 0 && H > 0 && I > 0 ? w4a4_workspace_bytes(T, H, I, E, k) : 0;
    st = check_forward(d_x, T, H, I, E, k, gate, up, down, ptrs, 6, d_out, d_ws, ws_bytes, need);
    if (st != MOE_OK || T == 0) return st;
    return w4a4_run(d_x, T, H, I, E, k, gate, up, down, input_scale_x, input_scale_h, nullptr,
                    const_cast<int32_t*>(d_topk_ids), const_cast<float*>(d_topk_w), const_cast<int32_t*>(d_counts),
                    const_cast<int32_t*>(d_offsets), const_cast<int32_t*>(d_sorted_slots),
                    const_cast<int32_t*>(d_slot_pos), d_out, d_ws, stream);
}

moe_status moe_w4a4_route_forward(const float* d_logits, const uint16_t* d_x, int32_t T, int32_t H, int32_t I,
                                  int32_t E, int32_t k, const moe_nvfp4_tensor* gate, const moe_nvfp4_tensor* up,
                                  const moe_nvfp4_tensor* down, float input_scale_x, float input_scale_h,
                                  int32_t* d_topk_ids, float* d_topk_w, int32_t* d_counts, int32_t* d_offsets,
                                  int32_t* d_sorted_slots, int32_t* d_slot_pos, uint16_t* d_out, void* d_ws,
                                  size_t ws_bytes, hipStream_t stream) {
    moe_status st = check_input_scale(input_scale_x);
    if (st != MOE_OK) return st;
    if ((st = check_input_scale(input_scale_h)) != MOE_OK) return st;
    const void* ptrs[] = {d_logits, d_topk_ids, d_topk_w, d_counts, d_offsets, d_sorted_slots, d_slot_pos};
    const size_t need = T > 0 && k > 0 && H > 0 && I > 0 ? w4a4_workspace_bytes(T, H, I, E, k) : 0;
    st = check_forward(d_x, T, H, I, E, k, gate, up, down, ptrs, 7, d_out, d_ws, ws_bytes, need);
    if (st != MOE_OK || T == 0) return st;
    return w4a4_run(d_x, T, H, I, E, k, gate, up, down, input_scale_x, input_scale_h, d_logits, d_topk_ids,
                    d_topk_w, d_counts, d_offsets, d_sorted_slots, d_slot_pos, d_out, d_ws, stream);
}

moe_status moe_router_logits(const uint16_t* d_x, int32_t T, int32_t H, const uint16_t* d_wr, int32_t E,
                             float* d_logits, hipStream_t stream) {
    if (T < 0 || H < 1 || E < 1 || !router_shape_supported(T, H, E)) return MOE_ERR_SHAPE;
    if ((int64_t)T * H > (int64_t)INT32_MAX || (int64_t)E * H > (int64_t)INT32_MAX ||
        (int64_t)T * E > (int64_t)INT32_MAX)
        return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!d_x || !d_wr || !d_logits) return MOE_ERR_INVALID_ARG;
    if (!aligned16(d_x) || !aligned16(d_wr) || !aligned16(d_logits)) return MOE_ERR_ALIGN;
    const size_t lb = (size_t)T * E * sizeof(float);
    if (ranges_overlap(d_logits, lb, d_x, (size_t)T * H * 2) || ranges_overlap(d_logits, lb, d_wr, (size_t)E * H * 2))
        return MOE_ERR_INVALID_ARG;
    return launch_router_logits(d_x, T, H, d_wr, E, d_logits, stream);
}

// Router + route workspace: [ticket word (zero between calls) | padding to
// 256 B | route scratch of the unfused path].
constexpr size_t kTicketBytes = 256;

size_t moe_router_route_workspace_size(int32_t T, int32_t E, int32_t k) {
    if (T <= 0 || E < 1 || k < 1) return kTicketBytes;
    return kTicketBytes + round_up(route_workspace_bytes(T, E, k), kAlign);
}

moe_status moe_router_route_topk(const uint16_t* d_x, int32_t T, int32_t H, const uint16_t* d_wr, int32_t E,
                                 int32_t k, float* d_logits, int32_t* d_topk_ids, float* d_topk_w,
                                 int32_t* d_counts, int32_t* d_offsets, int32_t* d_sorted_slots,
                                 int32_t* d_slot_pos, void* d_ws, size_t ws_bytes, hipStream_t stream) {
    if (T < 0 || H < 1 || E < 1 || k < 1 || !router_shape_supported(T, H, E)) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || k > E) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)T * H > (int64_t)INT32_MAX || (int64_t)E * H > (int64_t)INT32_MAX ||
        (int64_t)T * E > (int64_t)INT32_MAX || (int64_t)T * k > (int64_t)INT32_MAX / 2)
        return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    const void* ptrs[] = {d_x, d_wr, d_logits, d_topk_ids, d_topk_w, d_counts, d_offsets, d_sorted_slots,
                          d_slot_pos};
    for (const void* p : ptrs) {
        if (!p) return MOE_ERR_INVALID_ARG;
        if (!aligned16(p)) return MOE_ERR_ALIGN;
    }
    if (!d_ws) return MOE_ERR_WORKSPACE;
    if (!aligned16(d_ws)) return MOE_ERR_ALIGN;
    const size_t need = moe_router_route_workspace_size(T, E, k);
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    const size_t lb = (size_t)T * E * sizeof(float);
    if (ranges_overlap(d_logits, lb, d_x, (size_t)T * H * 2) || ranges_overlap(d_logits, lb, d_wr, (size_t)E * H * 2) ||
        ranges_overlap(d_ws, need, d_logits, lb))
        return MOE_ERR_INVALID_ARG;
    uint32_t* ticket = static_cast<uint32_t*>(d_ws);
    if (router_route_fused_supported(T, H, E, k))
        return launch_router_route(d_x, T, H, d_wr, E, k, d_logits, ticket, d_topk_ids, d_topk_w, d_counts,
                                   d_offsets, d_sorted_slots, d_slot_pos, stream);
    moe_status st = launch_router_logits(d_x, T, H, d_wr, E, d_logits, stream);
    if (st != MOE_OK) return st;
    return launch_route(d_logits, T, E, k, d_topk_ids, d_topk_w, d_counts, d_offsets, d_sorted_slots, d_slot_pos,
                        static_cast<uint8_t*>(d_ws) + kTicketBytes, stream);
}

size_t moe_w4a16_linear_workspace_size(int32_t T, int32_t K, int32_t N) {
    if (T <= 0 || K <= 0 || N <= 0) return 0;
    return linear_workspace_bytes(T, K, N);
}

moe_status moe_w4a16_linear(const uint16_t* d_x, int32_t T, int32_t K, int32_t N, const moe_nvfp4_tensor* w,
                            uint16_t* d_out, void* d_ws, size_t ws_bytes, hipStream_t stream) {
    if (T < 0 || K < 1 || N < 1) return MOE_ERR_SHAPE;
    if ((int64_t)T * N > (int64_t)INT32_MAX / 2 || (int64_t)T * K > (int64_t)INT32_MAX / 2) return MOE_ERR_SHAPE;
    if (!w) return MOE_ERR_INVALID_ARG;
    moe_status st = check_tensor(w, 1, N, K);
    if (st != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    const bool decode = linear_decode_supported(T, K, N);
    if (!decode && (N % 256 || K % 128)) return MOE_ERR_SHAPE;   // grouped-GEMM tiles
    if (!d_x || !d_out) return MOE_ERR_INVALID_ARG;
    if (!aligned16(d_x) || !aligned16(d_out)) return MOE_ERR_ALIGN;
    if (!d_ws) return MOE_ERR_WORKSPACE;
    if (!aligned16(d_ws)) return MOE_ERR_ALIGN;
    const size_t need = linear_workspace_bytes(T, K, N);
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    const size_t xb = (size_t)T * K * sizeof(uint16_t), ob = (size_t)T * N * sizeof(uint16_t);
    if (ranges_overlap(d_x, xb, d_out, ob) || ranges_overlap(d_ws, need, d_out, ob) ||
        ranges_overlap(d_ws, need, d_x, xb))
        return MOE_ERR_INVALID_ARG;
    const IdRoute R = id_route_layout(d_ws, T);
    FwdArgs a{};
    a.T = T; a.E = 1; a.k = 1;
    a.gate = a.up = a.down = w;
    a.ids = R.ids; a.topk_w = R.w; a.counts = R.counts; a.offsets = R.offsets;
    a.sorted_slots = R.sorted; a.slot_pos = R.pos;
    a.out = d_out;
    if (decode) {
        // the gate/up kernel's streaming with one stack (tokens in order, no
        // routing arrays): K = a.H, N = a.I, out through a.h
        a.x = d_x; a.H = K; a.I = N; a.h = d_out;
        return launch_linear_decode(a, stream);
    }
    st = launch_route_identity(T, R.ids, R.w, R.counts, R.offsets, R.sorted, R.pos, stream);
    if (st != MOE_OK) return st;
    // the down GEMM (x as its A operand, bf16 rows in the workspace) and the
    // combine with one slot of weight 1 (which returns those rows unchanged)
    a.H = N; a.I = K;
    a.h = const_cast<uint16_t*>(d_x);
    a.y = reinterpret_cast<uint16_t*>(R.rest);
    const bool pipe = prefill_pipe_supported(T, 1, N, K) && T >= kPipeMinRowsPerExpert;
    st = pipe ? launch_down_pipe(a, stream) : launch_down_grouped(a, stream);
    if (st != MOE_OK) return st;
    return launch_combine(a, stream);
}

size_t moe_w4a16_shared_expert_workspace_size(int32_t T, int32_t H, int32_t I) {
    if (T <= 0 || H <= 0 || I <= 0) return 0;
    return shared_workspace_bytes(T, H, I);
}

moe_status moe_w4a16_shared_expert(const uint16_t* d_x, int32_t T, int32_t H, int32_t I,
                                   const moe_nvfp4_tensor* gate, const moe_nvfp4_tensor* up,
                                   const moe_nvfp4_tensor* down, uint16_t* d_out, void* d_ws, size_t ws_bytes,
                                   hipStream_t stream) {
    if (T < 0) return MOE_ERR_SHAPE;
    const size_t idb = T > 0 ? id_route_bytes(T) : 0;
    if (T > 0 && d_ws && ws_bytes < idb) return MOE_ERR_WORKSPACE;
    void* fws = d_ws && T > 0 ? static_cast<uint8_t*>(d_ws) + idb : d_ws;
    moe_status st = check_forward(d_x, T, H, I, 1, 1, gate, up, down, nullptr, 0, d_out, fws,
                                  T > 0 && d_ws ? ws_bytes - idb : ws_bytes);
    if (st != MOE_OK || T == 0) return st;
    const size_t xb = (size_t)T * H * sizeof(uint16_t);
    if (ranges_overlap(d_ws, idb, d_x, xb) || ranges_overlap(d_ws, idb, d_out, xb)) return MOE_ERR_INVALID_ARG;
    const IdRoute R = id_route_layout(d_ws, T);
    const WsLayout L = ws_layout(R.rest, T, H, I, 1);
    const FwdArgs a = make_args(d_x, T, H, I, 1, 1, gate, up, down, R.ids, R.w, R.counts, R.offsets, R.sorted,
                                R.pos, d_out, L);
    // decode shapes: the decode kernels in their one-expert mode read no routing arrays
    if (decode_path_supported(T, 1, H, I)) return launch_forward_decode_one(a, stream);
    st = launch_route_identity(T, R.ids, R.w, R.counts, R.offsets, R.sorted, R.pos, stream);
    if (st != MOE_OK) return st;
    return launch_prefill(a, stream);
}

moe_status moe_bench_stream_read(const void* d_src, size_t bytes, uint32_t* d_sink, hipStream_t stream) {
    if (bytes == 0) return MOE_OK;
    if (!d_src || !d_sink) return MOE_ERR_INVALID_ARG;
    if (bytes % 16) return MOE_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(d_src) % 16 || reinterpret_cast<uintptr_t>(d_sink) % 4) return MOE_ERR_ALIGN;
    return launch_stream_read(d_src, bytes, d_sink, stream);
}

moe_status moe_debug_set_prefill_variant(int32_t variant) {
    if (variant < 0 || variant > 2) return MOE_ERR_INVALID_ARG;
    g_prefill_variant.store(variant, std::memory_order_relaxed);
    return MOE_OK;
}

moe_status moe_profile_begin(int32_t max_launches) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (auto& r : g_prof) {
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
    }
    g_prof.clear();
    g_prof.reserve(max_launches > 0 ? max_launches : 0);
    g_prof_max = max_launches > 0 ? max_launches : 0;
    g_prof_on.store(g_prof_max > 0, std::memory_order_relaxed);
    return MOE_OK;
}

int32_t moe_profile_end(char (*names)[64], int32_t* counts, double* total_ms, int32_t max) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on.store(false, std::memory_order_relaxed);
    std::vector<std::string> keys;
    std::vector<int32_t> cnt;
    std::vector<double> ms;
    for (auto& r : g_prof) {
        float t = 0.0f;
        if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess)
            t = -1.0f;
        size_t i = 0;
        while (i < keys.size() && keys[i] != r.name) ++i;
        if (i == keys.size()) {
            keys.push_back(r.name);
            cnt.push_back(0);
            ms.push_back(0.0);
        }
        cnt[i] += 1;
        ms[i] += t;
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
    }
    g_prof.clear();
    const int n = (int)std::min<size_t>(keys.size(), (size_t)std::max(max, 0));
    for (int i = 0; i < n; ++i) {
        if (names) {
            std::strncpy(names[i], keys[i].c_str(), 63);
            names[i][63] = '\0';
        }
        if (counts) counts[i] = cnt[i];
        if (total_ms) total_ms[i] = ms[i];
    }
    return n;
}

}  // extern "C"
