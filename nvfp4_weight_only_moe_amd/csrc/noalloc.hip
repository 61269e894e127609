// moe_w4a16_route_forward_noalloc: the route + layer call for callers that
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  Its workspace is a library-owned
// device array instead of a caller buffer; everything else is
// moe_w4a16_route_forward, the same kernels on the same arguments.
//
// The array is a file-scope __device__ object, so every GPU the library runs
// on holds its own copy (kNoAllocScratchBytes) from the code object's load
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host that name is only a stand-in): the device address is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and cached.  The forward's workspace needs no initialisation (a
// call writes every word it reads), so nothing is cleared here; calls that
// overlap on one GPU (different streams, or threads) race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace moe {
namespace {

constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up on the
// first call per device).  nullptr when HIP refuses.
void* scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_w4a16_route_forward_noalloc(
    const float* d_logits, const uint16_t* d_x, int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
    const moe_nvfp4_tensor* gate, const moe_nvfp4_tensor* up, const moe_nvfp4_tensor* down, int32_t* d_topk_ids,
    float* d_topk_w, int32_t* d_counts, int32_t* d_offsets, int32_t* d_sorted_slots, int32_t* d_slot_pos,
    uint16_t* d_out, hipStream_t stream) {
    if (T < 0 || H < 1 || I < 1 || E < 1 || k < 1) return MOE_ERR_SHAPE;
    if (T == 0)   // the usual argument checks, no workspace needed
        return moe_w4a16_route_forward(d_logits, d_x, T, H, I, E, k, gate, up, down, d_topk_ids, d_topk_w,
                                       d_counts, d_offsets, d_sorted_slots, d_slot_pos, d_out, nullptr, 0, stream);
    if ((int64_t)T * k > (int64_t)INT32_MAX / 2) return MOE_ERR_SHAPE;
    const size_t need = moe_w4a16_workspace_size(T, H, I, E, k);
    if (need > moe::kNoAllocScratchBytes) return MOE_ERR_WORKSPACE;
    void* ws = moe::scratch_on_current_device();
    if (!ws) return MOE_ERR_HIP;
    return moe_w4a16_route_forward(d_logits, d_x, T, H, I, E, k, gate, up, down, d_topk_ids, d_topk_w, d_counts,
                                   d_offsets, d_sorted_slots, d_slot_pos, d_out, ws, moe::kNoAllocScratchBytes,
                                   stream);
}
