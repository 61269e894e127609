// Decode-shape forward (1-8 tokens) in one persistent launch.
//
// With a few tokens the layer is a handful of matrix-vector products per
// touched expert and its time is the HBM read of the packed weights (the
// pages' memory-bandwidth wall: "GLM-5.3-Flash on Blackwell", "Two
// deployments, and the lever that reverses between them").  The W4A16 route
// dequantises weights to bf16 and never reads an activation scale ("GLM-5.3-
// Flash on Blackwell", "The model loaded, served an API, and produced
// garbage").  One launch per layer keeps every CU streaming instead of
// draining between dependent kernels.
//
// k_dec_fused runs one workgroup of kNW waves per CU, in three phases:
//   1. routing.  Every workgroup routes the T tokens itself: one wave per
//      token picks the top-k logits and their softmax weights (or the
//      routing given by the caller is read), and one wave sorts the T*k
//      slots by (expert, flat slot index) with ballots on the expert bits:
//      the stable counting sort of moe_route_topk, the same permutation.
//      The activation rows go to LDS by DMA meanwhile.
//   2. gate/up + SwiGLU.  Work unit = (touched expert, pair of features of
//      I), numbered expert by expert.  Each workgroup takes one contiguous
//      run of units of equal cost (a unit costs its weight read plus one dot
//      product per token of its expert), split evenly over its waves; a wave
//      has the next unit's codes in flight while one is computed.  A unit's
//      gate rows n, n+1 are one contiguous run of H codes, as are its up
//      rows; lane l takes 32-code chunks l + 64 j of both runs, so every load
//      is a 16-byte lane slice of a 1 KiB wave run.  A chunk's codes decode
//      once to exact bf16 pairs and meet every token's activations in
//      v_dot2_f32_bf16; the E4M3 group scale multiplies each 16-term partial
//      sum and the FP32 global scale the row total.  SwiGLU runs on the pair
//      and h (bf16) is staged in LDS; the workgroup stores its run at the end
//      with device-coherent stores, in expert-sorted row order.
//   3. down + combine.  Workgroup b owns a contiguous block of output row
//      pairs of H.  Its items (row pair, touched expert) are dealt evenly to
//      waves 1..kNW-1 (one output row per half-wave); each item's down codes
//      are requested before the wait for h, so they stream while the last
//      gate/up units finish.  An item's partial sums, w_j * g_e *
//      (h_j . D_e[row]) per token, go to LDS, and the workgroup adds them up
//      in ascending expert order in fp32 and writes out once in bf16 (no
//      atomics, fixed order).
//
// Hand-off between phases 2 and 3.  A workgroup that has stored all its h
// values waits for its stores to complete and adds one to a counter in the
// workspace; wave 0, which has no down items and so no loads in flight,
// polls it until it reaches the number of workgroups.  h is then read with
// device-coherent loads.  The wait is bounded: a workgroup whose wait runs
// out (possible only when not every workgroup of the grid is resident at
// once) computes every h value itself, with the same arithmetic and so the
// same bits, and goes on.  The last workgroup to finish resets the counters,
// so a workspace whose sync words start at zero stays usable for every
// later call.
#include "decode_fused_kernel.h"

namespace moe {

namespace {

int g_wait_limit = 1 << 20;               // polls of the hand-off counter before computing h locally

__global__ void k_zero_words(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

int cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

}  // namespace

bool fused_decode_supported(int T, int k, int H, int I) {
    using namespace fused;
    const int G = cu_count();
    const int npw_max = (H / 2 + G - 1) / G;
    return T >= 1 && T <= 8 && T * k <= kMaxSlots && H % 1024 == 0 && H / 1024 <= kMaxCPL && I % 512 == 0 &&
           I / 512 <= 4 && npw_max <= kMaxPairs && (size_t)T * H * sizeof(uint16_t) <= 128 * 1024;
}

moe_status launch_zero_words(uint32_t* p, int n, hipStream_t s) {
    MOE_LAUNCH("zero_words", k_zero_words, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
    return MOE_OK;
}

void set_decode_wait_limit(int polls) { g_wait_limit = polls < 0 ? 0 : polls; }

namespace {

fused::FusedParams make_params(const FwdArgs& a) {
    fused::FusedParams p{};
    p.x = a.x;
    p.T = a.T; p.H = a.H; p.I = a.I; p.E = a.E; p.k = a.k;
    p.ids_in = a.ids; p.w_in = a.topk_w;
    p.gc = a.gate->codes; p.gs = a.gate->scales; p.gg = a.gate->global_scale;
    p.uc = a.up->codes;   p.us = a.up->scales;   p.ug = a.up->global_scale;
    p.dc = a.down->codes; p.ds = a.down->scales; p.dg = a.down->global_scale;
    p.h = a.h;
    p.out = a.out;
    p.wait_limit = g_wait_limit;
    return p;
}

}  // namespace

moe_status launch_decode_fused(const FwdArgs& a, const float* logits, int32_t* ids_out, float* w_out,
                               int32_t* counts_out, int32_t* offsets_out, int32_t* sorted_out, int32_t* pos_out,
                               uint32_t* sync, hipStream_t s) {
    fused::FusedParams p = make_params(a);
    p.logits = logits;
    p.ids_out = ids_out; p.w_out = w_out; p.counts_out = counts_out; p.offsets_out = offsets_out;
    p.sorted_out = sorted_out; p.pos_out = pos_out;
    p.sync = sync;
    return a.T == 1 ? fused::launch_t1_fused(p, cu_count(), s) : fused::launch_t8_fused(p, cu_count(), s);
}

moe_status launch_decode_two(const FwdArgs& a, hipStream_t s) {
    const fused::FusedParams p = make_params(a);
    const int G = cu_count();
    moe_status st = a.T == 1 ? fused::launch_t1_gateup(p, G, s) : fused::launch_t8_gateup(p, G, s);
    if (st != MOE_OK) return st;
    return a.T == 1 ? fused::launch_t1_down(p, G, s) : fused::launch_t8_down(p, G, s);
}

}  // namespace moe
