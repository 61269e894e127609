// Router top-k + softmax and the expert-sorted permutation (hot path).
//
// The pages say every MoE layer has a BF16 router that is never quantized
// ("GLM-5.3-Flash on Blackwell", "The quantization"); they do not print the
// scoring rule.  Taken here: per token, the k largest fp32 logits (ties to
// the lower expert index) in descending order, and a softmax over those k.
//
// The permutation is a stable counting sort of the flat slots t*k+j by
// expert: a per-expert histogram, an exclusive scan, and a scatter whose
// in-expert order is the flat order.  Atomics only ever count (LDS
// histograms); positions come from ballots and prefix sums, so the result is
// deterministic.
//
//   decode T (T * k <= 64, T <= 16; one workgroup):  k_route_tiny   (1 launch)
//   small T (T <= 64, one workgroup):  k_route_small       (1 launch)
//   large T:  k_route_topk_hist -> k_route_colscan -> k_route_scatter
#include <float.h>
#include <limits.h>

#include "device_common.h"
#include "internal.h"
#include "route_common.h"

namespace moe {
namespace {

constexpr int kRT = 256;                 // threads per route workgroup
constexpr int kRW = kRT / kWave;         // waves per route workgroup
constexpr int kSmallMaxTokens = 64;      // one-workgroup path: T <= 64
constexpr int kSmallMaxSlots = kSmallMaxTokens * MOE_MAX_TOPK;
// Large-T path: a workgroup of 16 waves selects the top-k of 16 tokens, one
// token per wave, so the logits loads of a launch are all in flight at once
// (with 64 tokens per 4-wave workgroup each wave loaded and routed 16 tokens
// one after the other: 41 us at 1K tokens on MI355X).
constexpr int kTokensPerBlock = 16;
constexpr int kHistThreads = kTokensPerBlock * kWave;

// One wave: top-k of one token's E logits (wave_topk_select) written to
// ids/weights, and to LDS when ids_lds is given.
template <int EPL>
__device__ void wave_topk(const float* __restrict__ row, int E, int k, int32_t* __restrict__ ids_out,
                          float* __restrict__ w_out, int32_t* ids_lds) {
    const int lane = threadIdx.x & (kWave - 1);
    int id;
    float w;
    wave_topk_select<EPL>(row, E, k, id, w);
    if (lane < k) {
        ids_out[lane] = id;
        w_out[lane] = w;
        if (ids_lds) ids_lds[lane] = id;
    }
}

template <int EPL>
__device__ void topk_tokens(const float* logits, int t0, int t1, int E, int k, int32_t* ids, float* w,
                            int32_t* ids_lds /* indexed by (t - t0) * k, or null */) {
    const int wave = threadIdx.x / kWave;
    for (int t = t0 + wave; t < t1; t += kRW)
        wave_topk<EPL>(logits + (int64_t)t * E, E, k, ids + (int64_t)t * k, w + (int64_t)t * k,
                       ids_lds ? ids_lds + (t - t0) * k : nullptr);
}

// Top-k for tokens [t0, t1), dispatched on the number of logits per lane.
__device__ void topk_tokens_any(const float* logits, int t0, int t1, int E, int k, int32_t* ids, float* w,
                                int32_t* ids_lds) {
    if (E <= 64) topk_tokens<1>(logits, t0, t1, E, k, ids, w, ids_lds);
    else if (E <= 128) topk_tokens<2>(logits, t0, t1, E, k, ids, w, ids_lds);
    else if (E <= 256) topk_tokens<4>(logits, t0, t1, E, k, ids, w, ids_lds);
    else if (E <= 512) topk_tokens<8>(logits, t0, t1, E, k, ids, w, ids_lds);
    else topk_tokens<16>(logits, t0, t1, E, k, ids, w, ids_lds);
}

// Stable scatter of the flat slots [f0, f1) given the first free position of
// each expert for this block (base[e], LDS).  Each wave takes a contiguous
// run of slots; per-wave histograms give each wave its own starting
// positions, and inside a wave a slot's rank among equal experts comes from
// ballots on the expert id bits ("match any").
__device__ void block_scatter(const int32_t* ids, int f0, int f1, const int* base, int E,
                              int* hist /* [kRW][E] LDS */, int32_t* sorted_slots, int32_t* slot_pos) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int n = f1 - f0;
    const int per_wave = ((n + kRW - 1) / kRW + kWave - 1) / kWave * kWave;
    const int w0 = f0 + wave * per_wave;
    const int w1 = min(f1, w0 + per_wave);
    for (int i = threadIdx.x; i < kRW * E; i += kRT) hist[i] = 0;
    __syncthreads();
    for (int i = w0 + lane; i < w1; i += kWave) atomicAdd(&hist[wave * E + ids[i]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kRT) {
        int run = base[e];
        for (int w = 0; w < kRW; ++w) {
            const int c = hist[w * E + e];
            hist[w * E + e] = run;
            run += c;
        }
    }
    __syncthreads();
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
    int* my_hist = hist + wave * E;
    for (int c0 = w0; c0 < w1; c0 += kWave) {
        const int i = c0 + lane;
        const bool valid = i < w1;
        const int e = valid ? ids[i] : 0;
        int same = 0;
        const int rank = wave_rank_equal(e, valid, nbits, &same);
        int pos = 0;
        if (valid) pos = my_hist[e] + rank;
        __builtin_amdgcn_wave_barrier();
        if (valid && rank == 0) my_hist[e] += same;
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            sorted_slots[pos] = i;
            slot_pos[i] = pos;
        }
    }
}

// Whole route in one workgroup (T <= kSmallMaxTokens).
__global__ void __launch_bounds__(kRT) k_route_small(const float* __restrict__ logits, int T, int E, int k,
                                                     int32_t* __restrict__ ids, float* __restrict__ w,
                                                     int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ sorted_slots, int32_t* __restrict__ slot_pos) {
    __shared__ int32_t s_ids[kSmallMaxSlots];
    __shared__ int s_cnt[MOE_MAX_EXPERTS];
    __shared__ int s_off[MOE_MAX_EXPERTS + 1];
    __shared__ int s_hist[kRW * MOE_MAX_EXPERTS];
    topk_tokens_any(logits, 0, T, E, k, ids, w, s_ids);
    for (int e = threadIdx.x; e < E; e += kRT) s_cnt[e] = 0;
    __syncthreads();
    const int n = T * k;
    for (int i = threadIdx.x; i < n; i += kRT) atomicAdd(&s_cnt[s_ids[i]], 1);
    __syncthreads();
    block_exclusive_scan(s_cnt, s_off, E);
    for (int e = threadIdx.x; e < E; e += kRT) counts[e] = s_cnt[e];
    for (int e = threadIdx.x; e <= E; e += kRT) offsets[e] = s_off[e];
    block_scatter(s_ids, 0, n, s_off, E, s_hist, sorted_slots, slot_pos);
}

// Decode-sized route (T * k <= 64 slots, T <= 16 tokens): one wave per token
// selects its top-k, then one wave orders all the slots at once by ballots on
// the expert bits (wave_slot_order: the same order as the counting sort),
// and every thread fills the per-expert counts and offsets of its experts by
// a binary search over the touched experts (ascending).
constexpr int kTinyMaxSlots = 64, kTinyMaxTokens = 16;

template <int EPL>
__global__ void __launch_bounds__(kTinyMaxTokens * kWave)
k_route_tiny(const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids,
             float* __restrict__ w, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
             int32_t* __restrict__ sorted_slots, int32_t* __restrict__ slot_pos) {
    __shared__ int s_ids[kTinyMaxSlots];
    __shared__ int s_key[kTinyMaxTokens][MOE_MAX_TOPK], s_idx[kTinyMaxTokens][MOE_MAX_TOPK];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (wave < T) {
        int id;
        float v;
        wave_topk_ordered<EPL>(logits + (int64_t)wave * E, E, k, s_key[wave], s_idx[wave], id, v);
        const float wt = topk_softmax(v, k);
        if (lane < k) {
            ids[wave * k + lane] = id;
            w[wave * k + lane] = wt;
            s_ids[wave * k + lane] = id;
        }
    }
    __syncthreads();
    tiny_route_finish(s_ids, T, E, k, counts, offsets, sorted_slots, slot_pos);
}

// Large T, step 1: top-k per token (one wave each: wave_topk_ordered, the
// threshold selection ranked in wave_topk_ids' order) and a per-workgroup
// expert histogram.
template <int EPL>
__global__ void __launch_bounds__(kHistThreads) k_route_topk_hist(const float* __restrict__ logits, int T, int E,
                                                                  int k, int32_t* __restrict__ ids,
                                                                  float* __restrict__ w,
                                                                  int32_t* __restrict__ block_hist /* [B][E] */) {
    __shared__ int s_key[kTokensPerBlock][MOE_MAX_TOPK], s_idx[kTokensPerBlock][MOE_MAX_TOPK];
    __shared__ int s_cnt[MOE_MAX_EXPERTS];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int t = blockIdx.x * kTokensPerBlock + wave;
    for (int e = threadIdx.x; e < E; e += kHistThreads) s_cnt[e] = 0;
    __syncthreads();
    if (t < T) {
        int id;
        float v;
        wave_topk_ordered<EPL>(logits + (int64_t)t * E, E, k, s_key[wave], s_idx[wave], id, v);
        const float wt = topk_softmax(v, k);
        if (lane < k) {
            ids[(int64_t)t * k + lane] = id;
            w[(int64_t)t * k + lane] = wt;
            atomicAdd(&s_cnt[id], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kHistThreads) block_hist[(int64_t)blockIdx.x * E + e] = s_cnt[e];
}

// Large T, step 2: one wave per expert column: exclusive prefix over the
// workgroups (in place) and the expert's total count.  Lane l owns the
// contiguous run of workgroups [l * per, (l + 1) * per): its loads are
// independent of each other (all in flight at once), one DPP scan combines
// the lane sums, and a second pass over the run (L2 hits) writes it.
__global__ void __launch_bounds__(kRT) k_route_colscan(int32_t* __restrict__ block_hist, int B, int E,
                                                       int32_t* __restrict__ counts) {
    const int lane = threadIdx.x & (kWave - 1);
    const int e = blockIdx.x * kRW + threadIdx.x / kWave;
    if (e >= E) return;
    constexpr int kBatch = 16;                 // loads issued together
    const int per = (B + kWave - 1) / kWave;
    const int b0 = lane * per, b1 = min(B, b0 + per);
    int local = 0;
    for (int c = b0; c < b1; c += kBatch) {
        int v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) v[i] = c + i < b1 ? block_hist[(int64_t)(c + i) * E + e] : 0;
#pragma unroll
        for (int i = 0; i < kBatch; ++i) local += v[i];
    }
    const int incl = wave_inclusive_scan_dpp(local);
    int run = incl - local;
    for (int c = b0; c < b1; c += kBatch) {
        int v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) v[i] = c + i < b1 ? block_hist[(int64_t)(c + i) * E + e] : 0;
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            if (c + i < b1) block_hist[(int64_t)(c + i) * E + e] = run;
            run += v[i];
        }
    }
    if (lane == kWave - 1) counts[e] = incl;
}

// Large T, step 3: offsets (every workgroup recomputes them; workgroup 0
// stores them) and the stable scatter of this workgroup's slots.
__global__ void __launch_bounds__(kRT) k_route_scatter(const int32_t* __restrict__ ids, int T, int E, int k,
                                                       const int32_t* __restrict__ counts,
                                                       const int32_t* __restrict__ block_prefix,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ sorted_slots, int32_t* __restrict__ slot_pos) {
    __shared__ int s_cnt[MOE_MAX_EXPERTS];
    __shared__ int s_off[MOE_MAX_EXPERTS + 1];
    __shared__ int s_hist[kRW * MOE_MAX_EXPERTS];
    for (int e = threadIdx.x; e < E; e += kRT) s_cnt[e] = counts[e];
    __syncthreads();
    block_exclusive_scan(s_cnt, s_off, E);
    if (blockIdx.x == 0)
        for (int e = threadIdx.x; e <= E; e += kRT) offsets[e] = s_off[e];
    for (int e = threadIdx.x; e < E; e += kRT) s_off[e] += block_prefix[(int64_t)blockIdx.x * E + e];
    __syncthreads();
    const int t0 = blockIdx.x * kTokensPerBlock;
    const int t1 = min(T, t0 + kTokensPerBlock);
    block_scatter(ids, t0 * k, t1 * k, s_off, E, s_hist, sorted_slots, slot_pos);
}

// The routing of a single always-on expert (E = 1, k = 1, weight 1): every
// token's one slot goes to expert 0 and the sorted order is the token order.
__global__ void __launch_bounds__(256) k_route_identity(int T, int32_t* __restrict__ ids, float* __restrict__ w,
                                                        int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ sorted_slots,
                                                        int32_t* __restrict__ slot_pos) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < T) {
        ids[i] = 0;
        w[i] = 1.0f;
        sorted_slots[i] = i;
        slot_pos[i] = i;
    }
    if (i == 0) {
        counts[0] = T;
        offsets[0] = 0;
        offsets[1] = T;
    }
}

}  // namespace

size_t route_workspace_bytes(int T, int E, int k) {
    (void)k;
    if (T <= kSmallMaxTokens) return 0;
    const int64_t B = (T + kTokensPerBlock - 1) / kTokensPerBlock;
    return (size_t)(B * E * sizeof(int32_t));
}

moe_status launch_route_identity(int T, int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                                 int32_t* sorted_slots, int32_t* slot_pos, hipStream_t s) {
    MOE_LAUNCH("route_identity", k_route_identity, dim3((std::max(T, 1) + 255) / 256), dim3(256), 0, s, T, ids, w,
               counts, offsets, sorted_slots, slot_pos);
    return MOE_OK;
}

moe_status launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_slots, int32_t* slot_pos, void* ws, hipStream_t s) {
    if (T <= kTinyMaxTokens && T * k <= kTinyMaxSlots) {
        const dim3 block(kWave * std::max(T, 4));
        if (E <= 64) MOE_LAUNCH("route_tiny", k_route_tiny<1>, dim3(1), block, 0, s, logits, T, E, k, ids, w, counts,
                                offsets, sorted_slots, slot_pos);
        else if (E <= 128) MOE_LAUNCH("route_tiny", k_route_tiny<2>, dim3(1), block, 0, s, logits, T, E, k, ids, w,
                                      counts, offsets, sorted_slots, slot_pos);
        else if (E <= 256) MOE_LAUNCH("route_tiny", k_route_tiny<4>, dim3(1), block, 0, s, logits, T, E, k, ids, w,
                                      counts, offsets, sorted_slots, slot_pos);
        else if (E <= 512) MOE_LAUNCH("route_tiny", k_route_tiny<8>, dim3(1), block, 0, s, logits, T, E, k, ids, w,
                                      counts, offsets, sorted_slots, slot_pos);
        else MOE_LAUNCH("route_tiny", k_route_tiny<16>, dim3(1), block, 0, s, logits, T, E, k, ids, w, counts, offsets,
                        sorted_slots, slot_pos);
        return MOE_OK;
    }
    if (T <= kSmallMaxTokens) {
        MOE_LAUNCH("route_small", k_route_small, dim3(1), dim3(kRT), 0, s, logits, T, E, k, ids, w, counts,
                   offsets, sorted_slots, slot_pos);
        return MOE_OK;
    }
    const int B = (T + kTokensPerBlock - 1) / kTokensPerBlock;
    int32_t* hist = reinterpret_cast<int32_t*>(ws);
    const dim3 hg(B), hb(kHistThreads);
    if (E <= 64) MOE_LAUNCH("route_topk_hist", k_route_topk_hist<1>, hg, hb, 0, s, logits, T, E, k, ids, w, hist);
    else if (E <= 128) MOE_LAUNCH("route_topk_hist", k_route_topk_hist<2>, hg, hb, 0, s, logits, T, E, k, ids, w, hist);
    else if (E <= 256) MOE_LAUNCH("route_topk_hist", k_route_topk_hist<4>, hg, hb, 0, s, logits, T, E, k, ids, w, hist);
    else if (E <= 512) MOE_LAUNCH("route_topk_hist", k_route_topk_hist<8>, hg, hb, 0, s, logits, T, E, k, ids, w, hist);
    else MOE_LAUNCH("route_topk_hist", k_route_topk_hist<16>, hg, hb, 0, s, logits, T, E, k, ids, w, hist);
    MOE_LAUNCH("route_colscan", k_route_colscan, dim3((E + kRW - 1) / kRW), dim3(kRT), 0, s, hist, B, E, counts);
    MOE_LAUNCH("route_scatter", k_route_scatter, dim3(B), dim3(kRT), 0, s, (const int32_t*)ids, T, E, k,
               (const int32_t*)counts, (const int32_t*)hist, offsets, sorted_slots, slot_pos);
    return MOE_OK;
}

}  // namespace moe
