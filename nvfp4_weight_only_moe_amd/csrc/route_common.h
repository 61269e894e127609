// Device-side routing pieces shared by the route kernels and the fused
// decode kernel: per-token top-k + softmax in one wave, and the slot rank
// among equal experts.  See route.hip for the scoring rule.
#pragma once

#include <float.h>
#include <limits.h>

#include "device_common.h"

namespace moe {

// Order-preserving unsigned key of a float (no NaN; -0.0 folded into +0.0
// beforehand): larger float, larger key.  topk_key_value inverts it.
__device__ __forceinline__ uint32_t topk_key(float x) {
    const uint32_t u = __float_as_uint(x);
    return u ^ ((u >> 31) ? 0xFFFFFFFFu : 0x80000000u);
}
__device__ __forceinline__ float topk_key_value(uint32_t key) {
    return __uint_as_float(key ^ ((key >> 31) ? 0x80000000u : 0xFFFFFFFFu));
}

// One wave selects the top-k of one token's E logits.  EPL = logits per lane
// (E <= 64 * EPL); lane l holds experts l, l + 64, ...  Each candidate becomes
// one 64-bit key: the order-preserving bits of its logit above the complement
// of its expert index, so that a plain unsigned comparison is the selection
// order (larger logit first, then the lower expert).  Each lane sorts its EPL
// keys (insertion network, best first), so a round only has to find the best
// of the 64 lane heads: one DPP maximum of the logit halves, a ballot for the
// lanes holding it and, when several do (equal logits), a DPP minimum of
// their expert indices; the winning lane then drops its head.  On return
// lane j < k holds the j-th selection (expert in id_out, logit in v_out).
// -0.0 is folded into +0.0 so that the two compare equal; a NaN logit ranks
// as -inf.  A dropped head becomes key 0, below every candidate.
template <int EPL>
__device__ __forceinline__ void wave_topk_ids(const float* __restrict__ row, int E, int k, int& id_out,
                                              float& v_out) {
    const int lane = threadIdx.x & (kWave - 1);
    uint64_t kk[EPL];
    float xs[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) xs[i] = row[min(lane + kWave * i, E - 1)];   // all loads before any use
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int idx = lane + kWave * i;
        const float x = idx < E ? xs[i] + 0.0f : -INFINITY;
        kk[i] = ((uint64_t)topk_key(x != x ? -INFINITY : x) << 32) | (uint32_t)~idx;
    }
#pragma unroll
    for (int a = 1; a < EPL; ++a)
#pragma unroll
        for (int b = a; b > 0; --b) {
            const uint64_t hi = kk[b] > kk[b - 1] ? kk[b] : kk[b - 1];
            const uint64_t lo = kk[b] > kk[b - 1] ? kk[b - 1] : kk[b];
            kk[b - 1] = hi;
            kk[b] = lo;
        }
    float my_v = 0.0f;
    int my_i = 0;
    for (int r = 0; r < k; ++r) {
        const uint32_t head = (uint32_t)(kk[0] >> 32);
        const int head_ix = (int)~(uint32_t)kk[0];
        const uint32_t m = wave_max_u32_dpp(head);
        const uint64_t b = __ballot(head == m);
        int win = __ffsll((unsigned long long)b) - 1;
        if (__popcll(b) > 1) {     // equal logits: the lowest expert index among the heads
            const int mi = wave_min_i32_dpp(head == m ? head_ix : INT_MAX);
            win = __ffsll((unsigned long long)__ballot(head == m && head_ix == mi)) - 1;
        }
        const int sel = __builtin_amdgcn_readlane(head_ix, win);
        if (lane == win) {
#pragma unroll
            for (int i = 0; i + 1 < EPL; ++i) kk[i] = kk[i + 1];
            kk[EPL - 1] = 0u;
        }
        if (lane == r) {
            my_v = topk_key_value(m);
            my_i = sel;
        }
    }
    id_out = my_i;
    v_out = my_v;
}

// The k largest of one token's E logits as a SET, by a threshold search
// instead of k rounds of arg-max: the k-th largest order-preserving key is
// found bit by bit from the top (keep a bit when at least k keys reach the
// prefix with it set; one ballot per candidate slot and bit), stopping as
// soon as exactly k keys reach the prefix; keys equal to the final threshold
// are then taken in ascending expert index until k are taken.  EPL = logits
// per lane (lane l holds experts l, l + 64, ...).  On return key[i] holds the
// key of expert 64 i + lane and bit `lane` of sel[i] says whether it is
// selected; exactly k bits are set, and ascending (i, lane) is ascending
// expert index.  -0.0 is folded into +0.0, a NaN logit ranks as -inf and
// experts past E get key 0, below every real logit (the same order as
// wave_topk_ids).
template <int EPL>
__device__ __forceinline__ void wave_topk_set(const float* __restrict__ row, int E, int k, uint32_t (&key)[EPL],
                                              uint64_t (&sel)[EPL]) {
    const int lane = threadIdx.x & (kWave - 1);
    // every lane loads all its logits before any is used (clamped indices,
    // no branch around a load), so the EPL loads take one memory round trip
    float xs[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) xs[i] = row[min(lane + kWave * i, E - 1)];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int idx = lane + kWave * i;
        const float x = xs[i] + 0.0f;
        key[i] = idx < E ? topk_key(x != x ? -INFINITY : x) : 0u;
    }
    uint32_t P = 0u;                                   // count(key >= P) >= k throughout
    for (int b = 31; b >= 0; --b) {
        const uint32_t T = P | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) cnt += __popcll(__ballot(key[i] >= T));
        if (cnt >= k) {
            P = T;
            if (cnt == k) break;                       // exactly k keys reach P: the set is found
        }
    }
    int need = k;                                      // keys above P are all selected
#pragma unroll
    for (int i = 0; i < EPL; ++i) need -= __popcll(__ballot(key[i] > P));
#pragma unroll
    for (int i = 0; i < EPL; ++i) {                    // then keys equal to P, lowest expert first
        const uint64_t eq = __ballot(key[i] == P);
        const bool take = key[i] > P || (key[i] == P && __popcll(eq & lanemask_lt()) < need);
        sel[i] = __ballot(take);
        need -= __popcll(sel[i] & eq);
    }
}

// The same selection in wave_topk_ids' order (logit descending, ties to the
// lower expert): wave_topk_set, then each of the k selected ranks itself
// against the others through a small per-wave LDS scratch (s_key, s_idx:
// at least k ints each).  On return lane j < k holds the j-th selection
// (expert in id_out, logit in v_out), exactly as wave_topk_ids returns it.
template <int EPL>
__device__ __forceinline__ void wave_topk_ordered(const float* __restrict__ row, int E, int k, int* s_key,
                                                  int* s_idx, int& id_out, float& v_out) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t key[EPL];
    uint64_t sel[EPL];
    wave_topk_set<EPL>(row, E, k, key, sel);
    int base = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        if ((sel[i] >> lane) & 1u) {
            const int c = base + __popcll(sel[i] & lanemask_lt());
            s_key[c] = (int)key[i];
            s_idx[c] = kWave * i + lane;
        }
        base += __popcll(sel[i]);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // this wave's LDS writes land before its reads
    const int j = lane < k ? lane : 0;
    const uint32_t kj = (uint32_t)s_key[j];
    const int ij = s_idx[j];
    int rank = 0;
#pragma unroll
    for (int m = 0; m < MOE_MAX_TOPK; ++m) {       // a static loop: the LDS reads issue back to back
        if (m < k) {
            const uint32_t km = (uint32_t)s_key[m];
            rank += (km > kj || (km == kj && s_idx[m] < ij)) ? 1 : 0;
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // every read above is done before the slots are rewritten
    if (lane < k) {
        s_key[rank] = (int)kj;
        s_idx[rank] = ij;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    id_out = lane < k ? s_idx[lane] : 0;
    v_out = lane < k ? topk_key_value((uint32_t)s_key[lane]) : 0.0f;
}

// Routing weights of a wave_topk_ids selection: softmax over the k selected
// logits (lane j < k holds the j-th), computed from the largest.
__device__ __forceinline__ float topk_softmax(float my_v, int k) {
    const int lane = threadIdx.x & (kWave - 1);
    const float m0 = __shfl(my_v, 0, kWave);
    const float ex = lane < k ? expf(my_v - m0) : 0.0f;
    const float sum = wave_sum_dpp(ex);
    return ex / sum;
}

// Top-k experts and their routing weights (lane j < k: j-th selection).
template <int EPL>
__device__ __forceinline__ void wave_topk_select(const float* __restrict__ row, int E, int k, int& id_out,
                                                 float& w_out) {
    float v;
    wave_topk_ids<EPL>(row, E, k, id_out, v);
    w_out = topk_softmax(v, k);
}

// The order of the slots of a few tokens (one slot per lane, at most 64) by
// (expert, flat slot index) -- the order of moe_route_topk's stable counting
// sort -- from one ballot per expert bit: the lanes still equal so far split
// into smaller and equal.  For a valid lane: pos = its sorted position,
// eq = the lanes with its expert, less = how many slots hold smaller experts
// (its expert's first position), first = the lowest lane of its expert,
// u = its expert's rank among the touched experts; U = touched experts.
struct SlotOrder {
    uint64_t eq;
    int less, pos, u, U;
    bool first;
};
__device__ __forceinline__ SlotOrder wave_slot_order(int ex, bool valid, int E) {
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
    uint64_t eq = __ballot(valid), lessm = 0;
    for (int b = nbits - 1; b >= 0; --b) {
        const bool bit = (ex >> b) & 1;
        const uint64_t B = __ballot(valid && bit);
        if (bit) {
            lessm |= eq & ~B;
            eq &= B;
        } else {
            eq &= ~B;
        }
    }
    SlotOrder o;
    const uint64_t before = eq & lanemask_lt();
    o.eq = eq;
    o.less = __popcll(lessm);
    o.pos = o.less + __popcll(before);
    o.first = valid && before == 0;
    const uint64_t firsts = __ballot(o.first);
    o.u = __popcll(firsts & lessm);
    o.U = __popcll(firsts);
    return o;
}

// Rank of this lane's expert id among the valid lanes below it holding the
// same id ("match any" from one ballot per id bit), and how many valid lanes
// hold it.
__device__ __forceinline__ int wave_rank_equal(int e, bool valid, int nbits, int* total) {
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bal = __ballot(valid && bit);
        match &= bit ? bal : ~bal;
    }
    if (total) *total = __popcll(match);
    return __popcll(match & lanemask_lt());
}

// After the top-k of a few tokens (their ids in s_ids, LDS, all T * k slots):
// one wave orders the slots by ballots on the expert bits (wave_slot_order:
// the order of the counting sort) and stores sorted_slots and slot_pos, then
// every thread fills the counts and offsets of its experts by a binary
// search over the touched experts (ascending).  Called by a whole
// workgroup; contains barriers.
__device__ inline void tiny_route_finish(const int* s_ids, int T, int E, int k, int32_t* __restrict__ counts,
                                  int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots,
                                  int32_t* __restrict__ slot_pos) {
    __shared__ int s_list[64], s_ucnt[64], s_uoff[64];
    __shared__ int s_U;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int slots = T * k;
    if (wave == 0) {
        const bool valid = lane < slots;
        const int ex = valid ? s_ids[lane] : 0;
        const SlotOrder o = wave_slot_order(ex, valid, E);
        if (valid) {
            sorted_slots[o.pos] = lane;
            slot_pos[lane] = o.pos;
        }
        if (o.first) {
            s_list[o.u] = ex;
            s_ucnt[o.u] = __popcll(o.eq);
            s_uoff[o.u] = o.less;
        }
        if (lane == 0) s_U = o.U;
    }
    __syncthreads();
    const int U = s_U;
    for (int e = threadIdx.x; e <= E; e += blockDim.x) {
        int lo = 0, hi = U;                  // first touched expert >= e
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (s_list[mid] < e) lo = mid + 1;
            else hi = mid;
        }
        if (e < E) counts[e] = lo < U && s_list[lo] == e ? s_ucnt[lo] : 0;
        offsets[e] = lo < U ? s_uoff[lo] : slots;
    }
}

}  // namespace moe
