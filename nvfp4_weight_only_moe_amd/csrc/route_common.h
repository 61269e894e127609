// Device-side routing pieces shared by the route kernels and the fused
// decode kernel: per-token top-k + softmax in one wave, and the slot rank
// among equal experts.  See route.hip for the scoring rule.
#pragma once

#include <float.h>

#include "device_common.h"

namespace moe {

// One wave selects the top-k of one token's E logits.  EPL = logits per lane
// (E <= 64 * EPL).  Each round finds the maximum with a DPP reduction, then
// the lowest expert index holding it with one ballot per logit slot (slot i
// covers indices 64i .. 64i+63, so the first slot and lane with a match is the
// lowest index), and retires that logit.  On return lane j < k holds the j-th
// selection and its weight, a softmax over the k selected logits.  -0.0 is
// folded into +0.0 so that the two compare equal.
template <int EPL>
__device__ __forceinline__ void wave_topk_select(const float* __restrict__ row, int E, int k, int& id_out,
                                                 float& w_out) {
    const int lane = threadIdx.x & (kWave - 1);
    float v[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int idx = lane + kWave * i;
        v[i] = idx < E ? row[idx] + 0.0f : -INFINITY;
    }
    float my_v = 0.0f;
    int my_i = 0;
    for (int r = 0; r < k; ++r) {
        float lm = v[0];
#pragma unroll
        for (int i = 1; i < EPL; ++i) lm = fmaxf(lm, v[i]);
        const float m = wave_max_dpp(lm);
        int sel = -1;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const uint64_t b = __ballot(v[i] == m);
            if (sel < 0 && b) sel = kWave * i + __ffsll((unsigned long long)b) - 1;
        }
        if (lane == (sel & (kWave - 1))) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (i == sel / kWave) v[i] = -INFINITY;
        }
        if (lane == r) {
            my_v = m;
            my_i = sel;
        }
    }
    const float m0 = __shfl(my_v, 0, kWave);
    const float ex = lane < k ? expf(my_v - m0) : 0.0f;
    const float sum = wave_sum_dpp(ex);
    id_out = my_i;
    w_out = ex / sum;
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

}  // namespace moe
