// Device code of the single-launch decode path (see moe_decode_fused.hip);
// included by the translation units that instantiate it.
#pragma once

#include "device_common.h"
#include "internal.h"
#include "route_common.h"

#include <algorithm>

namespace moe {
namespace fused {

constexpr int kNW = 8;                    // waves per workgroup
constexpr int kFThreads = kNW * kWave;
constexpr int kMaxSlots = 64;             // T * k on this path
constexpr int kChunkExperts = 8;          // experts per phase-3 chunk (at most)
constexpr int kChunkSlots = 16;           // h rows staged in LDS per chunk (at most)
constexpr int kItemWaves = kNW - 1;       // waves with phase-3 items (wave 0 polls)
constexpr int kMaxItems = 16;             // phase-3 items per wave per chunk
constexpr int kMaxPairs = 16;             // output row pairs per workgroup
constexpr int kStageUnits = 32;           // gate/up units whose h a wave holds in LDS
constexpr int kMemCost = 4;               // a unit's weight read, in one token's dot products
constexpr int kSyncDone = 0, kSyncExit = 1;
// what one launch of k_dec_fused does: all three phases with the in-kernel
// hand-off, or the gate/up phase alone, or the down phase alone (the two
// halves of the layer as separate launches, the kernel boundary in between)
constexpr int kFused = 0, kGateUp = 1, kDown = 2;
constexpr int kMaxCPL = 5;                // H <= 5120 on this path


struct FusedParams {
    const uint16_t* x;
    int T, H, I, E, k;
    const float* logits;                  // non-null: route in the kernel
    int32_t* ids_out;                     // routing outputs (logits != null)
    float* w_out;
    int32_t* counts_out;
    int32_t* offsets_out;
    int32_t* sorted_out;
    int32_t* pos_out;
    const int32_t* ids_in;                // routing given (logits == null)
    const float* w_in;
    const uint8_t *gc, *gs;
    const float* gg;
    const uint8_t *uc, *us;
    const float* ug;
    const uint8_t *dc, *ds;
    const float* dg;
    uint16_t* h;                          // [T*k][I] bf16, expert-sorted rows
    uint32_t* sync;                       // [0] gate/up done count, [1] exit count
    uint16_t* out;
    int wait_limit;
};

__device__ __forceinline__ uint32_t coherent_load(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t counter_add(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Top-k of one token, dispatched on the number of logits per lane.
__device__ inline void topk_select_any(const float* row, int E, int k, int& id, float& w) {
    if (E <= 64) wave_topk_select<1>(row, E, k, id, w);
    else if (E <= 128) wave_topk_select<2>(row, E, k, id, w);
    else if (E <= 256) wave_topk_select<4>(row, E, k, id, w);
    else if (E <= 512) wave_topk_select<8>(row, E, k, id, w);
    else wave_topk_select<16>(row, E, k, id, w);
}

// MAXT: tokens handled per unit (1 for one-token decode, else 8); MODE:
// kFused, kGateUp or kDown.
template <int CPL, int GPL2, int MAXT, int MODE>
__global__ void __launch_bounds__(kFThreads, 1) k_dec_fused(const FusedParams P) {
    constexpr int kItems = GPL2 >= 4 ? 12 : kMaxItems;    // phase-3 items per wave (register budget)
    extern __shared__ uint4 smem[];       // phase 2: x [T][H/8]; phase 3: h rows [kChunkSlots][I/8]
    __shared__ uint32_t s_hst[kNW][kStageUnits][MAXT];    // staged h: bf16 pairs per unit and token
    __shared__ int s_fl_first[kNW], s_fl_n[kNW];           // each wave's staged run
    __shared__ float s_part[kItemWaves][kMaxPairs][2][MAXT];   // per wave and local row pair
    __shared__ int s_ids[kMaxSlots];      // flat slot -> expert
    __shared__ float s_wsel[kMaxSlots];   // flat slot -> routing weight
    __shared__ int s_pos[kMaxSlots];      // flat slot -> sorted row
    __shared__ int s_tok[kMaxSlots];      // sorted row -> token
    __shared__ float s_wrow[kMaxSlots];   // sorted row -> routing weight
    __shared__ int s_list[kMaxSlots];     // touched experts, ascending
    __shared__ int s_ucnt[kMaxSlots];     // their slot counts
    __shared__ int s_uoff[kMaxSlots];     // their first sorted row
    __shared__ int s_U, s_go;

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int T = P.T, H = P.H, I = P.I, E = P.E, k = P.k;
    const int slots = T * k;
    const int H8 = H / 8, I8 = I / 8;
    const int G = gridDim.x;

    // ---- phase 1: routing (logits first: they are on the critical path)
    if (P.logits) {
        if (wave < T) {
            int id;
            float w;
            topk_select_any(P.logits + (int64_t)wave * E, E, k, id, w);
            if (lane < k) {
                s_ids[wave * k + lane] = id;
                s_wsel[wave * k + lane] = w;
            }
        }
    } else if (threadIdx.x < slots) {
        s_ids[threadIdx.x] = P.ids_in[threadIdx.x];
        s_wsel[threadIdx.x] = P.w_in[threadIdx.x];
    }
    if constexpr (MODE != kDown) {   // activation rows to LDS
        const uint4* src = reinterpret_cast<const uint4*>(P.x);
        const int nchunk = T * H / 512;   // 1 KiB runs, H % 1024 == 0
        for (int c = wave; c < nchunk; c += kNW) wave_copy_1k_to_lds(src + c * 64, smem + c * 64);
    }
    wait_all_memory();
    __syncthreads();
    if (wave == 0) {
        // rank of each slot by (expert, flat index): per expert bit from the
        // top, lanes still equal so far split into smaller and equal
        int nbits = 1;
        while ((1 << nbits) < E) ++nbits;
        const bool valid = lane < slots;
        const int e = valid ? s_ids[lane] : 0;
        uint64_t eq = __ballot(valid), lessm = 0;
        for (int b = nbits - 1; b >= 0; --b) {
            const bool bit = (e >> b) & 1;
            const uint64_t B = __ballot(valid && bit);
            if (bit) {
                lessm |= eq & ~B;
                eq &= B;
            } else {
                eq &= ~B;
            }
        }
        const int less = __popcll(lessm);
        const uint64_t before = eq & lanemask_lt();
        const bool first = valid && before == 0;
        const uint64_t firsts = __ballot(first);
        if (valid) {
            const int pos = less + __popcll(before);
            s_pos[lane] = pos;
            s_tok[pos] = lane / k;
            s_wrow[pos] = s_wsel[lane];
        }
        if (first) {
            const int u = __popcll(firsts & lessm);
            s_list[u] = e;
            s_ucnt[u] = __popcll(eq);
            s_uoff[u] = less;
        }
        if (lane == 0) s_U = __popcll(firsts);
    }
    __syncthreads();
    const int U = s_U;

    // ---- phase 2: gate/up + SwiGLU
    const int pairs = I / 2;
    const int nunits = U * pairs;
    constexpr int ncr = 32 * CPL;         // 32-code chunks per weight row (H = 1024 * CPL)
    if constexpr (MODE != kDown) {
    uint4 cg[2][CPL], cu[2][CPL];
    uint32_t sg[2][CPL], su[2][CPL];
    float ggv[2], ugv[2];
#define MOE_FU_LOAD(b, unit)                                                                    \
    do {                                                                                        \
        const int u_ = (unit) / pairs;                                                          \
        const int e_ = s_list[u_];                                                              \
        const int64_t row_ = (int64_t)e_ * I + 2 * ((unit) - u_ * pairs);                       \
        ggv[b] = P.gg[e_];                                                                      \
        ugv[b] = P.ug[e_];                                                                      \
        const uint4* gcr_ = reinterpret_cast<const uint4*>(P.gc + row_ * (H / 2));              \
        const uint4* ucr_ = reinterpret_cast<const uint4*>(P.uc + row_ * (H / 2));              \
        const uint16_t* gsr_ = reinterpret_cast<const uint16_t*>(P.gs + row_ * (H / 16));       \
        const uint16_t* usr_ = reinterpret_cast<const uint16_t*>(P.us + row_ * (H / 16));       \
        _Pragma("unroll") for (int j = 0; j < CPL; ++j) {                                       \
            const int q = lane + kWave * j;                                                     \
            cg[b][j] = gcr_[q];                                                                 \
            cu[b][j] = ucr_[q];                                                                 \
            sg[b][j] = gsr_[q];                                                                 \
            su[b][j] = usr_[q];                                                                 \
        }                                                                                       \
        asm volatile("" ::: "memory");  /* issue here, not at the first use */                  \
    } while (0)

    // h for one unit from the codes in buffer b, for every token of its
    // expert, into this wave's LDS staging slot `slot`.  Stores to memory are
    // batched: one among the loads would make every later load wait for it.
#define MOE_FU_COMPUTE(b, unit, slot)                                                           \
    do {                                                                                        \
        const int u_ = (unit) / pairs;                                                          \
        const int ne_ = s_ucnt[u_], p0_ = s_uoff[u_];                                           \
        int xrow_[MAXT];                                                                        \
        _Pragma("unroll") for (int t = 0; t < MAXT; ++t)                                        \
            xrow_[t] = s_tok[p0_ + (t < ne_ ? t : 0)] * H8;                                     \
        float a0[MAXT], a1[MAXT], b0[MAXT], b1[MAXT];                                           \
        _Pragma("unroll") for (int t = 0; t < MAXT; ++t) a0[t] = a1[t] = b0[t] = b1[t] = 0.0f;  \
        _Pragma("unroll") for (int j = 0; j < CPL; ++j) {                                       \
            const int q = lane + kWave * j;                                                     \
            const bool second = q >= ncr;                                                       \
            const int xo = 4 * (second ? q - ncr : q);                                          \
            /* opaque copies: decode here, once per chunk, not hoisted */                       \
            uint4 g4 = cg[b][j], u4 = cu[b][j];                                                 \
            asm volatile("" : "+v"(g4.x), "+v"(g4.y), "+v"(g4.z), "+v"(g4.w));                  \
            asm volatile("" : "+v"(u4.x), "+v"(u4.y), "+v"(u4.z), "+v"(u4.w));                  \
            const uint32_t gw_[4] = {g4.x, g4.y, g4.z, g4.w};                                   \
            const uint32_t uw_[4] = {u4.x, u4.y, u4.z, u4.w};                                   \
            uint32_t gd[16], ud[16];                                                            \
            _Pragma("unroll") for (int w = 0; w < 4; ++w) {                                     \
                gd[4 * w + 0] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<0>(gw_[w]));        \
                gd[4 * w + 1] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<1>(gw_[w]));        \
                gd[4 * w + 2] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<2>(gw_[w]));        \
                gd[4 * w + 3] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<3>(gw_[w]));        \
                ud[4 * w + 0] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<0>(uw_[w]));        \
                ud[4 * w + 1] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<1>(uw_[w]));        \
                ud[4 * w + 2] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<2>(uw_[w]));        \
                ud[4 * w + 3] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<3>(uw_[w]));        \
            }                                                                                   \
            const float gs0 = e4m3_byte_to_f32<0>(sg[b][j]), gs1 = e4m3_byte_to_f32<1>(sg[b][j]); \
            const float us0 = e4m3_byte_to_f32<0>(su[b][j]), us1 = e4m3_byte_to_f32<1>(su[b][j]); \
            _Pragma("unroll") for (int t = 0; t < MAXT; ++t) {                                  \
                if (t < ne_) {                                                                  \
                    const uint4* xc = smem + xrow_[t] + xo;                                     \
                    const uint4 x0 = xc[0], x1 = xc[1], x2 = xc[2], x3 = xc[3];                 \
                    const uint32_t xw[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,    \
                                             x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};   \
                    float pg0 = 0.0f, pg1 = 0.0f, pu0 = 0.0f, pu1 = 0.0f;                       \
                    _Pragma("unroll") for (int w = 0; w < 8; ++w) {                             \
                        pg0 = dot2_bf16(gd[w], xw[w], pg0);                                     \
                        pg1 = dot2_bf16(gd[8 + w], xw[8 + w], pg1);                             \
                        pu0 = dot2_bf16(ud[w], xw[w], pu0);                                     \
                        pu1 = dot2_bf16(ud[8 + w], xw[8 + w], pu1);                             \
                    }                                                                           \
                    const float dg_ = fmaf(gs0, pg0, gs1 * pg1);                                \
                    const float du_ = fmaf(us0, pu0, us1 * pu1);                                \
                    a0[t] += second ? 0.0f : dg_;                                               \
                    a1[t] += second ? dg_ : 0.0f;                                               \
                    b0[t] += second ? 0.0f : du_;                                               \
                    b1[t] += second ? du_ : 0.0f;                                               \
                }                                                                               \
            }                                                                                   \
        }                                                                                       \
        _Pragma("unroll") for (int t = 0; t < MAXT; ++t) {                                      \
            if (t < ne_) {                                                                      \
                const float sa0 = wave_sum_dpp(a0[t]), sa1 = wave_sum_dpp(a1[t]);               \
                const float sb0 = wave_sum_dpp(b0[t]), sb1 = wave_sum_dpp(b1[t]);               \
                if (lane == 0) {                                                                \
                    const uint32_t h0 = f32_to_bf16_rne(silu(ggv[b] * sa0) * (ugv[b] * sb0));   \
                    const uint32_t h1 = f32_to_bf16_rne(silu(ggv[b] * sa1) * (ugv[b] * sb1));   \
                    s_hst[wave][slot][t] = h0 | (h1 << 16);                                     \
                }                                                                               \
            }                                                                                   \
        }                                                                                       \
    } while (0)

    // store staged unit j (unit first + j) of wave w, token t (device-coherent)
#define MOE_FU_STORE(w, first, j, t)                                                            \
    do {                                                                                        \
        const int unit_ = (first) + (j);                                                        \
        const int u_ = unit_ / pairs;                                                           \
        if ((t) < s_ucnt[u_]) {                                                                 \
            const int n_ = 2 * (unit_ - u_ * pairs);                                            \
            coherent_store(reinterpret_cast<uint32_t*>(P.h + (int64_t)(s_uoff[u_] + (t)) * I + n_), \
                           s_hst[w][j][t]);                                                     \
        }                                                                                       \
    } while (0)
#define MOE_FU_FLUSH(first, nst)                                                                \
    do {                                                                                        \
        for (int idx = lane; idx < (nst) * MAXT; idx += kWave)                                  \
            MOE_FU_STORE(wave, (first), idx / MAXT, idx % MAXT);                                \
    } while (0)

    // units [first, last): two code buffers, the next unit's codes in flight
    // while one is computed; h staged in LDS, flushed every kStageUnits
    // units (the caller stores the last nst_ staged units, from fl_ on)
#define MOE_FU_RUN(first, last)                                                                 \
    int fl_ = (first), nst_ = 0;                                                                \
    do {                                                                                        \
        if ((first) < (last)) MOE_FU_LOAD(0, (first));                                          \
        _Pragma("unroll 1") for (int i = (first); i < (last); i += 2) {                         \
            if (i + 1 < (last)) MOE_FU_LOAD(1, i + 1);                                          \
            MOE_FU_COMPUTE(0, i, nst_);                                                         \
            ++nst_;                                                                             \
            if (i + 1 >= (last)) break;                                                         \
            if (i + 2 < (last)) MOE_FU_LOAD(0, i + 2);                                          \
            MOE_FU_COMPUTE(1, i + 1, nst_);                                                     \
            ++nst_;                                                                             \
            if (nst_ == kStageUnits) {                                                          \
                MOE_FU_FLUSH(fl_, nst_);                                                        \
                fl_ += nst_;                                                                    \
                nst_ = 0;                                                                       \
            }                                                                                   \
        }                                                                                       \
    } while (0)

    {
        // this workgroup's run of units: equal shares of the total cost
        int64_t total = 0;
        for (int u = 0; u < U; ++u) total += (int64_t)pairs * (kMemCost + s_ucnt[u]);
        auto unit_at = [&](int64_t c) {
            int64_t cum = 0;
            for (int u = 0; u < U; ++u) {
                const int per = kMemCost + s_ucnt[u];
                const int64_t span = (int64_t)pairs * per;
                if (c < cum + span) return u * pairs + (int)((c - cum + per - 1) / per);
                cum += span;
            }
            return nunits;
        };
        const int wg0 = unit_at(total * blockIdx.x / G);
        const int wg1 = unit_at(total * (blockIdx.x + 1) / G);
        const int per_wave = (wg1 - wg0 + kNW - 1) / kNW;
        const int w0 = min(wg1, wg0 + wave * per_wave), w1 = min(wg1, w0 + per_wave);
        MOE_FU_RUN(w0, w1);
        if (lane == 0) {
            s_fl_first[wave] = fl_;
            s_fl_n[wave] = nst_;
        }
    }
    // the workgroup's staged h values go out together, then one count for
    // the workgroup
    __syncthreads();
    for (int idx = threadIdx.x; idx < kNW * kStageUnits * MAXT; idx += kFThreads) {
        const int w = idx / (kStageUnits * MAXT), j = (idx / MAXT) % kStageUnits, t = idx % MAXT;
        if (j < s_fl_n[w]) MOE_FU_STORE(w, s_fl_first[w], j, t);
    }
    if constexpr (MODE == kFused) {
        wait_all_memory();   // this wave's h stores are complete
        __syncthreads();
        if (threadIdx.x == 0) counter_add(P.sync + kSyncDone, 1u);
    }
    }   // MODE != kDown
    if constexpr (MODE == kGateUp) return;

    // ---- phase 3 set-up: this workgroup's row pairs, the first chunk's codes
    const int half = lane >> 5, l32 = lane & 31;
    const int npairs = H / 2;
    const int pb0 = (int)((int64_t)blockIdx.x * npairs / G);
    const int npw = (int)((int64_t)(blockIdx.x + 1) * npairs / G) - pb0;   // <= kMaxPairs
    const int chunk_cap = min(kChunkExperts, kItemWaves * kItems / max(npw, 1));
    const int ngroups = I / 16;           // scale bytes per down row (= 32 * GPL2)
    uint2 cw[kItems][GPL2];
    uint32_t sw[kItems];               // a row's scale bytes: half-wave lane l holds dword min(l, 8 GPL2 - 1)
    float dgv[kItems];
    // chunk [u0, u1) of the touched experts: at most chunk_cap experts and
    // kChunkSlots h rows (expert-sorted rows pA .. pB)
#define MOE_FD_CHUNK(u0, u1, pA, pB)                                                            \
    do {                                                                                        \
        pA = s_uoff[u0];                                                                        \
        u1 = u0 + 1;                                                                            \
        while (u1 < U && u1 - u0 < chunk_cap && s_uoff[u1] + s_ucnt[u1] - pA <= kChunkSlots)    \
            ++u1;                                                                               \
        pB = s_uoff[u1 - 1] + s_ucnt[u1 - 1];                                                   \
    } while (0)
    // the chunk's items (row pair, expert), pair-major, are dealt to waves
    // 1..kItemWaves in contiguous blocks of per_ (<= kItems): wave w takes
    // items [(w - 1) per_, w per_), walked with a running (pair, expert)
#define MOE_FD_BLOCK(nu_, i0_, i1_)                                                             \
    const int per_##i0_ = (npw * (nu_) + kItemWaves - 1) / kItemWaves;                          \
    const int i0_ = wave >= 1 ? min(npw * (nu_), (wave - 1) * per_##i0_) : npw * (nu_);        \
    const int i1_ = min(npw * (nu_), i0_ + per_##i0_)
#define MOE_FD_LOAD(u0, u1)                                                                     \
    do {                                                                                        \
        const int nu_ = (u1) - (u0);                                                            \
        MOE_FD_BLOCK(nu_, i0_, i1_);                                                            \
        int pl_ = i0_ / nu_, ul_ = i0_ - (i0_ / nu_) * nu_;                                     \
        _Pragma("unroll") for (int s = 0; s < kItems; ++s) {                                    \
            if (i0_ + s < i1_) {                                                                \
                const int e_ = s_list[(u0) + ul_];                                              \
                const int64_t row_ = (int64_t)e_ * H + 2 * (pb0 + pl_) + half;                  \
                dgv[s] = P.dg[e_];                                                              \
                _Pragma("unroll") for (int j = 0; j < GPL2; ++j)                                \
                    cw[s][j] = reinterpret_cast<const uint2*>(P.dc + row_ * (I / 2))[l32 + 32 * j]; \
                sw[s] = reinterpret_cast<const uint32_t*>(P.ds + row_ * ngroups)[min(l32, 8 * GPL2 - 1)]; \
            }                                                                                   \
            if (++ul_ == nu_) {                                                                 \
                ul_ = 0;                                                                        \
                ++pl_;                                                                          \
            }                                                                                   \
        }                                                                                       \
        asm volatile("" ::: "memory");                                                          \
    } while (0)
    int u0 = 0, u1 = 0, pA = 0, pB = 0;
    if (U > 0) {
        MOE_FD_CHUNK(u0, u1, pA, pB);
        MOE_FD_LOAD(u0, u1);     // streams while the last gate/up units finish
    }

    if constexpr (MODE == kFused) {
    // ---- hand-off: wave 0 (no loads in flight) polls the count
    if (threadIdx.x == 0) {
        bool ok = false;
        for (int polls = 0;; ++polls) {
            ok = coherent_load(P.sync + kSyncDone) >= (uint32_t)G;
            if (ok || polls >= P.wait_limit) break;
            __builtin_amdgcn_s_sleep(2);
        }
        s_go = ok ? 1 : 0;
    }
    wait_lds_barrier();   // not a full fence: the down codes stay in flight
    if (!s_go) {
        // not every workgroup of the grid has run yet: compute all of h here
        // with the same arithmetic (so the same bits as any other writer),
        // one unit and token at a time, straight from memory; the down codes
        // requested above stay in flight
        for (int unit = wave; unit < nunits; unit += kNW) {
            const int u = unit / pairs;
            const int e = s_list[u];
            const int n = 2 * (unit - u * pairs);
            const int64_t row = (int64_t)e * I + n;
            const uint4* gcr = reinterpret_cast<const uint4*>(P.gc + row * (H / 2));
            const uint4* ucr = reinterpret_cast<const uint4*>(P.uc + row * (H / 2));
            const uint16_t* gsr = reinterpret_cast<const uint16_t*>(P.gs + row * (H / 16));
            const uint16_t* usr = reinterpret_cast<const uint16_t*>(P.us + row * (H / 16));
            const float g_gate = P.gg[e], g_up = P.ug[e];
            for (int t = 0; t < s_ucnt[u]; ++t) {
                const int p = s_uoff[u] + t;
                const uint4* xq = smem + s_tok[p] * H8;
                float a0 = 0.0f, a1 = 0.0f, b0 = 0.0f, b1 = 0.0f;
                for (int j = 0; j < CPL; ++j) {
                    const int q = lane + kWave * j;
                    const bool second = q >= ncr;
                    const uint4* xc = xq + 4 * (second ? q - ncr : q);
                    const uint4 g4 = gcr[q], u4 = ucr[q];
                    const uint32_t gsc = gsr[q], usc = usr[q];
                    // the same operations in the same order as the main path
                    const float pg0 = group_dot(make_uint2(g4.x, g4.y), xc[0], xc[1]);
                    const float pg1 = group_dot(make_uint2(g4.z, g4.w), xc[2], xc[3]);
                    const float pu0 = group_dot(make_uint2(u4.x, u4.y), xc[0], xc[1]);
                    const float pu1 = group_dot(make_uint2(u4.z, u4.w), xc[2], xc[3]);
                    const float dg_ = fmaf(e4m3_byte_to_f32<0>(gsc), pg0, e4m3_byte_to_f32<1>(gsc) * pg1);
                    const float du_ = fmaf(e4m3_byte_to_f32<0>(usc), pu0, e4m3_byte_to_f32<1>(usc) * pu1);
                    a0 += second ? 0.0f : dg_;
                    a1 += second ? dg_ : 0.0f;
                    b0 += second ? 0.0f : du_;
                    b1 += second ? du_ : 0.0f;
                }
                a0 = wave_sum_dpp(a0);
                a1 = wave_sum_dpp(a1);
                b0 = wave_sum_dpp(b0);
                b1 = wave_sum_dpp(b1);
                if (lane == 0) {
                    const uint32_t h0 = f32_to_bf16_rne(silu(g_gate * a0) * (g_up * b0));
                    const uint32_t h1 = f32_to_bf16_rne(silu(g_gate * a1) * (g_up * b1));
                    coherent_store(reinterpret_cast<uint32_t*>(P.h + (int64_t)p * I + n), h0 | (h1 << 16));
                }
            }
        }
        wait_all_memory();
        __syncthreads();
    }
    }   // MODE == kFused
#undef MOE_FU_LOAD
#undef MOE_FU_COMPUTE
#undef MOE_FU_STORE
#undef MOE_FU_FLUSH
#undef MOE_FU_RUN

    // ---- phase 3: down + combine
    // thread (pair pc, half hc, token tc) owns one output value
    const int tc = threadIdx.x % MAXT, hc = (threadIdx.x / MAXT) & 1, pc = threadIdx.x / (2 * MAXT);
    float acc = 0.0f;
    while (u0 < U) {
        if (u0 > 0) {
            MOE_FD_CHUNK(u0, u1, pA, pB);
            MOE_FD_LOAD(u0, u1);
        }
        const int nu = u1 - u0;
        // h rows of the chunk straight to LDS with device-coherent loads
        {
            const uint4* hsrc = reinterpret_cast<const uint4*>(P.h + (int64_t)pA * I);
            const int nchunk = (pB - pA) * I8 / 64;   // I % 512 == 0
            for (int c = wave; c < nchunk; c += kNW)
                __builtin_amdgcn_global_load_lds(hsrc + c * 64 + lane, (lds_void*)(smem + c * 64), 16, 0,
                                                 16 /* sc1: device scope */);
        }
        wait_all_memory();
        __syncthreads();

        {
            // this wave's block: partial sums per token accumulate over the
            // block's experts of one row pair, then one half-wave reduction
            // per (row pair, token) goes to LDS
            MOE_FD_BLOCK(nu, i0, i1);
            int pl = i0 / nu, ul = i0 - (i0 / nu) * nu, lp = 0;
            float accp[MAXT];
#pragma unroll
            for (int t = 0; t < MAXT; ++t) accp[t] = 0.0f;
#pragma unroll
            for (int s = 0; s < kItems; ++s) {
                if (i0 + s < i1) {
                    const int u = u0 + ul;
                    float sc[GPL2];
#pragma unroll
                    for (int j = 0; j < GPL2; ++j) {
                        // scale byte of group l32 + 32 j: dword l32 / 4 + 8 j of the half-wave
                        const int src = (lane & 32) + (l32 >> 2) + 8 * j;
                        const uint32_t d = (uint32_t)__builtin_amdgcn_ds_bpermute(src * 4, (int)sw[s]);
                        sc[j] = e4m3_to_f32((d >> (8 * (l32 & 3))) & 0xFFu);
                    }
                    const int p0 = s_uoff[u], ne = s_ucnt[u];
                    for (int p = p0; p < p0 + ne; ++p) {
                        const uint4* hr = smem + (p - pA) * I8;
                        float a = 0.0f;
#pragma unroll
                        for (int j = 0; j < GPL2; ++j) {
                            const int g = l32 + 32 * j;
                            a += sc[j] * group_dot(cw[s][j], hr[2 * g], hr[2 * g + 1]);
                        }
                        const float wa = (s_wrow[p] * dgv[s]) * a;
                        if (MAXT == 1) {
                            accp[0] += wa;
                        } else {
                            const int t = s_tok[p];
#pragma unroll
                            for (int tt = 0; tt < MAXT; ++tt)
                                if (tt == t) accp[tt] += wa;
                        }
                    }
                    if (ul + 1 == nu || i0 + s + 1 == i1) {   // last item of this row pair in the block
#pragma unroll
                        for (int t = 0; t < MAXT; ++t) {
                            if (t < T) {
                                const float v = half_wave_sum_dpp(accp[t]);
                                if (l32 == 0) s_part[wave - 1][lp][half][t] = v;
                            }
                            accp[t] = 0.0f;
                        }
                        ++lp;
                    }
                }
                if (++ul == nu) {
                    ul = 0;
                    ++pl;
                }
            }
        }
        __syncthreads();
        if (pc < npw) {
            // the waves whose blocks hold items of pair pc, in order (ascending expert)
            const int per = (npw * nu + kItemWaves - 1) / kItemWaves;
            const int wa = pc * nu / per, wb = (pc * nu + nu - 1) / per;
            for (int w = wa; w <= wb; ++w) acc += s_part[w][pc - (w * per) / nu][hc][tc];
        }
        __syncthreads();   // s_part and the h rows are free again
        u0 = u1;
    }
#undef MOE_FD_CHUNK
#undef MOE_FD_LOAD
#undef MOE_FD_BLOCK
    if (pc < npw && tc < T) P.out[(int64_t)tc * H + 2 * (pb0 + pc) + hc] = f32_to_bf16_rne(acc);

    // ---- routing outputs (routed here): workgroup 0 the per-slot arrays,
    // every workgroup its share of the per-expert ones
    if (P.logits) {
        if (blockIdx.x == 0 && threadIdx.x < slots) {
            const int i = threadIdx.x, pos = s_pos[i];
            P.ids_out[i] = s_ids[i];
            P.w_out[i] = s_wsel[i];
            P.pos_out[i] = pos;
            P.sorted_out[pos] = i;
        }
        const int e0 = (int)((int64_t)blockIdx.x * E / G), e1 = (int)((int64_t)(blockIdx.x + 1) * E / G);
        for (int e = e0 + threadIdx.x; e < e1; e += kFThreads) {
            int cnt = 0, off = 0;
            for (int u = 0; u < U; ++u) {
                if (s_list[u] < e) off += s_ucnt[u];
                if (s_list[u] == e) cnt = s_ucnt[u];
            }
            P.counts_out[e] = cnt;
            P.offsets_out[e] = off;
        }
        if (blockIdx.x == G - 1 && threadIdx.x == 0) P.offsets_out[E] = slots;
    }

    // ---- exit: the last workgroup resets the hand-off counters
    if constexpr (MODE != kFused) return;
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t before = counter_add(P.sync + kSyncExit, 1u);
        if (before == (uint32_t)G - 1) {
            coherent_store(P.sync + kSyncDone, 0u);
            coherent_store(P.sync + kSyncExit, 0u);
        }
    }
}

template <int CPL, int GPL2, int MAXT, int MODE>
moe_status launch_one(const FusedParams& p, int grid, hipStream_t s) {
    const size_t xb = MODE == kDown ? 0 : (size_t)p.T * p.H;
    const size_t hb = MODE == kGateUp ? 0 : (size_t)kChunkSlots * p.I;
    const size_t shmem = std::max(xb, hb) * sizeof(uint16_t);
    auto kern = k_dec_fused<CPL, GPL2, MAXT, MODE>;
    if (allow_dynamic_lds(reinterpret_cast<const void*>(kern), shmem) != MOE_OK) return MOE_ERR_HIP;
    const char* name = MODE == kFused ? "dec_fused" : MODE == kGateUp ? "dec_gateup" : "dec_down";
    MOE_LAUNCH(name, kern, dim3(grid), dim3(kFThreads), shmem, s, p);
    return MOE_OK;
}

template <int CPL, int MAXT, int MODE>
moe_status launch_gpl2(const FusedParams& p, int grid, hipStream_t s) {
    switch (p.I / 512) {
        case 1: return launch_one<CPL, 1, MAXT, MODE>(p, grid, s);
        case 2: return launch_one<CPL, 2, MAXT, MODE>(p, grid, s);
        case 3: return launch_one<CPL, 3, MAXT, MODE>(p, grid, s);
        case 4: return launch_one<CPL, 4, MAXT, MODE>(p, grid, s);
        default: return MOE_ERR_UNSUPPORTED;
    }
}

// Launch k_dec_fused for p.H / 1024 (<= kMaxCPL) and p.I / 512; one
// translation unit per (MAXT, MODE) keeps the build parallel.
template <int MAXT, int MODE>
moe_status launch_shape(const FusedParams& p, int grid, hipStream_t s) {
    switch (p.H / 1024) {
        case 1: return launch_gpl2<1, MAXT, MODE>(p, grid, s);
        case 2: return launch_gpl2<2, MAXT, MODE>(p, grid, s);
        case 3: return launch_gpl2<3, MAXT, MODE>(p, grid, s);
        case 4: return launch_gpl2<4, MAXT, MODE>(p, grid, s);
        case 5: return launch_gpl2<5, MAXT, MODE>(p, grid, s);
        default: return MOE_ERR_UNSUPPORTED;
    }
}
moe_status launch_t1_fused(const FusedParams& p, int grid, hipStream_t s);
moe_status launch_t1_gateup(const FusedParams& p, int grid, hipStream_t s);
moe_status launch_t1_down(const FusedParams& p, int grid, hipStream_t s);
moe_status launch_t8_fused(const FusedParams& p, int grid, hipStream_t s);
moe_status launch_t8_gateup(const FusedParams& p, int grid, hipStream_t s);
moe_status launch_t8_down(const FusedParams& p, int grid, hipStream_t s);

}  // namespace fused
}  // namespace moe
