// Decode-shape forward (a few tokens): HBM-bound weight streaming.
//
// With 1-8 tokens the layer is a handful of matrix-vector products per
// touched expert; the time is the HBM read of the packed weights (the pages
// call this regime the memory-bandwidth wall: "GLM-5.3-Flash on Blackwell",
// "Two deployments, and the lever that reverses between them").  The W4A16
// route dequantises weights to bf16 and never reads an activation scale
// ("GLM-5.3-Flash on Blackwell", "The model loaded, served an API, and
// produced garbage").
//
// Weights are read with the non-temporal cache policy: each byte is used once
// per step, and streaming ~100 MB per layer through L2 and the Infinity Cache
// at the normal policy evicts the lines that the next launches need at once
// (measured on MI355X: one-token step 31.6 -> 29.4 us).
//
// Two kernels:
//   k_dec_gateup: one workgroup per (touched expert, block of rows of I).
//     The expert's tokens are staged once in LDS.  Lanes split K: lane l
//     owns the 16-groups l, l+64, ... of a row, so each wave load is a
//     contiguous 512 B run of codes.  A wave walks its rows with the next
//     row's gate and up codes already in flight (register double buffer).
//     Codes decode to bf16 pairs (gfx950 FP4 conversion) and meet x in
//     v_dot2_f32_bf16; the group scale multiplies each 16-term partial sum,
//     the global scale the row total.  Row sums are DPP reductions; SwiGLU
//     runs on the gate/up pair and h is rounded once to bf16 and stored in
//     expert-sorted row order.
//   k_dec_down: one workgroup per block of output rows of H; every wave owns
//     two rows (one per half-wave) and loops over every touched expert in
//     ascending order and every token of that expert, so the
//     routing-weighted combine happens in registers (fp32, fixed order, no
//     atomics) and out is written once in bf16.  Wave 0 orders the slots
//     from the top-k ids alone (ballots on the expert bits), so the weight
//     loads wait for one small load only.  A lane reads adjacent group
//     pairs (16-byte code loads) and the row's scales as whole dwords handed
//     out by ds_bpermute.  The h rows of a chunk of experts (contiguous in
//     sorted order) are staged in LDS once per workgroup, permuted so that
//     every LDS read is 32 consecutive 16-byte slots, and the weight codes of
//     the whole chunk are loaded before any of them is used.
#include "device_common.h"
#include "internal.h"
#include "quant_common.h"
#include "route_common.h"

namespace moe {
namespace {

constexpr int kGuThreads = 256;         // gate/up workgroup
constexpr int kGuWaves = kGuThreads / kWave;
constexpr int kDownMaxWaves = 12;
// A chunk: experts whose down codes are requested in one sequence, and the
// h rows staged in LDS for them.  One token touches k experts, so one chunk
// holds them all; with more tokens larger chunks mean fewer restarts of the
// load sequence (each costs a memory latency).
template <int MAXT> constexpr int down_chunk_experts() { return MAXT == 1 ? 8 : 16; }
template <int MAXT> constexpr int down_chunk_slots() { return MAXT == 1 ? 16 : 48; }
#ifndef MOE_DOWN_AHEAD
#define MOE_DOWN_AHEAD 3
#endif
constexpr int kDownAhead = MOE_DOWN_AHEAD;   // experts' down codes in flight ahead of the one computed
constexpr int kDownRows = 1;            // output rows per half-wave (more: fewer waves, measured slower)
constexpr int kDecodeMaxSlots = 64;     // T * k on the decode path
constexpr int kXTokens = 2;             // activation rows staged in LDS at a time (gate/up)
constexpr int kXTokensLinear = 4;       // the same for the one-stack projection (few registers, 4 per CU fit)
// one always-on expert (a shared expert): its few workgroups (I / 8) run one
// per CU, so every token's row is staged at once (8 tokens: 16.3 -> 15.3 us
// for the gate/up kernel at H 5120, I 1536; the one-stack projection, with
// five times the workgroups, measured slower with 8)
constexpr int kXTokensOne = 8;
template <bool LINEAR, bool ONE = false> constexpr int x_stage_tokens() {
    return LINEAR ? kXTokensLinear : ONE ? kXTokensOne : kXTokens;
}

// A wave computes two consecutive output features n, n + 1 per stage.  Their
// gate rows are one contiguous run of H codes (H / 16 chunks of 32), as are
// their up rows; lane l takes chunk q = l + 64 j (j < CPL, H = 1024 * CPL)
// of both runs, so gate and up share the activation chunk and every load is a
// uniform base plus a 16-byte lane offset.  Chunk q belongs to feature
// n + (q >= H / 32).  RW stages (2 * RW features) per wave, EPL = expert
// counts per lane (E <= 64 * EPL).
// The expert lookup needs one batch of small loads; the activation rows then
// go straight to LDS, and the codes of all stages are requested before any
// is used: stages are computed in order as they land (vector loads complete
// in issue order).
// Routing computed by the gate/up kernel itself, for one token
// (moe_w4a16_route_forward with T == 1): every workgroup recomputes the token's top-k from its E logits
// and the expert order of the k slots, which replaces the lookup of the
// routing outputs (one dependent load either way) and saves the route
// launch; the workgroups of expert column 0 store the routing outputs for the
// down kernel and the caller.  With more tokens every workgroup would repeat
// all their top-k selections, so those shapes route in their own kernel.
struct GuRoute {
    const float* logits;        // [1][E]
    int32_t* ids;               // [k]
    float* w;                   // [k]
    int32_t* counts;            // [E]
    int32_t* offsets;           // [E + 1]
    int32_t* sorted_slots;      // [k]
    int32_t* slot_pos;          // [k]
};

// LINEAR: one weight stack only (gc/gs/gg), no SwiGLU: the row sums times
// the global scale go out as bf16 (a dense projection; h is then the output).
// ONE: a single always-on expert (a shared expert): tokens in order, no
// routing arrays read (LINEAR implies it).
// QH (W4A4, RW == 2): a workgroup's 16 features of a token are one 16-group
// of h; the workgroup quantizes it to NVFP4 under h_qscale and stores the
// group's values E2M1 * E4M3 as bf16 (exact; the down kernel applies the
// input scale), so no separate quantization pass over h is needed.
template <int CPL, int RW, int EPL, bool ROUTE, bool LINEAR = false, bool ONE = false, bool QH = false>
__global__ void __launch_bounds__(kGuThreads, RW == 1 ? 4 : 3)
k_dec_gateup(const uint16_t* __restrict__ x, int H, int I, int E, int k, int slots,
             const uint8_t* gc, const uint8_t* gs, const float* __restrict__ gg,
             const uint8_t* uc, const uint8_t* us, const float* __restrict__ ug,
             const int32_t* __restrict__ counts, const int32_t* __restrict__ sorted_slots,
             uint16_t* __restrict__ h, const GuRoute R, float x_scale, float* __restrict__ hf, float h_qscale) {
    static_assert(!QH || (RW == 2 && !LINEAR), "a 16-feature workgroup per h group");
    constexpr int kXT = x_stage_tokens<LINEAR, ONE>();
    constexpr int kGroupFeatures = kGuWaves * 2 * RW;          // features of I per workgroup
    extern __shared__ uint4 xs[];   // [kXT][H / 8]
    __shared__ float s_hq[QH ? 8 : 1][QH ? kGroupFeatures : 1];  // this workgroup's h values per token (QH)
    __shared__ int s_ids[kDecodeMaxSlots], s_pos[kDecodeMaxSlots], s_sorted[kDecodeMaxSlots];
    __shared__ int s_list[kDecodeMaxSlots], s_ucnt[kDecodeMaxSlots], s_uoff[kDecodeMaxSlots];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int my_slot, e, ne, p0, U = 0;
    if constexpr (ROUTE) {
        // one token: the selected experts as a set (threshold search); with
        // one token each expert holds one slot, so the sorted slot order is
        // the ascending expert order that the selection flags give directly.
        // The order of the slots by logit is needed for the stored routing
        // outputs alone: the one workgroup that stores them ranks the
        // selection after its weight loads are out.
        if (wave == 0) {
            uint32_t key[EPL];
            uint64_t sel[EPL];
            wave_topk_set<EPL>(R.logits, E, k, key, sel);
            int base = 0;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                if ((sel[i] >> lane) & 1u) {
                    const int u = base + __popcll(sel[i] & lanemask_lt());
                    s_list[u] = kWave * i + lane;
                    s_ucnt[u] = 1;
                    s_uoff[u] = u;
                    s_sorted[u] = (int)key[i];          // the selected keys, ascending expert
                }
                base += __popcll(sel[i]);
            }
        }
        __syncthreads();
        U = slots;                                     // k distinct experts
        e = s_list[blockIdx.y];
        ne = 1;
        p0 = blockIdx.y;
        my_slot = 0;                                   // token 0 for every slot
    } else {
        if constexpr (LINEAR || ONE) {   // one always-on stack: token order, no routing arrays
            my_slot = lane;
            e = 0; ne = slots; p0 = 0;
        } else {
            my_slot = lane < slots ? sorted_slots[lane] : 0;   // slots <= 64 on this path
            const ActiveExpert ae = nth_active_expert<EPL>(counts, E, blockIdx.y);
            if (ae.e < 0) return;
            e = ae.e; ne = ae.count; p0 = ae.first_row;
        }
    }
    const int H8 = H / 8;
    constexpr int ncr = 32 * CPL;            // 32-wide chunks per weight row (H = 1024 * CPL)

    // activation rows of up to kXT tokens at a time live in LDS
    const int nchunk = H8 / 64;              // H % 512 == 0 on this path
    auto stage_x = [&](int q0) {
        for (int q = q0; q < min(ne, q0 + kXT); ++q) {
            const int t = __builtin_amdgcn_readlane(my_slot, p0 + q) / k;
            const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * H);
            for (int c = wave; c < nchunk; c += kGuWaves)
                wave_copy_1k_to_lds(src + c * 64, xs + (q - q0) * H8 + c * 64);
        }
    };
    stage_x(0);

    const int nb = (blockIdx.x * kGuWaves + wave) * (2 * RW);   // first feature of this wave
    const float g_gate = gg[e] * x_scale, g_up = LINEAR ? 0.0f : ug[e] * x_scale;
    constexpr int kLoadsPerChunk = LINEAR ? 2 : 4;
    // the codes of all RW stages are requested at once and stay in registers
    // for every token of the expert
    uint4 cg[RW][CPL], cu[RW][CPL];
    uint32_t sg[RW][CPL], su[RW][CPL];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const int64_t row = (int64_t)e * I + min(nb + 2 * r, I - 2);
        const uint4* gcr = reinterpret_cast<const uint4*>(gc + row * (H / 2));
        const uint4* ucr = reinterpret_cast<const uint4*>(uc + row * (H / 2));
        const uint16_t* gsr = reinterpret_cast<const uint16_t*>(gs + row * (H / 16));
        const uint16_t* usr = reinterpret_cast<const uint16_t*>(us + row * (H / 16));
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int q = lane + kWave * j;
            cg[r][j] = load_stream16(&gcr[q]);
            if constexpr (!LINEAR) cu[r][j] = load_stream16(&ucr[q]);
            else cu[r][j] = make_uint4(0, 0, 0, 0);
            sg[r][j] = load_stream(&gsr[q]);
            if constexpr (!LINEAR) su[r][j] = load_stream(&usr[q]);
            else su[r][j] = 0;
        }
    }
    asm volatile("" ::: "memory");           // issue here, not at the first use
    // x rows (issued first) and stage 0's codes; later stages stay in flight
    wait_vmem_at_most<kLoadsPerChunk * CPL * (RW - 1)>();
    __builtin_amdgcn_s_barrier();            // plain barrier: a fence would wait for every load

#pragma unroll 1
    for (int q0 = 0; q0 < ne; q0 += kXT) {
        if (q0 > 0) {                        // next tokens: restage x
            __syncthreads();
            stage_x(q0);
            wait_all_memory();
            __syncthreads();
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const int n = nb + 2 * r;
#pragma unroll 1
            for (int qt = q0; qt < min(ne, q0 + kXT); ++qt) {
                const uint4* xq = xs + (qt - q0) * H8;
                float a0 = 0.0f, a1 = 0.0f, b0 = 0.0f, b1 = 0.0f;
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    const int q = lane + kWave * j;
                    const bool second = q >= ncr;
                    const uint4* xc = xq + 4 * (second ? q - ncr : q);
                    const uint4 x0 = xc[0], x1 = xc[1], x2 = xc[2], x3 = xc[3];
                    // opaque copies: keep the code decode inside the token loop instead
                    // of hoisting 2 x CPL x 16 decoded pairs into registers
                    uint4 g4 = cg[r][j], u4 = cu[r][j];
                    const uint32_t gsc = sg[r][j], usc = su[r][j];
                    asm volatile("" : "+v"(g4.x), "+v"(g4.y), "+v"(g4.z), "+v"(g4.w));
                    asm volatile("" : "+v"(u4.x), "+v"(u4.y), "+v"(u4.z), "+v"(u4.w));
                    const float dg_ = e4m3_byte_to_f32<0>(gsc) * group_dot(make_uint2(g4.x, g4.y), x0, x1) +
                                      e4m3_byte_to_f32<1>(gsc) * group_dot(make_uint2(g4.z, g4.w), x2, x3);
                    const float du_ = LINEAR ? 0.0f
                                             : e4m3_byte_to_f32<0>(usc) * group_dot(make_uint2(u4.x, u4.y), x0, x1) +
                                                   e4m3_byte_to_f32<1>(usc) * group_dot(make_uint2(u4.z, u4.w), x2, x3);
                    a0 += second ? 0.0f : dg_;
                    a1 += second ? dg_ : 0.0f;
                    b0 += second ? 0.0f : du_;
                    b1 += second ? du_ : 0.0f;
                }
                a0 = wave_sum_dpp(a0);
                a1 = wave_sum_dpp(a1);
                if constexpr (!LINEAR) {
                    b0 = wave_sum_dpp(b0);
                    b1 = wave_sum_dpp(b1);
                }
                if (lane < 2 && n + lane < I) {
                    const float av = lane ? a1 : a0, bv = lane ? b1 : b0;
                    const float v = LINEAR ? g_gate * av : silu(g_gate * av) * (g_up * bv);
                    if constexpr (QH) {
                        s_hq[qt][n + lane - (int)blockIdx.x * kGroupFeatures] = v;
                    } else {
                        const int64_t idx = (int64_t)(p0 + qt) * I + n + lane;
                        if (hf) hf[idx] = v;
                        else h[idx] = f32_to_bf16_rne(v);
                    }
                }
            }
        }
    }

    if constexpr (QH) {
        // 16 lanes per token quantize the token's 16-feature group, one
        // feature each (every lane of a wave takes part in the group maximum)
        __syncthreads();
        const int t = (int)threadIdx.x;
        if (t < kWave * ((ne * 16 + kWave - 1) / kWave)) {        // whole waves
            const int q = t / 16, f = t % 16;
            const float v = q < ne ? s_hq[q][f] : 0.0f;
            const uint16_t b = nvfp4_lane_value_bf16(v, h_qscale);
            if (q < ne) h[(int64_t)(p0 + q) * I + (int64_t)blockIdx.x * kGroupFeatures + f] = b;
        }
    }

    // routing outputs: workgroup (0, 0) the per-slot arrays, the workgroups
    // of expert column 0 their share of the per-expert ones
    if constexpr (ROUTE) {
        if (blockIdx.y != 0) return;
        if (blockIdx.x == 0 && wave == 0) {
            // rank the k selections by (logit desc, expert asc): lane j < k
            // holds the j-th in ascending expert order (sorted position j)
            const int j = lane < slots ? lane : 0;
            const uint32_t kj = (uint32_t)s_sorted[j];
            const int ej = s_list[j];
            int rank = 0;
#pragma unroll
            for (int m = 0; m < MOE_MAX_TOPK; ++m) {   // slots = k <= 32 with one token
                if (m < slots) {
                    const uint32_t km = (uint32_t)s_sorted[m];
                    rank += (km > kj || (km == kj && s_list[m] < ej)) ? 1 : 0;
                }
            }
            if (lane < slots) {
                s_ids[rank] = ej;
                s_pos[rank] = lane;
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);        // this wave's LDS writes land before the reads below
            const int id = lane < slots ? s_ids[lane] : 0;
            const float v = lane < slots ? topk_key_value((uint32_t)s_sorted[s_pos[lane]]) : 0.0f;
            const float w = topk_softmax(v, k);
            if (lane < slots) {
                const int pos = s_pos[lane];           // slot `lane` (by logit) sits at sorted position pos
                R.ids[lane] = id;
                R.w[lane] = w;
                R.slot_pos[lane] = pos;
                R.sorted_slots[pos] = lane;
            }
        }
        const int G = gridDim.x;
        const int e0 = (int)((int64_t)blockIdx.x * E / G), e1 = (int)((int64_t)(blockIdx.x + 1) * E / G);
        for (int ee = e0 + (int)threadIdx.x; ee < e1; ee += kGuThreads) {
            int cnt = 0, off = 0;
            for (int u = 0; u < U; ++u) {
                if (s_list[u] < ee) off += s_ucnt[u];
                if (s_list[u] == ee) cnt = s_ucnt[u];
            }
            R.counts[ee] = cnt;
            R.offsets[ee] = off;
        }
        if (blockIdx.x == G - 1 && threadIdx.x == 0) R.offsets[E] = slots;
    }
}

// GPL2 = 16-groups per half-wave lane along I (I = 512 * GPL2); MAXT tokens.
// ONE: a single always-on expert, weight 1 (ids and weights are not read).
template <int GPL2, int MAXT, bool ONE = false>
__global__ void __launch_bounds__(kDownMaxWaves * kWave)
k_dec_down(const uint16_t* __restrict__ h, int T, int H, int I, int E, int k,
           const uint8_t* dc, const uint8_t* ds, const float* __restrict__ dg,
           const int32_t* __restrict__ ids, const float* __restrict__ topk_w,
           uint16_t* __restrict__ out, int slot_cap, float h_scale) {
    constexpr int kDownChunkExperts = down_chunk_experts<MAXT>();
    extern __shared__ uint4 hs[];     // [slot_cap][I / 8]
    __shared__ int s_list[kDecodeMaxSlots], s_ucnt[kDecodeMaxSlots], s_uoff[kDecodeMaxSlots];
    __shared__ uint32_t s_tmask[kDecodeMaxSlots];   // tokens routed to touched expert u (bit t)
    __shared__ float s_wgt[kDecodeMaxSlots];
    __shared__ int s_cu[kDecodeMaxSlots + 1];   // chunk c: touched experts [s_cu[c], s_cu[c + 1])
    __shared__ int s_U, s_NC;
    constexpr int R = kDownRows;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int half = lane >> 5, l32 = lane & 31;
    const int waves = blockDim.x / kWave;
    const int n0 = ((blockIdx.x * waves + wave) * 2 + half) * R;   // first output row of H
    const int ngroups = I / 16, I8 = I / 8;
    const int slots = T * k;                                   // <= kDecodeMaxSlots on this path

    // Wave 0 orders the slots by (expert, flat slot index) -- the order of
    // the h rows -- from the top-k ids alone, in registers: one ballot per
    // expert bit splits the lanes still equal so far into smaller and equal.
    // It then groups the touched experts (ascending) into chunks.
    if (wave == 0) {
        const bool valid = lane < slots;
        int ex = 0;
        float wv = valid ? 1.0f : 0.0f;
        if constexpr (!ONE) {
            // both loads issued together (clamped index, no branch around
            // either): one memory round trip before the slot order
            const int j = lane < slots ? lane : 0;
            const int ex_ = ids[j];
            const float wv_ = topk_w[j];
            ex = valid ? ex_ : 0;
            wv = valid ? wv_ : 0.0f;
        }
        ex = min(max(ex, 0), E - 1);     // keeps every weight address inside the stacks
        const SlotOrder o = wave_slot_order(ex, valid, E);
        const uint64_t eq = o.eq;
        const int less = o.less, uj = o.u;                     // uj: rank of this slot's expert
        const bool first = o.first;
        const int endj = less + __popcll(eq);                  // sorted end of this slot's expert
        if (valid) s_wgt[o.pos] = wv;
        if (first) {
            // a token routes to an expert at most once: its slots t*k .. t*k+k-1
            uint32_t tm = 0;
            const uint64_t km = k < 64 ? (1ull << k) - 1 : ~0ull;
            for (int t = 0; t < T; ++t) tm |= ((eq >> (t * k)) & km) ? 1u << t : 0u;
            s_list[uj] = ex;
            s_ucnt[uj] = __popcll(eq);
            s_uoff[uj] = less;
            s_tmask[uj] = tm;
        }
        const int U = o.U;
        int nc = 1;
        if (U > kDownChunkExperts || slots > slot_cap) {
            // greedy: a chunk takes experts while it holds at most
            // kDownChunkExperts of them and slot_cap h rows
            int c0 = 0, pA = 0;
            for (int u = 1; u < U; ++u) {
                const int src = __ffsll((unsigned long long)__ballot(first && uj == u)) - 1;
                const int end_u = __builtin_amdgcn_readlane(endj, src);
                if (u - c0 >= kDownChunkExperts || end_u - pA > slot_cap) {
                    if (lane == 0) s_cu[nc] = u;
                    ++nc;
                    c0 = u;
                    pA = __builtin_amdgcn_readlane(less, src);
                }
            }
        }
        if (lane == 0) {
            s_cu[0] = 0;
            s_cu[nc] = U;
            s_U = U;
            s_NC = nc;
        }
    }
    __syncthreads();
    const int NC = s_NC;

    // Lane l of a half-wave owns, in its row, the group pairs (64 p + 2 l,
    // 64 p + 2 l + 1), p < NP (one 16-byte code load each), and, when GPL2 is
    // odd, the single group 64 NP + l (one 8-byte load): every wave load is a
    // contiguous 512 B or 256 B run per row.  The row's scale bytes are
    // requested as whole dwords (lane m: dword m) and handed to their lanes
    // with ds_bpermute, so one expert costs NP + ODD + 1 vector loads per wave.
    constexpr int NP = GPL2 / 2, ODD = GPL2 & 1, NCHUNK = NP + ODD;
    constexpr int kLoadsPerExpert = (NCHUNK + 1) * kDownRows;
    uint32_t voc[R][NCHUNK], vos[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t nr = (uint32_t)min(n0 + r, H - 1);
#pragma unroll
        for (int p = 0; p < NCHUNK; ++p)
            voc[r][p] = nr * (uint32_t)(I / 2) + (uint32_t)(512 * p) + (uint32_t)l32 * (p < NP ? 16u : 8u);
        vos[r] = nr * (uint32_t)ngroups + 4u * (uint32_t)min(l32, 8 * GPL2 - 1);
    }
    int src_pair[NP > 0 ? NP : 1];
#pragma unroll
    for (int p = 0; p < NP; ++p) src_pair[p] = (half * 32 + 16 * p + (l32 >> 1)) * 4;
    const int src_single = (half * 32 + 16 * NP + (l32 >> 2)) * 4;
    const int sh_pair = 16 * (l32 & 1), sh_single = 8 * (l32 & 3);
    const int64_t code_stride = (int64_t)H * (I / 2), scale_stride = (int64_t)H * ngroups;


    float acc[MAXT][R];
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[t][r] = 0.0f;

    for (int c = 0; c < NC; ++c) {
        const int u0 = s_cu[c], u1 = s_cu[c + 1];
        const int pA = s_uoff[u0];
        const int pB = s_uoff[u1 - 1] + s_ucnt[u1 - 1];

        // h rows of the chunk straight to LDS (contiguous in sorted order).
        // Inside a row the 16-byte chunks are stored transposed to the order
        // in which the lanes read them: chunk 128 p + 4 l + i (pair p, lane l,
        // i < 4) at 128 p + 32 i + l, chunk 128 NP + 2 l + i at
        // 128 NP + 32 i + l, so that every LDS read of the loop is 32
        // consecutive 16-byte slots.  The DMA gathers: the lane that writes
        // slot P loads the chunk that belongs there.
        if (c > 0) __syncthreads();    // the previous chunk's LDS rows are no longer read
        {
            const int rc = 64 * GPL2;                      // 16-byte chunks per h row
            const int nq = (pB - pA) * GPL2;               // 1 KiB wave copies
            for (int q = wave; q < nq; q += waves) {
                const int slot = q * 64 + lane;
                const int row = slot / rc, P = slot - row * rc;
                const int blk = P >> 7, r = P & 127, i = r >> 5, l = r & 31;
                const int chunk = blk < NP ? 128 * blk + 4 * l + i : 128 * NP + 2 * l + i;
                const uint4* src = reinterpret_cast<const uint4*>(h + (int64_t)(pA + row) * I) + chunk;
                __builtin_amdgcn_global_load_lds(src, (lds_void*)(hs + q * 64), 16, 0, 0);
            }
        }
        // codes of every chunk slot (slots past the chunk re-read its last
        // expert, so the number of loads in flight is fixed); kDownAhead
        // experts are in flight while one is computed
        uint4 cw[kDownChunkExperts][R][NP > 0 ? NP : 1];
        uint2 cs[kDownChunkExperts][R];
        uint32_t sw[kDownChunkExperts][R];
        // each expert's global scale by a scalar load issued with its codes: a
        // vector load would sit in the same in-order queue as the weight and
        // h loads, and waiting for it would wait for them
        float gsc[kDownChunkExperts];
#define MOE_DOWN_LOAD(u)                                                                        \
        do {                                                                                    \
            const int e_ = __builtin_amdgcn_readfirstlane(s_list[min(u0 + (u), u1 - 1)]);       \
            gsc[u] = ((const __attribute__((address_space(4))) float*)dg)[e_];                   \
            const uint8_t* cb_ = dc + e_ * code_stride;                                         \
            const uint8_t* sb_ = ds + e_ * scale_stride;                                        \
            _Pragma("unroll") for (int r = 0; r < R; ++r) {                                     \
                _Pragma("unroll") for (int p = 0; p < NP; ++p)                                  \
                    cw[u][r][p] = load_stream16(reinterpret_cast<const uint4*>(cb_ + voc[r][p])); \
                if constexpr (ODD)                                                              \
                    cs[u][r] = load_stream8(reinterpret_cast<const uint2*>(cb_ + voc[r][NP]));   \
                sw[u][r] = load_stream(reinterpret_cast<const uint32_t*>(sb_ + vos[r]));        \
            }                                                                                   \
            asm volatile("" ::: "memory");  /* issue here, not at the first use */              \
        } while (0)
#pragma unroll
        for (int u = 0; u < kDownAhead; ++u) MOE_DOWN_LOAD(u);
        // this wave's h rows and its first expert's codes have landed
        wait_vmem_at_most<kLoadsPerExpert * (kDownAhead - 1)>();
        __builtin_amdgcn_s_barrier();   // plain barrier: a fence here would wait for every load

#pragma unroll
        for (int u = 0; u < kDownChunkExperts; ++u) {
            if (u + kDownAhead < kDownChunkExperts) MOE_DOWN_LOAD(u + kDownAhead);
            if (u0 + u < u1) {
                const float ge = gsc[u] * h_scale;
                const int q0 = s_uoff[u0 + u] - pA;
                float sp0[R][NP > 0 ? NP : 1], sp1[R][NP > 0 ? NP : 1], s1[R];
#pragma unroll
                for (int r = 0; r < R; ++r) {
#pragma unroll
                    for (int p = 0; p < NP; ++p) {
                        const uint32_t w =
                            (uint32_t)__builtin_amdgcn_ds_bpermute(src_pair[p], (int)sw[u][r]) >> sh_pair;
                        sp0[r][p] = e4m3_byte_to_f32<0>(w);
                        sp1[r][p] = e4m3_byte_to_f32<1>(w);
                    }
                    s1[r] = ODD ? e4m3_to_f32((uint32_t)__builtin_amdgcn_ds_bpermute(src_single, (int)sw[u][r]) >>
                                              sh_single)
                                : 0.0f;
                }
                // the expert's tokens in ascending order (its h rows q0, q0 + 1,
                // ...): a static loop over the token index with wave-uniform
                // branches, so each token's accumulator is a fixed register
                const uint32_t tmask = (uint32_t)__builtin_amdgcn_readfirstlane((int)s_tmask[u0 + u]);
                int q = q0;
#pragma unroll
                for (int t = 0; t < MAXT; ++t) {
                    if (!((tmask >> t) & 1u)) continue;
                    const float wgt = __builtin_bit_cast(
                        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, s_wgt[pA + q]))) * ge;
                    const uint4* hr = hs + q * I8 + l32;
                    float a[R];
#pragma unroll
                    for (int r = 0; r < R; ++r) a[r] = 0.0f;
#pragma unroll
                    for (int p = 0; p < NP; ++p) {
                        const uint4* hp = hr + 128 * p;
                        const uint4 x0 = hp[0], x1 = hp[32], x2 = hp[64], x3 = hp[96];
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            a[r] += sp0[r][p] * group_dot(make_uint2(cw[u][r][p].x, cw[u][r][p].y), x0, x1);
                            a[r] += sp1[r][p] * group_dot(make_uint2(cw[u][r][p].z, cw[u][r][p].w), x2, x3);
                        }
                    }
                    if constexpr (ODD) {
                        const uint4* hp = hr + 128 * NP;
                        const uint4 y0 = hp[0], y1 = hp[32];
#pragma unroll
                        for (int r = 0; r < R; ++r) a[r] += s1[r] * group_dot(cs[u][r], y0, y1);
                    }
#pragma unroll
                    for (int r = 0; r < R; ++r) acc[t][r] += wgt * a[r];
                    ++q;
                }
            }
        }
#undef MOE_DOWN_LOAD
    }
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float v = half_wave_sum_dpp(acc[t][r]);
            if (t < T && l32 == 0 && n0 + r < H) out[(int64_t)t * H + n0 + r] = f32_to_bf16_rne(v);
        }
}

// Stages of two features per gate/up wave.  One token: two stages, so the
// 768 workgroups of a 1536-feature, 8-expert layer are all resident at once
// (145 VGPRs, 3 waves per SIMD).  More tokens: one stage; the grid is then
// larger than one resident round anyway (a column per slot, most of them
// empty after the lookup), and smaller workgroups start streaming sooner
// (measured on MI355X at 8 tokens, 35 experts: 70 us against 75).
template <int CPL, int RW, int EPL, bool ROUTE, bool ONE = false, bool QH = false>
moe_status launch_gateup_epl(const FwdArgs& a, const GuRoute& R, hipStream_t s) {
    const int rows_per_block = kGuWaves * 2 * RW;
    const dim3 grid((a.I + rows_per_block - 1) / rows_per_block, std::min(a.T * a.k, a.E));
    const size_t shmem = (size_t)std::min(a.T, x_stage_tokens<false, ONE>()) * a.H * sizeof(uint16_t);
    auto kern = k_dec_gateup<CPL, RW, EPL, ROUTE, false, ONE, QH>;
    if (allow_dynamic_lds(reinterpret_cast<const void*>(kern), shmem) != MOE_OK) return MOE_ERR_HIP;
    MOE_LAUNCH(ROUTE ? "dec_gateup_route" : "dec_gateup", kern, grid, dim3(kGuThreads), shmem, s, a.x, a.H, a.I,
               a.E, a.k, a.T * a.k, (const uint8_t*)a.gate->codes, (const uint8_t*)a.gate->scales,
               (const float*)a.gate->global_scale, (const uint8_t*)a.up->codes, (const uint8_t*)a.up->scales,
               (const float*)a.up->global_scale, a.counts, a.sorted_slots, a.h, R, a.xs, QH ? nullptr : a.hf, a.hq);
    return MOE_OK;
}

template <int CPL, int RW>
moe_status launch_gateup_rw(const FwdArgs& a, const GuRoute* R, hipStream_t s) {
    if (R) return a.E <= 256 ? launch_gateup_epl<CPL, RW, 4, true>(a, *R, s) : launch_gateup_epl<CPL, RW, 16, true>(a, *R, s);
    const GuRoute none{};
    return a.E <= 256 ? launch_gateup_epl<CPL, RW, 4, false>(a, none, s)
                      : launch_gateup_epl<CPL, RW, 16, false>(a, none, s);
}

template <int CPL>
moe_status launch_gateup_gpl(const FwdArgs& a, const GuRoute* R, hipStream_t s, bool one) {
    if (one) return launch_gateup_epl<CPL, 1, 4, false, true>(a, GuRoute{}, s);
    if (a.hq > 0.0f) {      // W4A4, one token: 16-feature workgroups that quantize their own h groups
        if (a.T != 1) return MOE_ERR_UNSUPPORTED;
        if (R)
            return a.E <= 256 ? launch_gateup_epl<CPL, 2, 4, true, false, true>(a, *R, s)
                              : launch_gateup_epl<CPL, 2, 16, true, false, true>(a, *R, s);
        return a.E <= 256 ? launch_gateup_epl<CPL, 2, 4, false, false, true>(a, GuRoute{}, s)
                          : launch_gateup_epl<CPL, 2, 16, false, false, true>(a, GuRoute{}, s);
    }
    // two stages per wave when enough expert columns fill the chip with
    // resident workgroups; with one or two experts (a shared expert) one
    // stage, which doubles the workgroups streaming at once
    if (a.T == 1 && (R || std::min(a.T * a.k, a.E) >= 4)) return launch_gateup_rw<CPL, 2>(a, R, s);
    const GuRoute none{};     // the in-kernel route is for one token only
    return a.E <= 256 ? launch_gateup_epl<CPL, 1, 4, false>(a, none, s) : launch_gateup_epl<CPL, 1, 16, false>(a, none, s);
}

int down_waves_per_block(int H) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    // one workgroup per CU when the rows divide evenly: 2 * kDownRows rows per wave
    int w = (H + 2 * kDownRows * cus - 1) / (2 * kDownRows * cus);
    return std::max(1, std::min(w, kDownMaxWaves));
}

// h rows staged per chunk: the chunk size, at most T * k, within a 128 KiB
// LDS budget (an expert's rows, at most T <= 8, always fit: I <= 2048)
constexpr int kDownLdsBudget = 128 * 1024;

template <int GPL2, int MAXT, bool ONE>
moe_status launch_down_t(const FwdArgs& a, hipStream_t s) {
    const int waves = down_waves_per_block(a.H);
    const int rows_per_block = 2 * kDownRows * waves;
    const int slot_cap = std::min({down_chunk_slots<MAXT>(), a.T * a.k, kDownLdsBudget / (a.I * 2)});
    const size_t shmem = (size_t)slot_cap * a.I * sizeof(uint16_t);
    if (allow_dynamic_lds(reinterpret_cast<const void*>(&k_dec_down<GPL2, MAXT, ONE>), shmem) != MOE_OK)
        return MOE_ERR_HIP;
    MOE_LAUNCH("dec_down", (k_dec_down<GPL2, MAXT, ONE>), dim3((a.H + rows_per_block - 1) / rows_per_block),
               dim3(waves * kWave), shmem, s, (const uint16_t*)a.h, a.T, a.H, a.I, a.E, a.k,
               (const uint8_t*)a.down->codes, (const uint8_t*)a.down->scales, (const float*)a.down->global_scale,
               a.ids, a.topk_w, a.out, slot_cap, a.hs);
    return MOE_OK;
}

template <int GPL2, bool ONE>
moe_status launch_down_tt(const FwdArgs& a, hipStream_t s) {
    if (a.T <= 1) return launch_down_t<GPL2, 1, ONE>(a, s);
    if (a.T <= 2) return launch_down_t<GPL2, 2, ONE>(a, s);
    if (a.T <= 4) return launch_down_t<GPL2, 4, ONE>(a, s);
    return launch_down_t<GPL2, 8, ONE>(a, s);
}

template <int GPL2>
moe_status launch_down_gpl(const FwdArgs& a, hipStream_t s, bool one) {
    return one ? launch_down_tt<GPL2, true>(a, s) : launch_down_tt<GPL2, false>(a, s);
}

}  // namespace

bool decode_path_supported(int T, int k, int H, int I) {
    return T >= 1 && T <= 8 && T * k <= kDecodeMaxSlots && H % 1024 == 0 && H / 1024 <= 8 && I % 512 == 0 &&
           I / 512 <= 4;
}

namespace {

moe_status launch_decode_gateup_part(const FwdArgs& a, const GuRoute* R, hipStream_t s, bool one) {
    switch (a.H / 1024) {
        case 1: return launch_gateup_gpl<1>(a, R, s, one);
        case 2: return launch_gateup_gpl<2>(a, R, s, one);
        case 3: return launch_gateup_gpl<3>(a, R, s, one);
        case 4: return launch_gateup_gpl<4>(a, R, s, one);
        case 5: return launch_gateup_gpl<5>(a, R, s, one);
        case 6: return launch_gateup_gpl<6>(a, R, s, one);
        case 7: return launch_gateup_gpl<7>(a, R, s, one);
        case 8: return launch_gateup_gpl<8>(a, R, s, one);
        default: return MOE_ERR_UNSUPPORTED;
    }
}

moe_status launch_decode_down_part(const FwdArgs& a, hipStream_t s, bool one) {
    switch (a.I / 512) {
        case 1: return launch_down_gpl<1>(a, s, one);
        case 2: return launch_down_gpl<2>(a, s, one);
        case 3: return launch_down_gpl<3>(a, s, one);
        case 4: return launch_down_gpl<4>(a, s, one);
        default: return MOE_ERR_UNSUPPORTED;
    }
}

moe_status launch_decode_pair(const FwdArgs& a, const GuRoute* R, hipStream_t s, bool one = false) {
    const moe_status st = launch_decode_gateup_part(a, R, s, one);
    if (st != MOE_OK) return st;
    return launch_decode_down_part(a, s, one);
}

}  // namespace

moe_status launch_forward_decode_gateup(const FwdArgs& a, hipStream_t s) {
    return launch_decode_gateup_part(a, nullptr, s, false);
}
moe_status launch_forward_decode_down(const FwdArgs& a, hipStream_t s) { return launch_decode_down_part(a, s, false); }

moe_status launch_forward_decode_gateup_routed(const FwdArgs& a, const float* logits, int32_t* ids, float* w,
                                               int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* pos,
                                               hipStream_t s) {
    if (a.T != 1) return MOE_ERR_UNSUPPORTED;
    const GuRoute R{logits, ids, w, counts, offsets, sorted, pos};
    return launch_decode_gateup_part(a, &R, s, false);
}

moe_status launch_forward_decode(const FwdArgs& a, hipStream_t s) { return launch_decode_pair(a, nullptr, s); }

moe_status launch_forward_decode_one(const FwdArgs& a, hipStream_t s) {
    if (a.E != 1 || a.k != 1) return MOE_ERR_UNSUPPORTED;
    return launch_decode_pair(a, nullptr, s, true);
}

namespace {

template <int CPL, int RW>
moe_status launch_linear_rw(const FwdArgs& a, hipStream_t s) {
    const int rows_per_block = kGuWaves * 2 * RW;
    const dim3 grid((a.I + rows_per_block - 1) / rows_per_block, 1);
    const size_t shmem = (size_t)std::min(a.T, kXTokensLinear) * a.H * sizeof(uint16_t);
    auto kern = k_dec_gateup<CPL, RW, 4, false, true>;
    if (allow_dynamic_lds(reinterpret_cast<const void*>(kern), shmem) != MOE_OK) return MOE_ERR_HIP;
    const GuRoute none{};
    MOE_LAUNCH("dec_linear", kern, grid, dim3(kGuThreads), shmem, s, a.x, a.H, a.I, 1, 1, a.T,
               (const uint8_t*)a.gate->codes, (const uint8_t*)a.gate->scales, (const float*)a.gate->global_scale,
               (const uint8_t*)a.gate->codes, (const uint8_t*)a.gate->scales, (const float*)a.gate->global_scale,
               a.counts, a.sorted_slots, a.h, none, 1.0f, (float*)nullptr, 0.0f);
    return MOE_OK;
}

template <int CPL>
moe_status launch_linear_cpl(const FwdArgs& a, hipStream_t s) {
    return launch_linear_rw<CPL, 1>(a, s);   // one stack: one stage per wave, twice the workgroups
}

}  // namespace

bool linear_decode_supported(int T, int K, int N) {
    return T >= 1 && T <= 8 && K % 1024 == 0 && K / 1024 >= 1 && K / 1024 <= 8 && N >= 2;
}

moe_status launch_linear_decode(const FwdArgs& a, hipStream_t s) {
    if (a.E != 1 || a.k != 1 || !linear_decode_supported(a.T, a.H, a.I)) return MOE_ERR_UNSUPPORTED;
    switch (a.H / 1024) {
        case 1: return launch_linear_cpl<1>(a, s);
        case 2: return launch_linear_cpl<2>(a, s);
        case 3: return launch_linear_cpl<3>(a, s);
        case 4: return launch_linear_cpl<4>(a, s);
        case 5: return launch_linear_cpl<5>(a, s);
        case 6: return launch_linear_cpl<6>(a, s);
        case 7: return launch_linear_cpl<7>(a, s);
        case 8: return launch_linear_cpl<8>(a, s);
        default: return MOE_ERR_UNSUPPORTED;
    }
}

moe_status launch_forward_decode_routed(const FwdArgs& a, const float* logits, int32_t* ids, float* w,
                                        int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* pos,
                                        hipStream_t s) {
    if (a.T != 1) return MOE_ERR_UNSUPPORTED;
    const GuRoute R{logits, ids, w, counts, offsets, sorted, pos};
    return launch_decode_pair(a, &R, s);
}

}  // namespace moe
