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
// Two kernels:
//   k_dec_gateup: one workgroup per (touched expert, block of rows of I).
//     Lanes split K: lane l owns the 16-groups l, l+64, ... of every row, so
//     each wave load is a contiguous 512 B run of codes and its x chunk is
//     loaded once and reused for every row the wave owns.  Codes decode to
//     bf16 pairs (gfx950 FP4 conversion) and meet x in v_dot2_f32_bf16; the
//     group scale multiplies each 16-term partial sum, the global scale the
//     row total.  SwiGLU runs on the reduced gate/up pair; h is rounded once
//     to bf16 and stored in expert-sorted row order.
//   k_dec_down: one wave per 2 output rows of H, looping over every touched
//     expert in ascending order and every token of that expert, so the
//     routing-weighted combine happens in registers (fp32, fixed order, no
//     atomics) and out is written once in bf16.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kDecWaves = 4;            // waves per gate/up workgroup
constexpr int kDecRows = 2;             // rows of I per gate/up wave
constexpr int kDownExpertChunk = 8;     // experts whose weights are in flight together

// Dot of 8 bf16 pairs (one 16-group of x) with the 16 codes of a group,
// unscaled: codes decode to exact bf16 pairs, v_dot2 accumulates in fp32.
__device__ __forceinline__ float group_dot(uint2 codes, const uint32_t* xw) {
    float acc = 0.0f;
    acc = dot2_bf16(__builtin_bit_cast(uint32_t, e2m1x2_to_bf16<0>(codes.x)), xw[0], acc);
    acc = dot2_bf16(__builtin_bit_cast(uint32_t, e2m1x2_to_bf16<1>(codes.x)), xw[1], acc);
    acc = dot2_bf16(__builtin_bit_cast(uint32_t, e2m1x2_to_bf16<2>(codes.x)), xw[2], acc);
    acc = dot2_bf16(__builtin_bit_cast(uint32_t, e2m1x2_to_bf16<3>(codes.x)), xw[3], acc);
    acc = dot2_bf16(__builtin_bit_cast(uint32_t, e2m1x2_to_bf16<0>(codes.y)), xw[4], acc);
    acc = dot2_bf16(__builtin_bit_cast(uint32_t, e2m1x2_to_bf16<1>(codes.y)), xw[5], acc);
    acc = dot2_bf16(__builtin_bit_cast(uint32_t, e2m1x2_to_bf16<2>(codes.y)), xw[6], acc);
    acc = dot2_bf16(__builtin_bit_cast(uint32_t, e2m1x2_to_bf16<3>(codes.y)), xw[7], acc);
    return acc;
}

// GPL = 16-groups per lane along H (H = 1024 * GPL).
template <int GPL>
__global__ void __launch_bounds__(kDecWaves * kWave)
k_dec_gateup(const uint16_t* __restrict__ x, int H, int I, int E, int k,
             const uint8_t* __restrict__ gc, const uint8_t* __restrict__ gs, const float* __restrict__ gg,
             const uint8_t* __restrict__ uc, const uint8_t* __restrict__ us, const float* __restrict__ ug,
             const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
             const int32_t* __restrict__ sorted_slots, uint16_t* __restrict__ h) {
    const int e = nth_active_expert(counts, E, blockIdx.y);
    if (e < 0) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int n0 = (blockIdx.x * kDecWaves + wave) * kDecRows;
    const int ngroups = H / 16;

    // Issue every weight load of this wave first.
    uint2 cw[2][kDecRows][GPL];
    uint32_t sw[2][kDecRows][GPL];
#pragma unroll
    for (int r = 0; r < kDecRows; ++r) {
        const int64_t row = (int64_t)e * I + n0 + r;
#pragma unroll
        for (int j = 0; j < GPL; ++j) {
            const int g = lane + kWave * j;
            cw[0][r][j] = reinterpret_cast<const uint2*>(gc + row * (H / 2))[g];
            cw[1][r][j] = reinterpret_cast<const uint2*>(uc + row * (H / 2))[g];
            sw[0][r][j] = gs[row * ngroups + g];
            sw[1][r][j] = us[row * ngroups + g];
        }
    }
    const float g_gate = gg[e], g_up = ug[e];
    const int p0 = offsets[e];
    const int ne = counts[e];
    float sc[2][kDecRows][GPL];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int r = 0; r < kDecRows; ++r)
#pragma unroll
            for (int j = 0; j < GPL; ++j) sc[p][r][j] = e4m3_to_f32(sw[p][r][j]);

    for (int q = 0; q < ne; ++q) {
        const int slot = sorted_slots[p0 + q];
        const int t = slot / k;
        const uint16_t* xr = x + (int64_t)t * H;
        uint32_t xw[GPL][8];
#pragma unroll
        for (int j = 0; j < GPL; ++j) {
            const uint4* src = reinterpret_cast<const uint4*>(xr + (lane + kWave * j) * 16);
            const uint4 a = src[0], b = src[1];
            xw[j][0] = a.x; xw[j][1] = a.y; xw[j][2] = a.z; xw[j][3] = a.w;
            xw[j][4] = b.x; xw[j][5] = b.y; xw[j][6] = b.z; xw[j][7] = b.w;
        }
        float acc[2][kDecRows];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int r = 0; r < kDecRows; ++r) {
                float a = 0.0f;
#pragma unroll
                for (int j = 0; j < GPL; ++j) a += sc[p][r][j] * group_dot(cw[p][r][j], xw[j]);
                acc[p][r] = wave_sum(a);
            }
        if (lane < kDecRows) {
            float av = acc[0][0], bv = acc[1][0];
#pragma unroll
            for (int r = 1; r < kDecRows; ++r)
                if (lane == r) { av = acc[0][r]; bv = acc[1][r]; }
            const float hv = silu(g_gate * av) * (g_up * bv);
            h[(int64_t)(p0 + q) * I + n0 + lane] = f32_to_bf16_rne(hv);
        }
    }
}

// GPL2 = 16-groups per half-wave lane along I (I = 512 * GPL2); MAXT tokens.
template <int GPL2, int MAXT>
__global__ void __launch_bounds__(kWave)
k_dec_down(const uint16_t* __restrict__ h, int T, int H, int I, int E, int k,
           const uint8_t* __restrict__ dc, const uint8_t* __restrict__ ds, const float* __restrict__ dg,
           const float* __restrict__ topk_w, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
           const int32_t* __restrict__ sorted_slots, uint16_t* __restrict__ out) {
    __shared__ int s_list[MOE_MAX_EXPERTS];
    const int lane = threadIdx.x;
    const int half = lane >> 5, l32 = lane & 31;
    const int n = blockIdx.x * 2 + half;           // output row of H
    const int ngroups = I / 16;

    // Compact list of touched experts, ascending.
    int U = 0;
    for (int base = 0; base < E; base += kWave) {
        const int e = base + lane;
        const bool act = e < E && counts[e] > 0;
        const uint64_t m = __ballot(act);
        if (act) s_list[U + __popcll(m & lanemask_lt())] = e;
        U += __popcll(m);
    }
    __syncthreads();

    float acc[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) acc[t] = 0.0f;

    for (int u0 = 0; u0 < U; u0 += kDownExpertChunk) {
        const int nu = min(kDownExpertChunk, U - u0);
        uint2 cw[kDownExpertChunk][GPL2];
        uint32_t sw[kDownExpertChunk][GPL2];
#pragma unroll
        for (int u = 0; u < kDownExpertChunk; ++u) {
            if (u < nu) {
                const int e = s_list[u0 + u];
                const int64_t row = (int64_t)e * H + n;
#pragma unroll
                for (int j = 0; j < GPL2; ++j) {
                    const int g = l32 + 32 * j;
                    cw[u][j] = reinterpret_cast<const uint2*>(dc + row * (I / 2))[g];
                    sw[u][j] = ds[row * ngroups + g];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kDownExpertChunk; ++u) {
            if (u < nu) {
                const int e = s_list[u0 + u];
                const float ge = dg[e];
                const int p0 = offsets[e], ne = counts[e];
                float sc[GPL2];
#pragma unroll
                for (int j = 0; j < GPL2; ++j) sc[j] = e4m3_to_f32(sw[u][j]);
                for (int q = 0; q < ne; ++q) {
                    const int slot = sorted_slots[p0 + q];
                    const int t = slot / k;
                    const float wgt = topk_w[slot] * ge;
                    const uint16_t* hr = h + (int64_t)(p0 + q) * I;
                    float a = 0.0f;
#pragma unroll
                    for (int j = 0; j < GPL2; ++j) {
                        const uint4* src = reinterpret_cast<const uint4*>(hr + (l32 + 32 * j) * 16);
                        const uint4 va = src[0], vb = src[1];
                        const uint32_t hw[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
                        a += sc[j] * group_dot(cw[u][j], hw);
                    }
#pragma unroll
                    for (int tt = 0; tt < MAXT; ++tt)
                        if (tt == t) acc[tt] += wgt * a;
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
        const float v = half_wave_sum(acc[t]);
        if (t < T && l32 == 0) out[(int64_t)t * H + n] = f32_to_bf16_rne(v);
    }
}

template <int GPL>
moe_status launch_gateup_gpl(const FwdArgs& a, hipStream_t s) {
    const dim3 grid(a.I / (kDecWaves * kDecRows), std::min(a.T * a.k, a.E));
    MOE_LAUNCH("dec_gateup", k_dec_gateup<GPL>, grid, dim3(kDecWaves * kWave), 0, s, a.x, a.H, a.I, a.E, a.k,
               (const uint8_t*)a.gate->codes, (const uint8_t*)a.gate->scales, (const float*)a.gate->global_scale,
               (const uint8_t*)a.up->codes, (const uint8_t*)a.up->scales, (const float*)a.up->global_scale,
               a.counts, a.offsets, a.sorted_slots, a.h);
    return MOE_OK;
}

template <int GPL2, int MAXT>
moe_status launch_down_t(const FwdArgs& a, hipStream_t s) {
    MOE_LAUNCH("dec_down", (k_dec_down<GPL2, MAXT>), dim3(a.H / 2), dim3(kWave), 0, s, (const uint16_t*)a.h, a.T,
               a.H, a.I, a.E, a.k, (const uint8_t*)a.down->codes, (const uint8_t*)a.down->scales,
               (const float*)a.down->global_scale, a.topk_w, a.counts, a.offsets, a.sorted_slots, a.out);
    return MOE_OK;
}

template <int GPL2>
moe_status launch_down_gpl(const FwdArgs& a, hipStream_t s) {
    if (a.T <= 1) return launch_down_t<GPL2, 1>(a, s);
    if (a.T <= 2) return launch_down_t<GPL2, 2>(a, s);
    if (a.T <= 4) return launch_down_t<GPL2, 4>(a, s);
    return launch_down_t<GPL2, 8>(a, s);
}

}  // namespace

bool decode_path_supported(int T, int H, int I) {
    return T >= 1 && T <= 8 && H % 1024 == 0 && H / 1024 <= 8 && I % 512 == 0 && I / 512 <= 4 &&
           I % (kDecWaves * kDecRows) == 0;
}

moe_status launch_forward_decode(const FwdArgs& a, hipStream_t s) {
    moe_status st;
    switch (a.H / 1024) {
        case 1: st = launch_gateup_gpl<1>(a, s); break;
        case 2: st = launch_gateup_gpl<2>(a, s); break;
        case 3: st = launch_gateup_gpl<3>(a, s); break;
        case 4: st = launch_gateup_gpl<4>(a, s); break;
        case 5: st = launch_gateup_gpl<5>(a, s); break;
        case 6: st = launch_gateup_gpl<6>(a, s); break;
        case 7: st = launch_gateup_gpl<7>(a, s); break;
        case 8: st = launch_gateup_gpl<8>(a, s); break;
        default: return MOE_ERR_UNSUPPORTED;
    }
    if (st != MOE_OK) return st;
    switch (a.I / 512) {
        case 1: return launch_down_gpl<1>(a, s);
        case 2: return launch_down_gpl<2>(a, s);
        case 3: return launch_down_gpl<3>(a, s);
        case 4: return launch_down_gpl<4>(a, s);
        default: return MOE_ERR_UNSUPPORTED;
    }
}

}  // namespace moe
