// NVFP4 weight-only quantization, the dequantization test hook and the
// validation scan (load time; not on the hot path).
//
// The pages describe a calibration-free, deterministic weight-only NVFP4
// conversion with group size 16 and a FP32 per-tensor second-level scale
// ("GLM-5.3-Flash NVFP4 W4A16 for 2x RTX PRO 6000 Blackwell", intro;
// "GLM-5.3-Flash-NVFP4-h -- W4A16 dense-side quantization", "Config
// expectations").  The scale arithmetic is fixed here as
//   g = amax|W| / 2688 (1 if that is 0),  s = E4M3((amax_group / 6) / g),
//   code = E2M1(W / (E4M3(s) * g)),
// every step one correctly rounded fp32 operation, in that order, so that a
// different order cannot flip a scale byte.  The library is built with
// correctly rounded fp32 division and without denormal flushing, and
// contraction is off in this file.
#include "device_common.h"
#include "internal.h"
#include "quant_common.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

constexpr int kQBlock = 256;

__device__ __forceinline__ float global_scale_from_amax(uint32_t amax_bits) {
    const float g = __uint_as_float(amax_bits) / 2688.0f;
    return (g > 0.0f) ? g : 1.0f;  // all-zero (or underflowing) tensor
}

__global__ void k_amax_clear(uint32_t* amax_bits, int E) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e < E) amax_bits[e] = 0u;
}

// |W| maximum per expert.  Non-negative fp32 values order like their bit
// patterns, so an unsigned atomic max gives the exact maximum in any order.
__global__ void __launch_bounds__(kQBlock) k_amax(const float* __restrict__ w, int64_t per_expert,
                                                  uint32_t* amax_bits) {
    const int e = blockIdx.y;
    const float4* src = reinterpret_cast<const float4*>(w + (int64_t)e * per_expert);
    const int64_t n4 = per_expert / 4;
    uint32_t m = 0;
    for (int64_t i = (int64_t)blockIdx.x * kQBlock + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kQBlock) {
        const float4 v = src[i];
        m = max(m, __float_as_uint(v.x) & 0x7FFFFFFFu);
        m = max(m, __float_as_uint(v.y) & 0x7FFFFFFFu);
        m = max(m, __float_as_uint(v.z) & 0x7FFFFFFFu);
        m = max(m, __float_as_uint(v.w) & 0x7FFFFFFFu);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, kWave));
    __shared__ uint32_t red[kQBlock / kWave];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < kQBlock / kWave; ++i) m = max(m, red[i]);
        atomicMax(amax_bits + e, m);
    }
}

// One thread per 16-group: group scale byte and 16 codes (8 bytes).
__global__ void __launch_bounds__(kQBlock) k_quant_groups(const float* __restrict__ w, int64_t groups_per_expert,
                                                          const uint32_t* __restrict__ amax_bits,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const int e = blockIdx.y;
    const int64_t gi = (int64_t)blockIdx.x * kQBlock + threadIdx.x;
    if (gi >= groups_per_expert) return;
    const int64_t gidx = (int64_t)e * groups_per_expert + gi;
    const float g = global_scale_from_amax(amax_bits[e]);

    const float4* src = reinterpret_cast<const float4*>(w) + gidx * 4;
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 q = src[i];
        v[4 * i + 0] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));

    const float s_f = (amax / 6.0f) / g;
    const uint32_t sb = e4m3_encode_rne_sat(s_f);
    const float d = e4m3_to_f32(sb) * g;

    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t c = (d == 0.0f) ? ((__float_as_uint(v[i]) >> 31) << 3) : e2m1_encode_rne_sat(v[i] / d);
        if (i < 8) lo |= c << (4 * i);
        else hi |= c << (4 * (i - 8));
    }
    reinterpret_cast<uint2*>(codes)[gidx] = make_uint2(lo, hi);
    scales[gidx] = (uint8_t)sb;
}

__global__ void k_amax_to_global(uint32_t* amax_bits_then_g, int E) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e < E) {
        const float g = global_scale_from_amax(amax_bits_then_g[e]);
        reinterpret_cast<float*>(amax_bits_then_g)[e] = g;
    }
}

// Test hook: (E2M1 * E4M3) * g in fp32 with the forward's decode routines.
__global__ void __launch_bounds__(kQBlock) k_dequant(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                     const float* __restrict__ gscale, int64_t groups_per_expert,
                                                     float* __restrict__ out) {
    const int e = blockIdx.y;
    const int64_t gi = (int64_t)blockIdx.x * kQBlock + threadIdx.x;
    if (gi >= groups_per_expert) return;
    const int64_t gidx = (int64_t)e * groups_per_expert + gi;
    const uint2 c = reinterpret_cast<const uint2*>(codes)[gidx];
    const float s = e4m3_to_f32(scales[gidx]);
    const float g = gscale[e];
    float r[16];
    const uint32_t words[2] = {c.x, c.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        floatx2 p0 = e2m1x2_to_f32<0>(words[h]);
        floatx2 p1 = e2m1x2_to_f32<1>(words[h]);
        floatx2 p2 = e2m1x2_to_f32<2>(words[h]);
        floatx2 p3 = e2m1x2_to_f32<3>(words[h]);
        const float cv[8] = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
        for (int i = 0; i < 8; ++i) r[8 * h + i] = (cv[i] * s) * g;
    }
    float4* dst = reinterpret_cast<float4*>(out) + gidx * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_float4(r[4 * i], r[4 * i + 1], r[4 * i + 2], r[4 * i + 3]);
}

// Flags: bit 0 = non-finite global scale, bit 1 = global scale <= 0,
// bit 2 = NaN E4M3 scale byte.
__global__ void __launch_bounds__(kQBlock) k_validate(const uint8_t* __restrict__ scales, int64_t nbytes,
                                                      const float* __restrict__ gscale, int E, uint32_t* flag) {
    uint32_t f = 0;
    const int64_t tid = (int64_t)blockIdx.x * kQBlock + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kQBlock;
    if (tid < E) {
        const float g = gscale[tid];
        if (!isfinite(g)) f |= 1u;
        else if (!(g > 0.0f)) f |= 2u;
    }
    const int64_t n16 = nbytes / 16;
    for (int64_t i = tid; i < n16; i += stride) {
        const uint4 v = reinterpret_cast<const uint4*>(scales)[i];
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t x = wd[j] & 0x7F7F7F7Fu;
            // a byte equals 0x7F iff (x ^ 0x7F...) has a zero byte
            const uint32_t y = x ^ 0x7F7F7F7Fu;
            if (((y - 0x01010101u) & ~y & 0x80808080u) != 0u) f |= 4u;
        }
    }
    for (int64_t i = n16 * 16 + tid; i < nbytes; i += stride)
        if ((scales[i] & 0x7Fu) == 0x7Fu) f |= 4u;
    if (f) atomicOr(flag, f);
}

// Clears n words with vector stores (a fill kernel, not a memset node, so
// that it is safe inside a captured graph).
__global__ void k_zero_words(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// ---- W4A4: activations quantized like the weights, with a static input
// scale in the place of the global scale ("GLM-5.3-Flash-NVFP4-h", opening:
// the routed experts' stock W4A4 quantization; "GLM-5.3-Flash · 512k + MTP +
// vision ...", "Input-scales provenance": the per-tensor input_scale).  One
// thread per 16-group of a row:
//   s = E4M3((amax / 6) / input_scale),  code = E2M1(v / (E4M3(s) * input_scale)),
// the same correctly rounded fp32 steps as the weights.  Output either the
// packed codes and scale bytes (the canonical activation layout), or the
// group's values E2M1(code) * E4M3(s) as bf16 -- exact (at most 6
// significant bits) and without the input scale, which the GEMM epilogue
// applies with the weight's global scale.
template <bool IN_F32, bool PACKED>
__global__ void __launch_bounds__(kQBlock) k_quant_act(const void* __restrict__ in, int64_t groups, float input_scale,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                       uint16_t* __restrict__ deq) {
    const int64_t gi = (int64_t)blockIdx.x * kQBlock + threadIdx.x;
    if (gi >= groups) return;
    float v[16];
    if constexpr (IN_F32) {
        const float4* src = reinterpret_cast<const float4*>(in) + gi * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 q = src[i];
            v[4 * i + 0] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
        }
    } else {
        const uint4* src = reinterpret_cast<const uint4*>(in) + gi * 2;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint4 q = src[i];
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * i + 2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
                v[8 * i + 2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
            }
        }
    }
    if constexpr (PACKED) {
        uint32_t c[16];
        const uint32_t sb = nvfp4_group_codes(v, input_scale, c);
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            lo |= c[i] << (4 * i);
            hi |= c[8 + i] << (4 * i);
        }
        reinterpret_cast<uint2*>(codes)[gi] = make_uint2(lo, hi);
        scales[gi] = (uint8_t)sb;
    } else {
        uint32_t o[8];
        nvfp4_group_values_bf16(v, input_scale, o);
        uint4* dst = reinterpret_cast<uint4*>(deq) + gi * 2;
        dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
}

inline int blocks_for(int64_t n, int per) { return (int)((n + per - 1) / per); }

}  // namespace

moe_status launch_quant_act(const void* in, bool in_f32, int64_t rows, int K, float input_scale, uint8_t* codes,
                            uint8_t* scales, uint16_t* deq, hipStream_t s) {
    const int64_t groups = rows * (K / 16);
    if (groups == 0) return MOE_OK;
    const dim3 grid(blocks_for(groups, kQBlock));
    if (codes) {
        if (in_f32)
            MOE_LAUNCH("quant_act", (k_quant_act<true, true>), grid, dim3(kQBlock), 0, s, in, groups, input_scale,
                       codes, scales, deq);
        else
            MOE_LAUNCH("quant_act", (k_quant_act<false, true>), grid, dim3(kQBlock), 0, s, in, groups, input_scale,
                       codes, scales, deq);
    } else if (in_f32) {
        MOE_LAUNCH("quant_act", (k_quant_act<true, false>), grid, dim3(kQBlock), 0, s, in, groups, input_scale,
                   codes, scales, deq);
    } else {
        MOE_LAUNCH("quant_act", (k_quant_act<false, false>), grid, dim3(kQBlock), 0, s, in, groups, input_scale,
                   codes, scales, deq);
    }
    return MOE_OK;
}

moe_status launch_quantize_pack(const float* w, int E, int N, int K, const moe_nvfp4_tensor* out,
                                hipStream_t s) {
    uint32_t* amax = reinterpret_cast<uint32_t*>(out->global_scale);
    const int64_t per_expert = (int64_t)N * K;
    const int64_t groups = per_expert / 16;
    MOE_LAUNCH("quant_amax_clear", k_amax_clear, dim3(blocks_for(E, 256)), dim3(256), 0, s, amax, E);
    const int ablocks = (int)std::min<int64_t>(std::max<int64_t>(blocks_for(per_expert / 4, kQBlock), 1), 256);
    MOE_LAUNCH("quant_amax", k_amax, dim3(ablocks, E), dim3(kQBlock), 0, s, w, per_expert, amax);
    MOE_LAUNCH("quant_groups", k_quant_groups, dim3(blocks_for(groups, kQBlock), E), dim3(kQBlock), 0, s, w,
               groups, (const uint32_t*)amax, out->codes, out->scales);
    MOE_LAUNCH("quant_finalize", k_amax_to_global, dim3(blocks_for(E, 256)), dim3(256), 0, s, amax, E);
    return MOE_OK;
}

moe_status launch_dequantize(const moe_nvfp4_tensor* t, float* w_out, hipStream_t s) {
    const int64_t groups = (int64_t)t->N * t->K / 16;
    MOE_LAUNCH("dequantize", k_dequant, dim3(blocks_for(groups, kQBlock), t->E), dim3(kQBlock), 0, s,
               (const uint8_t*)t->codes, (const uint8_t*)t->scales, (const float*)t->global_scale, groups, w_out);
    return MOE_OK;
}

moe_status launch_zero_words(uint32_t* p, int n, hipStream_t s) {
    if (n <= 0) return MOE_OK;
    MOE_LAUNCH("zero_words", k_zero_words, dim3(blocks_for(n, kQBlock)), dim3(kQBlock), 0, s, p, n);
    return MOE_OK;
}

moe_status launch_validate(const moe_nvfp4_tensor* t, uint32_t* d_flag, hipStream_t s) {
    const int64_t nbytes = (int64_t)t->E * t->N * (t->K / 16);
    const int blocks = (int)std::min<int64_t>(std::max<int64_t>(blocks_for(nbytes / 16, kQBlock),
                                                                blocks_for(t->E, kQBlock)), 4096);
    MOE_LAUNCH("validate", k_validate, dim3(std::max(blocks, 1)), dim3(kQBlock), 0, s,
               (const uint8_t*)t->scales, nbytes, (const float*)t->global_scale, t->E, d_flag);
    return MOE_OK;
}

}  // namespace moe
