// NVFP4 rounding and the per-group quantization of activations, shared by
// the activation quantizer (quantize.hip) and the decode gate/up kernel, which
// quantizes its own output groups in the W4A4 variant.  Every step is one
// correctly rounded fp32 operation in a fixed order (the library is built
// with correctly rounded division and without denormal flushing; no
// contraction in these functions), so that every caller gets the same bits.
#pragma once

#include "device_common.h"

namespace moe {

// Round a non-negative fp32 value to the nearest E4M3 byte, ties to even,
// saturating at 448 (0x7E).  Works on the integer significand: the value is
// scaled by a power of two (exact) so that its E4M3 grid step becomes 1, then
// rounded half-to-even.
__device__ __forceinline__ uint32_t e4m3_encode_rne_sat(float x) {
#pragma clang fp contract(off)
    if (!(x < 448.0f)) return 0x7Eu;                       // also NaN -> saturate
    if (x < 0x1p-6f) return (uint32_t)rintf(x * 512.0f);   // subnormal grid 2^-9
    const int e = (int)((__float_as_uint(x) >> 23) & 0xFF) - 127;   // -6..8
    const float q = x * __uint_as_float((uint32_t)(127 + 3 - e) << 23);  // [8, 16)
    const uint32_t code = (uint32_t)((e + 7) << 3) + (uint32_t)rintf(q) - 8u;
    return code > 0x7Eu ? 0x7Eu : code;
}

// Nearest E2M1 code of q (ties to the even code, saturating at 6), sign bit
// copied from q.  The decision points are the midpoints between neighbouring
// magnitudes; ">=" where the upper neighbour has the even code.
__device__ __forceinline__ uint32_t e2m1_encode_rne_sat(float q) {
    const float a = fabsf(q);
    const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                       (uint32_t)(a > 5.0f);
    return c | ((__float_as_uint(q) >> 31) << 3);
}

// One 16-group of activations quantized to NVFP4 under a static per-tensor
// input scale, exactly like a weight group under its global scale:
//   s = E4M3((amax / 6) / input_scale),  code = E2M1(v / (E4M3(s) * input_scale));
// a group whose E4M3(s) * input_scale is 0 gets magnitude-0 codes with the
// values' signs.  nvfp4_group_scale gives the scale byte and its value from
// the group's amax, nvfp4_code one element's code; nvfp4_group_codes does a
// whole group in one thread (returns the scale byte; the codes go to c).
__device__ __forceinline__ uint32_t nvfp4_group_scale(float amax, float input_scale, float& s_q) {
#pragma clang fp contract(off)
    const float s_f = (amax / 6.0f) / input_scale;
    const uint32_t sb = e4m3_encode_rne_sat(s_f);
    s_q = e4m3_to_f32(sb);
    return sb;
}
__device__ __forceinline__ uint32_t nvfp4_code(float v, float s_q, float input_scale) {
#pragma clang fp contract(off)
    const float d = s_q * input_scale;
    return (d == 0.0f) ? ((__float_as_uint(v) >> 31) << 3) : e2m1_encode_rne_sat(v / d);
}
__device__ __forceinline__ uint32_t nvfp4_group_codes(const float (&v)[16], float input_scale, uint32_t (&c)[16]) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    float s_q;
    const uint32_t sb = nvfp4_group_scale(amax, input_scale, s_q);
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = nvfp4_code(v[i], s_q, input_scale);
    return sb;
}

// The group's NVFP4 values E2M1(code) * E4M3(s), without the input scale, as
// 8 bf16 pairs (element 2i in the low half of o[i]): exact, at most 6
// significant bits; the consumer applies the input scale in its epilogue.
__device__ __forceinline__ void nvfp4_group_values_bf16(const float (&v)[16], float input_scale, uint32_t (&o)[8]) {
#pragma clang fp contract(off)
    uint32_t c[16];
    const float s_q = e4m3_to_f32(nvfp4_group_codes(v, input_scale, c));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const floatx2 f = e2m1x2_to_f32<0>(c[2 * i] | (c[2 * i + 1] << 4));
        o[i] = pack_bf16x2_exact(f[0] * s_q, f[1] * s_q);
    }
}

// One element of a group whose 16 elements sit in 16 consecutive lanes
// (lanes 16 j .. 16 j + 15 of a wave, all active): the group's NVFP4 value
// for this lane's v, E2M1(code) * E4M3(s) without the input scale, as bf16
// bits (exact).  The same steps as nvfp4_group_codes, one element per lane.
__device__ __forceinline__ uint16_t nvfp4_lane_value_bf16(float v, float input_scale) {
#pragma clang fp contract(off)
    float amax = fabsf(v);
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
    float s_q;
    (void)nvfp4_group_scale(amax, input_scale, s_q);
    const uint32_t c = nvfp4_code(v, s_q, input_scale);
    const floatx2 f = e2m1x2_to_f32<0>(c);
    return (uint16_t)(__float_as_uint(f[0] * s_q) >> 16);
}

}  // namespace moe
