// Device-side helpers shared by the HIP kernels of libmoe_w4a16 (gfx950).
//
// Format facts used here (the pages name NVFP4 with group size 16 and a FP32
// per-tensor scale -- "GLM-5.3-Flash-NVFP4-h -- W4A16 dense-side
// quantization", "Config expectations"; the bit layouts are those of the OCP
// Microscaling v1.0 FP4 E2M1 and OCP 8-bit E4M3 "FN" formats):
//   E2M1: s e1 e0 m, values +-{0, .5, 1, 1.5, 2, 3, 4, 6}
//   E4M3: s eeee mmm, bias 7, subnormal m * 2^-9, max 448, 0x7F/0xFF NaN
// Every E2M1 * E4M3 product has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in bf16 and in fp32: weights reach the
// matrix units without rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float floatx2 __attribute__((__vector_size__(2 * sizeof(float))));
typedef float floatx4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));

constexpr int kWave = 64;

// ---------------------------------------------------------------- decode
// Two E2M1 codes held in byte SEL of `word` (low nibble first) -> two fp32
// values, exactly.  gfx950's scaled FP4 conversion with a unit scale is a
// plain format conversion.
template <int SEL>
__device__ __forceinline__ floatx2 e2m1x2_to_f32(uint32_t word) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
}

// Same, straight to a packed bf16 pair (element 0 = low nibble).
template <int SEL>
__device__ __forceinline__ bf16x2 e2m1x2_to_bf16(uint32_t word) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, SEL);
}

// E4M3 ("FN") byte -> fp32, exactly, from the bit fields.  NaN patterns are
// rejected by moe_w4a16_validate and are not special-cased here.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20))
                        : (float)m * 0x1p-9f;
    return (b & 0x80u) ? -mag : mag;
}

// fp32 pair -> bf16 pair by truncation.  Only used on values that are exact
// in bf16 (E2M1 * E4M3 products), where truncation is exact.
__device__ __forceinline__ uint32_t pack_bf16x2_exact(float lo, float hi) {
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// bf16 pair (as a 32-bit word) dot bf16 pair, accumulated into fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Sum over the 32 lanes of each half-wave (lanes 0..31 and 32..63 separately).
__device__ __forceinline__ float half_wave_sum(float v) {
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = threadIdx.x & (kWave - 1);
    return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// Index of the b-th expert with a nonzero count (ascending), or -1.  Called
// by a whole wave; counts has E entries.
__device__ __forceinline__ int nth_active_expert(const int32_t* __restrict__ counts, int E, int b) {
    const int lane = threadIdx.x & (kWave - 1);
    int seen = 0;
    for (int base = 0; base < E; base += kWave) {
        const int e = base + lane;
        const bool act = e < E && counts[e] > 0;
        const uint64_t m = __ballot(act);
        const int n = __popcll(m);
        if (b < seen + n) {
            const int want = b - seen;  // the want-th set bit of m
            const int rank = __popcll(m & lanemask_lt());
            const uint64_t hit = __ballot(act && rank == want);
            return base + __ffsll((unsigned long long)hit) - 1;
        }
        seen += n;
    }
    return -1;
}

// Exclusive scan of cnt[0..E) into off[0..E] (off[E] = total) by a
// 256-thread workgroup; cnt/off may live in LDS or global memory.
// Contains __syncthreads: every thread of the workgroup must call it.
__device__ inline void block_exclusive_scan(const int* cnt, int* off, int E) {
    constexpr int kThreads = 256, kWaves = kThreads / kWave;
    __shared__ int wave_tot[kWaves];
    const int per = (E + kThreads - 1) / kThreads;
    const int begin = threadIdx.x * per;
    int local = 0;
    for (int i = 0; i < per; ++i)
        if (begin + i < E) local += cnt[begin + i];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    int incl = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    int wave_base = 0;
    for (int i = 0; i < wave; ++i) wave_base += wave_tot[i];
    int run = wave_base + incl - local;
    for (int i = 0; i < per; ++i)
        if (begin + i < E) {
            off[begin + i] = run;
            run += cnt[begin + i];
        }
    if (threadIdx.x == kThreads - 1) off[E] = wave_base + incl;
    __syncthreads();
}

}  // namespace moe
