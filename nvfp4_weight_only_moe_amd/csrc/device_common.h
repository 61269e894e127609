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

// E4M3 ("FN") byte SEL of `word` -> fp32, exactly, with gfx950's FP8
// conversion (OCP E4M3: bias 7, subnormals m * 2^-9, 0x7F/0xFF NaN; NaN
// patterns are rejected by moe_w4a16_validate).
template <int SEL>
__device__ __forceinline__ float e4m3_byte_to_f32(uint32_t word) {
    return __builtin_amdgcn_cvt_f32_fp8((int)word, SEL);
}
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) { return e4m3_byte_to_f32<0>(b); }

// fp32 pair -> bf16 pair by truncation.  Only used on values that are exact
// in bf16 (E2M1 * E4M3 products), where truncation is exact.
__device__ __forceinline__ uint32_t pack_bf16x2_exact(float lo, float hi) {
    // one v_perm_b32: bytes 2, 3 of lo, then bytes 2, 3 of hi
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
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

// Dot of 8 bf16 pairs (one 16-group of activations) with the 16 codes of a
// group, unscaled: codes decode to exact bf16 pairs, v_dot2 accumulates in
// fp32.
__device__ __forceinline__ float group_dot(uint2 codes, uint4 xa, uint4 xb) {
    float acc = 0.0f;
    acc = dot2_bf16(__builtin_bit_cast(uint32_t, e2m1x2_to_bf16<0>(codes.x)), xa.x, acc);
    acc = dot2_bf16(__builtin_bit_cast(uint32_t, e2m1x2_to_bf16<1>(codes.x)), xa.y, acc);
    acc = dot2_bf16(__builtin_bit_cast(uint32_t, e2m1x2_to_bf16<2>(codes.x)), xa.z, acc);
    acc = dot2_bf16(__builtin_bit_cast(uint32_t, e2m1x2_to_bf16<3>(codes.x)), xa.w, acc);
    acc = dot2_bf16(__builtin_bit_cast(uint32_t, e2m1x2_to_bf16<0>(codes.y)), xb.x, acc);
    acc = dot2_bf16(__builtin_bit_cast(uint32_t, e2m1x2_to_bf16<1>(codes.y)), xb.y, acc);
    acc = dot2_bf16(__builtin_bit_cast(uint32_t, e2m1x2_to_bf16<2>(codes.y)), xb.z, acc);
    acc = dot2_bf16(__builtin_bit_cast(uint32_t, e2m1x2_to_bf16<3>(codes.y)), xb.w, acc);
    return acc;
}

// ---------------------------------------------------------------- LDS DMA
typedef __attribute__((address_space(3))) void lds_void;

// One wave copies 64 x 16 B (1 KiB) from global memory straight into LDS
// (gfx950 global_load_lds_dwordx4): lane i's 16 bytes land at lds + 16 i.
// No registers are involved; completion is tracked like any vector load.
__device__ __forceinline__ void wave_copy_1k_to_lds(const uint4* __restrict__ src, uint4* lds) {
    const int lane = threadIdx.x & 63;
    __builtin_amdgcn_global_load_lds(src + lane, (lds_void*)lds, 16, 0, 0);
}

// The same LDS-DMA, 16 or 4 bytes per lane, issued as inline assembly: the
// compiler does not see the LDS write, so it inserts no wait on it before
// later LDS reads (it would wait for every load in flight); the caller must
// wait (vmcnt) and synchronise before the data is read.  The s_nop gives the
// M0 write its wait state.
__device__ __forceinline__ void lds_dma16(const void* gsrc, lds_void* ldst) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"((uint32_t)(uintptr_t)ldst)
                 : "memory");
}
__device__ __forceinline__ void lds_dma4(const void* gsrc, lds_void* ldst) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gsrc), "{m0}"((uint32_t)(uintptr_t)ldst)
                 : "memory");
}

// The same with a wave-uniform 64-bit base (SGPR pair) and a 32-bit per-lane
// byte offset: the base can move on by scalar arithmetic alone.
__device__ __forceinline__ void lds_dma16_sv(const void* sbase, uint32_t voff, lds_void* ldst) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
                 "{m0}"((uint32_t)(uintptr_t)ldst) : "memory");
}
__device__ __forceinline__ void lds_dma4_sv(const void* sbase, uint32_t voff, lds_void* ldst) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase),
                 "{m0}"((uint32_t)(uintptr_t)ldst) : "memory");
}

// Non-temporal 16- and 8-byte loads (the "nt" cache policy): for weights
// that are read exactly once per step, so that streaming them does not evict
// what stays hot between launches (kernel code, activations, routing data)
// from L2 and the Infinity Cache.
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int nt_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_stream16(const uint4* p) {
    const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 load_stream8(const uint2* p) {
    const nt_u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x2*>(p));
    return make_uint2(v[0], v[1]);
}
template <class Tv>
__device__ __forceinline__ Tv load_stream(const Tv* p) { return __builtin_nontemporal_load(p); }

// Wait for every outstanding memory operation of this wave.
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Workgroup barrier that waits only for this wave's LDS operations, not for
// its vector-memory loads in flight (a __syncthreads fence waits for all).
__device__ __forceinline__ void wait_lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt 63 (no wait), expcnt 7 (no wait), lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Wait until at most N vector-memory loads of this wave are outstanding
// (they complete in issue order); LDS and scalar counters are not waited on.
template <int N>
__device__ __forceinline__ void wait_vmem_at_most() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// ---------------------------------------------------------------- wave ops
// DPP moves (GFX9 data-parallel primitives): a lane reads a neighbour's
// register without going through LDS.  Lanes whose source is outside the
// row, or whose row is masked off, receive `old`.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float old, float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                 __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                                                 0xF, false));
}
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// Inclusive prefix sums inside each row of 16 lanes (lane 15 of a row holds
// the row total).
__device__ __forceinline__ float row_prefix_sum(float v) {
    v += dpp_f32<kDppRowShr1>(0.0f, v);
    v += dpp_f32<kDppRowShr2>(0.0f, v);
    v += dpp_f32<kDppRowShr4>(0.0f, v);
    v += dpp_f32<kDppRowShr8>(0.0f, v);
    return v;
}

// Sum over all 64 lanes, returned in every lane (DPP, no LDS traffic).
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v = row_prefix_sum(v);
    v += dpp_f32<kDppRowBcast15, 0xA>(0.0f, v);   // rows 1, 3 += lane 15 / 47
    v += dpp_f32<kDppRowBcast31, 0xC>(0.0f, v);   // rows 2, 3 += lane 31
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Sums over lanes 0..31 and 32..63; returns the sum of the caller's half.
__device__ __forceinline__ float half_wave_sum_dpp(float v) {
    v = row_prefix_sum(v);
    v += dpp_f32<kDppRowBcast15, 0xA>(0.0f, v);   // lane 31 = rows 0+1, lane 63 = rows 2+3
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
    return (threadIdx.x & 32) ? hi : lo;
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i32(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes (lane i gets lanes 0..i), DPP only.
__device__ __forceinline__ int wave_inclusive_scan_dpp(int v) {
    v += dpp_i32<kDppRowShr1>(0, v);
    v += dpp_i32<kDppRowShr2>(0, v);
    v += dpp_i32<kDppRowShr4>(0, v);
    v += dpp_i32<kDppRowShr8>(0, v);
    v += dpp_i32<kDppRowBcast15, 0xA>(0, v);
    v += dpp_i32<kDppRowBcast31, 0xC>(0, v);
    return v;
}

// Maximum over all 64 lanes (NaN-free inputs), returned in every lane.
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = fmaxf(v, dpp_f32<kDppRowShr1>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<kDppRowShr2>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<kDppRowShr4>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<kDppRowShr8>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<kDppRowBcast15, 0xA>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<kDppRowBcast31, 0xC>(-INFINITY, v));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Maximum over all 64 lanes of unsigned keys, returned in every lane.
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t u) {
    int v = (int)u;
    v = (int)max((uint32_t)v, (uint32_t)dpp_i32<kDppRowShr1>(0, v));
    v = (int)max((uint32_t)v, (uint32_t)dpp_i32<kDppRowShr2>(0, v));
    v = (int)max((uint32_t)v, (uint32_t)dpp_i32<kDppRowShr4>(0, v));
    v = (int)max((uint32_t)v, (uint32_t)dpp_i32<kDppRowShr8>(0, v));
    v = (int)max((uint32_t)v, (uint32_t)dpp_i32<kDppRowBcast15, 0xA>(0, v));
    v = (int)max((uint32_t)v, (uint32_t)dpp_i32<kDppRowBcast31, 0xC>(0, v));
    return (uint32_t)__builtin_amdgcn_readlane(v, 63);
}

// Minimum over all 64 lanes, returned in every lane.
__device__ __forceinline__ int wave_min_i32_dpp(int v) {
    v = min(v, dpp_i32<kDppRowShr1>(INT_MAX, v));
    v = min(v, dpp_i32<kDppRowShr2>(INT_MAX, v));
    v = min(v, dpp_i32<kDppRowShr4>(INT_MAX, v));
    v = min(v, dpp_i32<kDppRowShr8>(INT_MAX, v));
    v = min(v, dpp_i32<kDppRowBcast15, 0xA>(INT_MAX, v));
    v = min(v, dpp_i32<kDppRowBcast31, 0xC>(INT_MAX, v));
    return __builtin_amdgcn_readlane(v, 63);
}

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

// The b-th expert with a nonzero count (ascending), its count and its first
// row in expert-sorted order (the exclusive prefix of the counts), or e = -1.
// Called by a whole wave.  All count loads are issued before any is used
// (EPL = ceil(E / 64) per lane), so the lookup costs one memory latency.
struct ActiveExpert {
    int e, count, first_row;
};
template <int EPL>
__device__ __forceinline__ ActiveExpert nth_active_expert(const int32_t* __restrict__ counts, int E, int b) {
    const int lane = threadIdx.x & (kWave - 1);
    int c[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = i * kWave + lane;
        c[i] = e < E ? counts[e] : 0;
    }
    int seen = 0, rows = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const uint64_t m = __ballot(c[i] > 0);
        const int n = __popcll(m);
        const int incl = wave_inclusive_scan_dpp(c[i]);   // counts over the lanes of this chunk
        if (b < seen + n) {
            const int want = b - seen;
            const uint64_t hit = __ballot(c[i] > 0 && __popcll(m & lanemask_lt()) == want);
            const int src = __ffsll((unsigned long long)hit) - 1;
            const int cnt = __builtin_amdgcn_readlane(c[i], src);
            const int excl = __builtin_amdgcn_readlane(incl, src) - cnt;
            return ActiveExpert{i * kWave + src, cnt, rows + excl};
        }
        seen += n;
        rows += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    return ActiveExpert{-1, 0, 0};
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
