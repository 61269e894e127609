// Router logits: the BF16 gate in front of the top-k, logits[t][e] =
// sum_i x[t][i] * W[e][i] with fp32 accumulation (the routers stay BF16 and
// are never quantized: "GLM-5.3-Flash on Blackwell", "The quantization").
//
// Two shapes of the same product:
//  * 1-8 tokens (decode): a GEMV that streams W once.  One workgroup per
//    expert row, its two waves take one half of the row each; every lane
//    requests its 16-byte weight chunks and the tokens' matching x chunks
//    (L2-resident) before using any, dots them in fp32 (v_dot2_f32_bf16),
//    and the halves meet in LDS.  2.6 MB of weights at H 5120, E 256.
//  * more tokens: v_mfma_f32_16x16x32_bf16 tiles.  A workgroup owns 32 token
//    rows; each of its four waves computes 32 x 64 expert tiles, reading
//    both operands straight from global memory (the whole W stays in L2):
//    per 64-wide K stage a lane loads 32 contiguous bytes of each of its
//    rows, one 16-byte piece per MFMA step; A and B see the same K order, so
//    the dot products are unchanged.  Every workgroup reads all of W from
//    L2, which bounds this shape (about 2 GB of L2 reads at 16K tokens).
// Both are deterministic: fixed summation order, no atomics.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kRgThreads = 128;     // GEMV: two waves per expert row
constexpr int kRgBatch = 5;         // 16-byte chunks per lane per batch (one batch at H 5120)
constexpr int kRmThreads = 256;     // MFMA: four waves
constexpr int kRmRows = 32;         // token rows per workgroup
constexpr int kRmCols = 64;         // experts per wave tile
constexpr int kRmK = 64;            // K per stage (H % 64 == 0)

// 8 bf16 pairs into an fp32 accumulator (v_dot2_f32_bf16: exact products)
__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b, float acc) {
    acc = dot2_bf16(a.x, b.x, acc);
    acc = dot2_bf16(a.y, b.y, acc);
    acc = dot2_bf16(a.z, b.z, acc);
    return dot2_bf16(a.w, b.w, acc);
}

// NT = the token count exactly (one instance per count): no branch stands
// between the loads, so every weight and x chunk of a batch is requested
// before the first dot product waits.  Lanes past the row's end re-read its
// last chunk and drop the result (a select, not a branch).
template <int NT>
__global__ void __launch_bounds__(kRgThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) k_router_gemv(const uint16_t* x, const uint16_t* w, int H, int E,
                                                            float* __restrict__ logits) {
    // (x and w without __restrict__: their loads would count as invariant
    // and could sink past the issue point below)
    __shared__ float s_part[2][NT];
    const int e = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int nch = H / 8;                          // 16-byte chunks per row
    const int half = (nch + 1) / 2;
    const int c0 = wave * half, c1 = min(nch, c0 + half);
    const uint4* wr = reinterpret_cast<const uint4*>(w + (int64_t)e * H);

    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
    for (int cb = c0; cb < c1; cb += kWave * kRgBatch) {
        int cc[kRgBatch];
        bool ok[kRgBatch];
        uint4 wv[kRgBatch], xv[NT][kRgBatch];
#pragma unroll
        for (int j = 0; j < kRgBatch; ++j) {
            const int c = cb + lane + kWave * j;
            ok[j] = c < c1;
            cc[j] = ok[j] ? c : c1 - 1;
            wv[j] = wr[cc[j]];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < kRgBatch; ++j) xv[t][j] = reinterpret_cast<const uint4*>(x + (int64_t)t * H)[cc[j]];
        asm volatile("" ::: "memory");              // issue every load here, not at its first use
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < kRgBatch; ++j) {
                const float a = dot8_bf16(wv[j], xv[t][j], acc[t]);
                acc[t] = ok[j] ? a : acc[t];
            }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const float v = wave_sum_dpp(acc[t]);
        if (lane == 0) s_part[wave][t] = v;
    }
    __syncthreads();
    if ((int)threadIdx.x < NT) logits[(int64_t)threadIdx.x * E + e] = s_part[0][threadIdx.x] + s_part[1][threadIdx.x];
}

__global__ void __launch_bounds__(kRmThreads)
k_router_mfma(const uint16_t* x, const uint16_t* w, int T, int H, int E, float* __restrict__ logits) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int lcol = lane & 15, kq = lane >> 4;
    const int t0 = blockIdx.x * kRmRows;
    const int ngroups = (E + kRmCols - 1) / kRmCols;
    // operand rows of this lane (clamped inside the tensors; stores are masked)
    const uint16_t* arow[2];
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
        arow[ms] = x + (int64_t)min(t0 + ms * 16 + lcol, T - 1) * H + (kRmK / 4) * kq;

    for (int g = wave; g < ngroups; g += kRmThreads / kWave) {
        const uint16_t* brow[4];
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
            brow[ns] = w + (int64_t)min(g * kRmCols + ns * 16 + lcol, E - 1) * H + (kRmK / 4) * kq;
        floatx4 acc[2][4];
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = floatx4{0.f, 0.f, 0.f, 0.f};
        // a lane's K slice of a stage: kRmK / 4 contiguous elements, one
        // 16-byte piece per MFMA step
        constexpr int kSteps = kRmK / 32;
        for (int k0 = 0; k0 < H; k0 += kRmK) {
            uint4 a[2][kSteps], b[4][kSteps];
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                for (int i = 0; i < kSteps; ++i) a[ms][i] = *reinterpret_cast<const uint4*>(arow[ms] + k0 + 8 * i);
#pragma unroll
            for (int ns = 0; ns < 4; ++ns)
#pragma unroll
                for (int i = 0; i < kSteps; ++i) b[ns][i] = *reinterpret_cast<const uint4*>(brow[ns] + k0 + 8 * i);
#pragma unroll
            for (int i = 0; i < kSteps; ++i)
#pragma unroll
                for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                    for (int ns = 0; ns < 4; ++ns)
                        acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, a[ms][i]), __builtin_bit_cast(bf16x8, b[ns][i]),
                            acc[ms][ns], 0, 0, 0);
        }
        // lane holds rows 4 kq + r of each 16-row subtile, column lcol
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + ms * 16 + 4 * kq + r;
                if (t >= T) continue;
#pragma unroll
                for (int ns = 0; ns < 4; ++ns) {
                    const int e = g * kRmCols + ns * 16 + lcol;
                    if (e < E) logits[(int64_t)t * E + e] = acc[ms][ns][r];
                }
            }
    }
}

template <int NT>
moe_status launch_gemv(const uint16_t* x, int H, const uint16_t* w, int E, float* logits, hipStream_t s) {
    MOE_LAUNCH("router_gemv", (k_router_gemv<NT>), dim3(E), dim3(kRgThreads), 0, s, x, w, H, E, logits);
    return MOE_OK;
}

}  // namespace

bool router_shape_supported(int T, int H, int E) { return T >= 0 && E >= 1 && H >= kRmK && H % kRmK == 0; }

moe_status launch_router_logits(const uint16_t* x, int T, int H, const uint16_t* w, int E, float* logits,
                                hipStream_t s) {
    if (!router_shape_supported(T, H, E)) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    switch (T) {
        case 1: return launch_gemv<1>(x, H, w, E, logits, s);
        case 2: return launch_gemv<2>(x, H, w, E, logits, s);
        case 3: return launch_gemv<3>(x, H, w, E, logits, s);
        case 4: return launch_gemv<4>(x, H, w, E, logits, s);
        case 5: return launch_gemv<5>(x, H, w, E, logits, s);
        case 6: return launch_gemv<6>(x, H, w, E, logits, s);
        case 7: return launch_gemv<7>(x, H, w, E, logits, s);
        case 8: return launch_gemv<8>(x, H, w, E, logits, s);
        default: break;
    }
    const int grid = (T + kRmRows - 1) / kRmRows;
    MOE_LAUNCH("router_mfma", k_router_mfma, dim3(grid), dim3(kRmThreads), 0, s, x, w, T, H, E, logits);
    return MOE_OK;
}

}  // namespace moe
