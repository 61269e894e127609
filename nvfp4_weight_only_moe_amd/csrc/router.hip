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
//  * more tokens: v_mfma_f32_16x16x32_bf16 tiles.  A workgroup owns a tile of
//    32 or 64 tokens x 64 experts and its four waves split K in quarters, each
//    reading its operand rows straight from global memory (W stays in L2):
//    per 64-wide K stage a lane loads 32 contiguous bytes of each of its
//    rows, one 16-byte piece per MFMA step; A and B see the same K order, so
//    the dot products are unchanged.  The quarters meet in LDS and wave 0
//    adds them in wave order.  Splitting K rather than the tile keeps many
//    small waves in flight to cover the load latency of each stage.
// Both are deterministic: fixed summation order, no atomics.
//
// k_router_route (decode token counts): the GEMV and the route in one launch.
// Every workgroup stores its expert's logits at device scope and, once the
// stores are done, takes a ticket (one device-scope vector atomic); the
// workgroup that takes the last ticket reads every logit and routes there --
// top-k per token by a threshold search, the slot order by ballots, counts
// and offsets -- exactly as moe_route_topk would, then puts the ticket word
// back to zero for the next call.
#include "device_common.h"
#include "internal.h"
#include "route_common.h"

namespace moe {
namespace {

constexpr int kRgThreads = 128;     // GEMV: two waves per expert row
constexpr int kRrThreads = 512;     // GEMV + route: eight waves, one token per wave in the routing workgroup
constexpr int kRgBatch = 5;         // 16-byte chunks per lane per batch (one batch at H 5120)
constexpr int kRmThreads = 256;     // MFMA: four waves
constexpr int kRmSmallT = 4096;     // up to here 32-token tiles, above 64
constexpr int kRmCols = 64;         // experts per workgroup tile
constexpr int kRmK = 64;            // K per stage (H % 64 == 0)

// 8 bf16 pairs into an fp32 accumulator (v_dot2_f32_bf16: exact products)
__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b, float acc) {
    acc = dot2_bf16(a.x, b.x, acc);
    acc = dot2_bf16(a.y, b.y, acc);
    acc = dot2_bf16(a.z, b.z, acc);
    return dot2_bf16(a.w, b.w, acc);
}

// One workgroup's expert row e: the NT logits x[t] . W[e] into logits[t][e]
// (COHERENT: stored at device scope, through to the level every CU reads,
// for a workgroup of the same launch to read them).  Waves 0 .. NWV - 1 take
// equal parts of the row (the split fixes the summation order); further
// waves of a larger workgroup only meet the barrier.
template <int NT, bool COHERENT = false, int NWV = 2>
__device__ __forceinline__ void router_gemv_row(const uint16_t* x, const uint16_t* w, int H, int E, int e,
                                                float* __restrict__ logits) {
    // (x and w without __restrict__: their loads would count as invariant
    // and could sink past the issue point below)
    __shared__ float s_part[NWV][NT];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int nch = H / 8;                          // 16-byte chunks per row
    const int part = (nch + NWV - 1) / NWV;          // chunks per wave
    const int c0 = wave < NWV ? min(nch, wave * part) : nch, c1 = min(nch, c0 + part);
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
        if (lane == 0 && wave < NWV) s_part[wave][t] = v;
    }
    __syncthreads();
    if ((int)threadIdx.x < NT) {
        float v = s_part[0][threadIdx.x];
#pragma unroll
        for (int i = 1; i < NWV; ++i) v += s_part[i][threadIdx.x];
        float* dst = logits + (int64_t)threadIdx.x * E + e;
        if constexpr (COHERENT) __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else *dst = v;
    }
}

// NT = the token count exactly (one instance per count): no branch stands
// between the loads, so every weight and x chunk of a batch is requested
// before the first dot product waits.  Lanes past the row's end re-read its
// last chunk and drop the result (a select, not a branch).
template <int NT>
__global__ void __launch_bounds__(kRgThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) k_router_gemv(const uint16_t* x, const uint16_t* w, int H, int E,
                                                            float* __restrict__ logits) {
    router_gemv_row<NT>(x, w, H, E, blockIdx.x, logits);
}

struct RouteOut {
    int32_t* ids;
    float* w;
    int32_t* counts;
    int32_t* offsets;
    int32_t* sorted_slots;
    int32_t* slot_pos;
};

// The hand-off needs no cache-wide flush: the logits are stored and read at
// device scope (coherent across the XCDs' L2s), a workgroup takes its ticket
// only after its stores have completed, and the last workgroup copies the
// logits into LDS with device-scope loads before routing from there.
template <int NT, int EPL>
__global__ void __launch_bounds__(kRrThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
k_router_route(const uint16_t* x, const uint16_t* w, int H, int E, int k, float* logits, uint32_t* ticket,
               const RouteOut R) {
    __shared__ int s_last;
    __shared__ int s_ids[64];
    __shared__ int s_key[kRrThreads / kWave][MOE_MAX_TOPK], s_idx[kRrThreads / kWave][MOE_MAX_TOPK];
    __shared__ float s_logits[NT * 64 * EPL];
    router_gemv_row<NT, true, 2>(x, w, H, E, blockIdx.x, logits);   // the GEMV's own split: the same logit bits
    __syncthreads();                                    // waits for this workgroup's stores to complete
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = old == gridDim.x - 1;
    }
    __syncthreads();
    if (!s_last) return;
    // every other workgroup stored its logits before taking its ticket
    for (int i = threadIdx.x; i < NT * E; i += kRrThreads)
        s_logits[i] = __hip_atomic_load(logits + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    for (int t = wave; t < NT; t += kRrThreads / kWave) {
        int id;
        float v;
        wave_topk_ordered<EPL>(s_logits + t * E, E, k, s_key[wave], s_idx[wave], id, v);
        const float wt = topk_softmax(v, k);
        if (lane < k) {
            R.ids[t * k + lane] = id;
            R.w[t * k + lane] = wt;
            s_ids[t * k + lane] = id;
        }
    }
    __syncthreads();
    tiny_route_finish(s_ids, NT, E, k, R.counts, R.offsets, R.sorted_slots, R.slot_pos);
    if (threadIdx.x == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int ROWS>
__global__ void __launch_bounds__(kRmThreads) __attribute__((amdgpu_waves_per_eu(2, 4)))
k_router_mfma(const uint16_t* x, const uint16_t* w, int T, int H, int E, float* __restrict__ logits) {
    constexpr int kMs = ROWS / 16, kNs = kRmCols / 16;
    constexpr int kWaves = kRmThreads / kWave;
    constexpr int kSteps = kRmK / 32;                 // MFMA steps per stage
    // partial tiles of waves 1..3, summed by wave 0: [wave - 1][ms][ns][lane] floatx4
    __shared__ floatx4 part[kWaves - 1][kMs][kNs][kWave];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int lcol = lane & 15, kq = lane >> 4;
    const int t0 = blockIdx.x * ROWS, e0 = blockIdx.y * kRmCols;
    // this wave's share of the K stages
    const int nst = H / kRmK;
    const int s0 = nst * wave / kWaves, s1 = nst * (wave + 1) / kWaves;
    // operand rows of this lane (clamped inside the tensors; stores are masked)
    const uint16_t* arow[kMs];
    const uint16_t* brow[kNs];
#pragma unroll
    for (int ms = 0; ms < kMs; ++ms)
        arow[ms] = x + (int64_t)min(t0 + ms * 16 + lcol, T - 1) * H + (kRmK / 4) * kq;
#pragma unroll
    for (int ns = 0; ns < kNs; ++ns)
        brow[ns] = w + (int64_t)min(e0 + ns * 16 + lcol, E - 1) * H + (kRmK / 4) * kq;

    floatx4 acc[kMs][kNs];
#pragma unroll
    for (int ms = 0; ms < kMs; ++ms)
#pragma unroll
        for (int ns = 0; ns < kNs; ++ns) acc[ms][ns] = floatx4{0.f, 0.f, 0.f, 0.f};
    // a lane's K slice of a stage: kRmK / 4 contiguous elements, one 16-byte
    // piece per MFMA step
    for (int st = s0; st < s1; ++st) {
        const int k0 = st * kRmK;
        uint4 a[kMs][kSteps], b[kNs][kSteps];
#pragma unroll
        for (int ms = 0; ms < kMs; ++ms)
#pragma unroll
            for (int i = 0; i < kSteps; ++i) a[ms][i] = *reinterpret_cast<const uint4*>(arow[ms] + k0 + 8 * i);
#pragma unroll
        for (int ns = 0; ns < kNs; ++ns)
#pragma unroll
            for (int i = 0; i < kSteps; ++i) b[ns][i] = *reinterpret_cast<const uint4*>(brow[ns] + k0 + 8 * i);
#pragma unroll
        for (int i = 0; i < kSteps; ++i)
#pragma unroll
            for (int ms = 0; ms < kMs; ++ms)
#pragma unroll
                for (int ns = 0; ns < kNs; ++ns)
                    acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, a[ms][i]), __builtin_bit_cast(bf16x8, b[ns][i]), acc[ms][ns], 0, 0,
                        0);
    }
    // the K quarters meet in LDS; wave 0 adds them in wave order
    if (wave > 0) {
#pragma unroll
        for (int ms = 0; ms < kMs; ++ms)
#pragma unroll
            for (int ns = 0; ns < kNs; ++ns) part[wave - 1][ms][ns][lane] = acc[ms][ns];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int v = 0; v < kWaves - 1; ++v)
#pragma unroll
        for (int ms = 0; ms < kMs; ++ms)
#pragma unroll
            for (int ns = 0; ns < kNs; ++ns) acc[ms][ns] += part[v][ms][ns][lane];
    // lane holds rows 4 kq + r of each 16-row subtile, column lcol
#pragma unroll
    for (int ms = 0; ms < kMs; ++ms)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + ms * 16 + 4 * kq + r;
            if (t >= T) continue;
#pragma unroll
            for (int ns = 0; ns < kNs; ++ns) {
                const int e = e0 + ns * 16 + lcol;
                if (e < E) logits[(int64_t)t * E + e] = acc[ms][ns][r];
            }
        }
}

template <int NT>
moe_status launch_gemv(const uint16_t* x, int H, const uint16_t* w, int E, float* logits, hipStream_t s) {
    MOE_LAUNCH("router_gemv", (k_router_gemv<NT>), dim3(E), dim3(kRgThreads), 0, s, x, w, H, E, logits);
    return MOE_OK;
}

template <int NT, int EPL>
moe_status launch_router_route_t(const uint16_t* x, int H, const uint16_t* w, int E, int k, float* logits,
                                 uint32_t* ticket, const RouteOut& R, hipStream_t s) {
    MOE_LAUNCH("router_route", (k_router_route<NT, EPL>), dim3(E), dim3(kRrThreads), 0, s, x, w, H, E, k, logits,
               ticket, R);
    return MOE_OK;
}

template <int NT>
moe_status launch_router_route_n(const uint16_t* x, int H, const uint16_t* w, int E, int k, float* logits,
                                 uint32_t* ticket, const RouteOut& R, hipStream_t s) {
    if (E <= 64) return launch_router_route_t<NT, 1>(x, H, w, E, k, logits, ticket, R, s);
    if (E <= 128) return launch_router_route_t<NT, 2>(x, H, w, E, k, logits, ticket, R, s);
    if (E <= 256) return launch_router_route_t<NT, 4>(x, H, w, E, k, logits, ticket, R, s);
    if (E <= 512) return launch_router_route_t<NT, 8>(x, H, w, E, k, logits, ticket, R, s);
    return launch_router_route_t<NT, 16>(x, H, w, E, k, logits, ticket, R, s);
}

}  // namespace

bool router_route_fused_supported(int T, int H, int E, int k) {
    return T >= 1 && T <= 8 && T * k <= 64 && k <= MOE_MAX_TOPK && E >= 1 && E <= MOE_MAX_EXPERTS &&
           router_shape_supported(T, H, E);
}

moe_status launch_router_route(const uint16_t* x, int T, int H, const uint16_t* w, int E, int k, float* logits,
                               uint32_t* ticket, int32_t* ids, float* wts, int32_t* counts, int32_t* offsets,
                               int32_t* sorted_slots, int32_t* slot_pos, hipStream_t s) {
    if (!router_route_fused_supported(T, H, E, k)) return MOE_ERR_UNSUPPORTED;
    const RouteOut R{ids, wts, counts, offsets, sorted_slots, slot_pos};
    switch (T) {
        case 1: return launch_router_route_n<1>(x, H, w, E, k, logits, ticket, R, s);
        case 2: return launch_router_route_n<2>(x, H, w, E, k, logits, ticket, R, s);
        case 3: return launch_router_route_n<3>(x, H, w, E, k, logits, ticket, R, s);
        case 4: return launch_router_route_n<4>(x, H, w, E, k, logits, ticket, R, s);
        case 5: return launch_router_route_n<5>(x, H, w, E, k, logits, ticket, R, s);
        case 6: return launch_router_route_n<6>(x, H, w, E, k, logits, ticket, R, s);
        case 7: return launch_router_route_n<7>(x, H, w, E, k, logits, ticket, R, s);
        default: return launch_router_route_n<8>(x, H, w, E, k, logits, ticket, R, s);
    }
}

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
    // 32-token tiles double the workgroups where tokens are few; 64-token
    // tiles halve the W_r re-reads where there are many
    if (T <= kRmSmallT) {
        const dim3 grid((T + 31) / 32, (E + kRmCols - 1) / kRmCols);
        MOE_LAUNCH("router_mfma", k_router_mfma<32>, grid, dim3(kRmThreads), 0, s, x, w, T, H, E, logits);
    } else {
        const dim3 grid((T + 63) / 64, (E + kRmCols - 1) / kRmCols);
        MOE_LAUNCH("router_mfma", k_router_mfma<64>, grid, dim3(kRmThreads), 0, s, x, w, T, H, E, logits);
    }
    return MOE_OK;
}

}  // namespace moe
