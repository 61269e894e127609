// A plain streaming read, the achievable-rate reference the benchmark sets
// beside the spec HBM peak: a kernel that only reads (16-byte non-temporal
// loads, the decode kernels' load width and cache policy), with every
// thread's loads issued before any is used, and writes nothing back except
// in the (never taken in practice) case that its reduction equals a magic
// value, so that the compiler keeps the loads.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamLoads = 12;       // 16-byte loads per thread (48 KiB per workgroup)
constexpr uint32_t kStreamMagic = 0x9E3779B9u;

__global__ void __launch_bounds__(kStreamThreads) k_stream_read(const uint4* __restrict__ src, int64_t chunks,
                                                                uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int64_t base = ((int64_t)blockIdx.x * (kStreamThreads / kWave) + wave) * kStreamLoads * kWave;
    uint4 v[kStreamLoads];
#pragma unroll
    for (int u = 0; u < kStreamLoads; ++u) {
        const int64_t i = base + (int64_t)u * kWave + lane;
        v[u] = i < chunks ? load_stream16(src + i) : make_uint4(0, 0, 0, 0);
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < kStreamLoads; ++u) acc ^= v[u].x + v[u].y + v[u].z + v[u].w;
    if (acc == kStreamMagic) *sink = acc;
}

}  // namespace

moe_status launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
    const int64_t chunks = (int64_t)(bytes / 16);
    if (chunks == 0) return MOE_OK;
    const int64_t per_block = (int64_t)kStreamThreads * kStreamLoads;
    const int64_t blocks = (chunks + per_block - 1) / per_block;
    if (blocks > INT32_MAX) return MOE_ERR_SHAPE;
    MOE_LAUNCH("stream_read", k_stream_read, dim3((unsigned)blocks), dim3(kStreamThreads), 0, s,
               static_cast<const uint4*>(src), chunks, sink);
    return MOE_OK;
}

}  // namespace moe
