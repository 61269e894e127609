// Prefill-shape forward (many tokens): grouped GEMMs on the bf16 MFMA units.
//
// The W4A16 route dequantises the 4-bit weights to bf16 inside the GEMM and
// feeds bf16 matrix instructions; no activation scale is involved ("GLM-5.3-
// Flash on Blackwell", "The model loaded, served an API, and produced
// garbage").  E2M1 * E4M3 is exact in bf16, so the MFMA sees the exact
// weight up to the FP32 global scale, which is applied once per output in
// the epilogue.
//
// k_grouped_gemm<GATEUP, BM, BK, NW, SDMA> computes, for every expert e and
// its rows of the expert-sorted permutation (offsets[e] .. offsets[e+1]):
//   GATEUP: h[p, :] = bf16( silu(gg_e * x_t . G_e^T) * (gu_e * x_t . U_e^T) ),
//           t = sorted_slots[p] / k          (rows gathered from x)
//   DOWN:   y[p, :] = bf16(gd_e * h_p . D_e^T)
// Workgroup tile: up to BM rows x 32 NW h-columns (GATEUP, gate and up
// together) or x 64 NW columns (DOWN); NW waves (4 or 8), each owning 4
// column subtiles of 16 and all the tile's rows, so each weight element is
// decoded by exactly one wave; a tile computes only the 16-row subtiles its
// rows need.  The activation tile of a K stage (BK = 128 or 256) is staged
// in LDS (double buffered); weights stream from HBM straight into registers
// with 16-byte loads and are decoded there; their E4M3 scales come through
// LDS in blocks (SDMA).  MFMA: v_mfma_f32_16x16x32_bf16.
//
// The K order inside a stage is permuted identically for both operands
// (lane group q holds k = (BK / 4) q + 8 s .. + 7 at k-step s), which lets
// one 16-byte load feed a lane's weight codes for four k-steps.
//
// The grid is persistent; tiles are numbered expert by expert, within an
// expert in groups of 8 row tiles x all column tiles, and handed out so that
// each XCD (workgroup id mod 8) works on a contiguous run of tiles: row tiles
// that share a weight column tile meet in the same L2.
//
// k_combine: out[t] = bf16( sum_j w[t,j] * y[slot_pos[t*k+j]] ), fp32, j order
// (y is stored as bf16: half the bytes of the round trip through memory).
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kMGroup = 8;                  // row tiles per scheduling group

struct GemmParams {
    const uint16_t* a;          // GATEUP: x [T][K]; DOWN: h [T*k][K]
    const int32_t* sorted_slots;
    int topk;
    int K, N, E;
    const uint8_t *c0, *s0;     // gate (GATEUP) or down (DOWN)
    const float* g0;
    const uint8_t *c1, *s1;     // up (GATEUP only)
    const float* g1;
    const int32_t* counts;
    const int32_t* offsets;
    void* out;                  // GATEUP: h bf16 [T*k][N]; DOWN: y bf16 [T*k][N]
    int ntn;                    // column tiles per expert
    float gmul;                 // multiplies the global scales (W4A4 input scale; 1 for W4A16)
    float* hf;                  // gate/up: fp32 h instead of bf16 into out, when set (W4A4)
};

__device__ __forceinline__ bf16x8 decode8(uint32_t word, float s) {
    const floatx2 p0 = e2m1x2_to_f32<0>(word);
    const floatx2 p1 = e2m1x2_to_f32<1>(word);
    const floatx2 p2 = e2m1x2_to_f32<2>(word);
    const floatx2 p3 = e2m1x2_to_f32<3>(word);
    u32x4 r;
    r[0] = pack_bf16x2_exact(p0[0] * s, p0[1] * s);
    r[1] = pack_bf16x2_exact(p1[0] * s, p1[1] * s);
    r[2] = pack_bf16x2_exact(p2[0] * s, p2[1] * s);
    r[3] = pack_bf16x2_exact(p3[0] * s, p3[1] * s);
    return __builtin_bit_cast(bf16x8, r);
}

// Workgroups per CU: with four waves the 32-row tiles fit three (164
// VGPRs), which keeps more weight loads in flight at the few rows per
// expert they serve; eight-wave workgroups run one per CU.
template <int BM, int NW> constexpr int gemm_wg_per_cu() {
    return NW == 8 ? 1 : BM >= 128 ? 1 : BM == 32 ? 3 : 2;
}

// One tile: the tile's rows (rows <= 16 MSR) of NW waves, each owning 4
// column subtiles of 16 (gate/up: 32 h columns as 32 gate + 32 up weight
// rows; down: 64 output columns) for all 16 MSR rows, so the tile is
// 16 MSR rows x 32 NW (gate/up) or 64 NW (down) columns and each weight
// element is decoded by exactly one wave.  MSR is the number of 16-row
// subtiles the tile's rows need: a tile of an expert with 20 rows issues half
// the MFMAs and activation-fragment reads of a full 64-row tile.  BK = K per
// stage: 128, or 256 so that a weight row's codes of one stage fill a whole
// 128-byte line (its next bytes are not left for a later stage, when another
// tile's lines may have evicted the line from L2).
template <bool GATEUP, int BK, int NW, bool SDMA, int MSR>
__device__ __forceinline__ void grouped_tile(const GemmParams& P, uint8_t* smem, uint8_t* sscale, int e, int nt,
                                             int p0, int rows) {
    constexpr int kThreads = NW * kWave;
    constexpr int NS = 4;                       // column subtiles per wave
    constexpr int BN = (GATEUP ? 32 : 64) * NW; // output columns per tile
    constexpr int kRows = 16 * MSR;             // rows staged and computed
    constexpr int kLdsRow = BK * 2 + 16;        // bytes per staged activation row (padded)
    constexpr int kRowChunks = BK * 2 / 16;     // 16-byte activation chunks per row per stage
    constexpr int APT = kRows * kRowChunks / kThreads;   // activation chunks per thread per stage
    constexpr int KSTEPS = BK / 32;             // MFMA k-steps per stage
    constexpr int CW = BK / 128;                // 16-byte code words per lane per subtile per stage
    // Scales through LDS (SDMA, when K % 256 == 0): each weight row's E4M3 bytes of
    // SB stages (64 bytes) go to LDS by LDS-DMA as four 16-byte pieces, the
    // next block while the current one is used; a lane then reads its scale
    // word of a stage from LDS.  Loaded straight from memory instead, every
    // stage costs each lane one 2- or 4-byte load per subtile, 16 rows of 16
    // bytes per wave instruction: at 1K tokens those loads alone took ~145 of
    // the gate/up kernel's ~570 us of loads and staging.
    constexpr int SB = 1024 / BK;               // stages per scale block (64 bytes of a row)
    constexpr int kSRows = 64 * NW;             // weight rows of the tile
    constexpr int kSBlock = kSRows * 64;        // bytes per scale block
    static_assert(APT * kThreads == kRows * kRowChunks, "activation stage split over the threads");
    static_assert(!SDMA || kSRows * 4 == 4 * kThreads, "four 16-byte scale pieces per thread per block");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lcol = lane & 15, kq = lane >> 4;
    const int nst = P.K / BK;

    // activation chunks this thread stages: chunk c = tid + kThreads * i
    // of the stage, row c / kRowChunks, 16-byte unit c % kRowChunks
    int64_t a_off[APT];
#pragma unroll
    for (int i = 0; i < APT; ++i) {
        const int c = tid + kThreads * i;
        const int r = c / kRowChunks;
        int64_t off = -1;
        if (r < rows) {
            const int64_t src_row = GATEUP ? (int64_t)(P.sorted_slots[p0 + r] / P.topk) : (int64_t)(p0 + r);
            off = src_row * P.K + (c % kRowChunks) * 8;
        }
        a_off[i] = off;
    }
    // weight rows of this wave's column subtiles
    const uint8_t* cp[NS];
    const uint8_t* sp[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
        int col;
        const uint8_t *cb, *sb;
        if (GATEUP) {
            col = nt * BN + wave * 32 + (ns & 1) * 16 + lcol;
            cb = ns < 2 ? P.c0 : P.c1;
            sb = ns < 2 ? P.s0 : P.s1;
        } else {
            col = nt * BN + wave * 64 + ns * 16 + lcol;
            cb = P.c0;
            sb = P.s0;
        }
        const int64_t row = (int64_t)e * P.N + col;
        cp[ns] = cb + row * (P.K / 2) + kq * 16 * CW;
        sp[ns] = sb + row * (P.K / 16) + kq * 2 * CW;
    }

    floatx4 acc[MSR][NS];
#pragma unroll
    for (int i = 0; i < MSR; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // scale block b -> LDS buffer b & 1: piece c = tid + kThreads i is bytes
    // 16 (c % 4) .. + 15 of the block in tile weight row c / 4 (gate/up:
    // rows [0, BN) of the gate matrix, then [BN, 2 BN) of the up matrix), so
    // each wave instruction fills 1 KiB of LDS in order (lane j at + 16 j)
    auto load_scale_block = [&](int b) {
        if constexpr (SDMA) {
            uint8_t* dst = sscale + (b & 1) * kSBlock;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = tid + kThreads * i;
                const int r = c >> 2, boff = b * 64 + (c & 3) * 16;
                const uint8_t* sb;
                int64_t row;
                if (GATEUP) {
                    sb = r < BN ? P.s0 : P.s1;
                    row = (int64_t)e * P.N + nt * BN + (r < BN ? r : r - BN);
                } else {
                    sb = P.s0;
                    row = (int64_t)e * P.N + nt * BN + r;
                }
                if (boff < P.K / 16)       // whole pieces: K % 256 == 0 on this path
                    lds_dma16(sb + row * (P.K / 16) + boff, (lds_void*)(dst + (c - lane) * 16));
            }
        }
    };
    // this lane's scale row in the block, per subtile
    int s_lds[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
        const int r = GATEUP ? (ns < 2 ? 0 : BN) + wave * 32 + (ns & 1) * 16 + lcol : wave * 64 + ns * 16 + lcol;
        s_lds[ns] = r * 64 + kq * 2 * CW;
    }
    uint4 a_reg[APT];
    uint4 b_code[NS][CW];
    uint32_t b_scale[NS];
    auto load_stage = [&](int st) {
        const int k0 = st * BK;
#pragma unroll
        for (int i = 0; i < APT; ++i)
            a_reg[i] = a_off[i] >= 0 ? *reinterpret_cast<const uint4*>(P.a + a_off[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
#pragma unroll
            for (int w = 0; w < CW; ++w) b_code[ns][w] = *reinterpret_cast<const uint4*>(cp[ns] + k0 / 2 + 16 * w);
            if constexpr (!SDMA) {
                if constexpr (CW == 1) b_scale[ns] = *reinterpret_cast<const uint16_t*>(sp[ns] + k0 / 16);
                else b_scale[ns] = *reinterpret_cast<const uint32_t*>(sp[ns] + k0 / 16);
            }
        }
    };
    // block 0 before stage 0's loads: waiting for those (in order) covers it
    load_scale_block(0);
    load_stage(0);
    for (int st = 0; st < nst; ++st) {
        uint8_t* buf = smem + (st & 1) * (kRows * kLdsRow);
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int c = tid + kThreads * i;
            *reinterpret_cast<uint4*>(buf + (c / kRowChunks) * kLdsRow + (c % kRowChunks) * 16) = a_reg[i];
        }
        uint4 cur_code[NS][CW];
        uint32_t cur_scale[NS];
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
#pragma unroll
            for (int w = 0; w < CW; ++w) cur_code[ns][w] = b_code[ns][w];
            if constexpr (!SDMA) cur_scale[ns] = b_scale[ns];
        }
        __syncthreads();
        if constexpr (SDMA) {
            // this stage's scale words; at a block's first stage the next
            // block's DMA goes out ahead of the next stage's loads (the
            // wave's wait for those loads, in order, covers the DMA, and
            // the barrier of the next block's first stage publishes it)
            const int b = st / SB, j = st - b * SB;
            const uint8_t* blk = sscale + (b & 1) * kSBlock + j * (BK / 16);
#pragma unroll
            for (int ns = 0; ns < NS; ++ns)
                cur_scale[ns] = CW == 1 ? (uint32_t) * reinterpret_cast<const uint16_t*>(blk + s_lds[ns])
                                        : *reinterpret_cast<const uint32_t*>(blk + s_lds[ns]);
            if (j == 0 && (b + 1) * SB < nst) load_scale_block(b + 1);
        }
        if (st + 1 < nst) load_stage(st + 1);
        // decoded weights of subtile ns at k-step s (8 codes times their
        // group's E4M3 scale, exact in bf16)
        auto decode_sub = [&](int ns, int s) {
            const uint4 cw4 = cur_code[ns][s >> 2];
            const int sw = s & 3;
            const uint32_t word = sw == 0 ? cw4.x : sw == 1 ? cw4.y : sw == 2 ? cw4.z : cw4.w;
            // the group of k-step s: byte s / 2 of the lane's scale word
            const int sb = s >> 1;
            const float sc = sb == 0 ? e4m3_byte_to_f32<0>(cur_scale[ns])
                           : sb == 1 ? e4m3_byte_to_f32<1>(cur_scale[ns])
                           : sb == 2 ? e4m3_byte_to_f32<2>(cur_scale[ns])
                                     : e4m3_byte_to_f32<3>(cur_scale[ns]);
            return decode8(word, sc);
        };
        auto read_frag = [&](int ms, int s) {
            return *reinterpret_cast<const bf16x8*>(buf + (ms * 16 + lcol) * kLdsRow + kq * 64 * CW + s * 16);
        };
        // Each subtile's MFMAs are interleaved with the decode of the next
        // subtile (the last one's with the next k-step's first), and the next
        // k-step's activation fragments are read during this one's MFMAs, so
        // the matrix pipe of a SIMD and its vector ALU work at the same time.
        bf16x8 af[2][MSR];
#pragma unroll
        for (int ms = 0; ms < MSR; ++ms) af[0][ms] = read_frag(ms, 0);
        bf16x8 bnext = decode_sub(0, 0);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
            for (int ns = 0; ns < NS; ++ns) {
                const bf16x8 bf = bnext;
                if (ns + 1 < NS) bnext = decode_sub(ns + 1, s);
                else if (s + 1 < KSTEPS) bnext = decode_sub(0, s + 1);
#pragma unroll
                for (int ms = 0; ms < MSR; ++ms)
                    acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s & 1][ms], bf, acc[ms][ns], 0, 0, 0);
#pragma unroll
                for (int i = 0; i < MSR; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 18 / MSR, 0);       // VALU
                }
                if (ns == 1 && s + 1 < KSTEPS) {
#pragma unroll
                    for (int ms = 0; ms < MSR; ++ms) af[(s + 1) & 1][ms] = read_frag(ms, s + 1);
                }
            }
        }
    }

    // epilogue: lane holds rows 4*kq + i (i < 4) of each 16-row subtile, column lcol
    if (GATEUP) {
        const float gg = P.g0[e] * P.gmul, gu = P.g1[e] * P.gmul;
        uint16_t* h = reinterpret_cast<uint16_t*>(P.out);
#pragma unroll
        for (int ms = 0; ms < MSR; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = ms * 16 + kq * 4 + i;
                if (r < rows) {
#pragma unroll
                    for (int ns = 0; ns < 2; ++ns) {
                        const float a = gg * acc[ms][ns][i];
                        const float b = gu * acc[ms][ns + 2][i];
                        const int col = nt * BN + wave * 32 + ns * 16 + lcol;
                        const int64_t idx = (int64_t)(p0 + r) * P.N + col;
                        const float v = silu(a) * b;
                        if (P.hf) P.hf[idx] = v;
                        else h[idx] = f32_to_bf16_rne(v);
                    }
                }
            }
    } else {
        const float gd = P.g0[e] * P.gmul;
        uint16_t* y = reinterpret_cast<uint16_t*>(P.out);
#pragma unroll
        for (int ms = 0; ms < MSR; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = ms * 16 + kq * 4 + i;
                if (r < rows) {
#pragma unroll
                    for (int ns = 0; ns < NS; ++ns) {
                        const int col = nt * BN + wave * 64 + ns * 16 + lcol;
                        y[(int64_t)(p0 + r) * P.N + col] = f32_to_bf16_rne(gd * acc[ms][ns][i]);
                    }
                }
            }
    }
}

// Persistent grouped GEMM over tiles of up to BM rows (each computed by
// grouped_tile with the row subtiles its rows need).
template <bool GATEUP, int BM, int BK, int NW, bool SDMA>
__global__ void __launch_bounds__(NW * kWave, (gemm_wg_per_cu<BM, NW>())) k_grouped_gemm(GemmParams P) {
    constexpr int kThreads = NW * kWave;
    constexpr int MS = BM / 16;                 // row subtiles of a full tile
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ int s_prefix[MOE_MAX_EXPERTS + 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // tiles per expert -> exclusive prefix (wave 0, DPP scan over lane runs)
    for (int e = tid; e < P.E; e += kThreads) s_prefix[e] = ((P.counts[e] + BM - 1) / BM) * P.ntn;
    __syncthreads();
    if (wave == 0) {
        const int per = (P.E + kWave - 1) / kWave, b = lane * per;
        int local = 0;
        for (int i = 0; i < per; ++i)
            if (b + i < P.E) local += s_prefix[b + i];
        const int incl = wave_inclusive_scan_dpp(local);
        int run = incl - local;
        for (int i = 0; i < per; ++i)
            if (b + i < P.E) {
                const int c = s_prefix[b + i];
                s_prefix[b + i] = run;
                run += c;
            }
        if (lane == kWave - 1) s_prefix[P.E] = incl;
    }
    __syncthreads();
    const int total = s_prefix[P.E];

    const int G = gridDim.x;
    const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
    const bool remap = (G & 7) == 0;

    for (int it = 0;; ++it) {
        const int tile = it * G + (remap ? xcd * (G >> 3) + q : (int)blockIdx.x);
        if (tile >= total) break;
        // tile -> expert (largest e with prefix[e] <= tile)
        int lo = 0, hi = P.E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_prefix[mid] <= tile) lo = mid; else hi = mid - 1;
        }
        const int e = __builtin_amdgcn_readfirstlane(lo);
        const int L = tile - s_prefix[e];
        const int ne = P.counts[e];
        const int mte = (ne + BM - 1) / BM;
        const int full = mte / kMGroup;
        int mt, nt;
        if (L < full * kMGroup * P.ntn) {
            const int g = L / (kMGroup * P.ntn), r = L % (kMGroup * P.ntn);
            nt = r / kMGroup;
            mt = g * kMGroup + r % kMGroup;
        } else {
            const int r = L - full * kMGroup * P.ntn, last = mte - full * kMGroup;
            nt = r / last;
            mt = full * kMGroup + r % last;
        }
        nt = __builtin_amdgcn_readfirstlane(nt);
        const int p0 = __builtin_amdgcn_readfirstlane(P.offsets[e] + mt * BM);
        const int rows = __builtin_amdgcn_readfirstlane(min(BM, ne - mt * BM));
        // the tile's 16-row subtiles: half, three quarters or all of BM
        const int need = (rows + 15) >> 4;
        uint8_t* sscale = smem + 2 * BM * (BK * 2 + 16);   // after the activation buffers
        if (need <= MS / 2) grouped_tile<GATEUP, BK, NW, SDMA, MS / 2>(P, smem, sscale, e, nt, p0, rows);
        else if (need <= 3 * MS / 4) grouped_tile<GATEUP, BK, NW, SDMA, 3 * MS / 4>(P, smem, sscale, e, nt, p0, rows);
        else grouped_tile<GATEUP, BK, NW, SDMA, MS>(P, smem, sscale, e, nt, p0, rows);
        __syncthreads();   // LDS buffers are rewritten by the next tile
    }
}

// out[t, c..c+7] = bf16( sum_j w[t,j] * y[slot_pos[t*k+j], c..c+7] ), j ascending.
__global__ void __launch_bounds__(256) k_combine(const uint16_t* __restrict__ y, const float* __restrict__ topk_w,
                                                 const int32_t* __restrict__ slot_pos, int T, int H, int k,
                                                 uint16_t* __restrict__ out) {
    const int t = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * 8;
    if (c >= H) return;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
        const int slot = t * k + j;
        const float w = topk_w[slot];
        const uint4 v = *reinterpret_cast<const uint4*>(y + (int64_t)slot_pos[slot] * H + c);
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += w * bf16_bits_to_f32(u[i] & 0xFFFFu);
            acc[2 * i + 1] += w * bf16_bits_to_f32(u[i] >> 16);
        }
    }
    uint4 o;
    o.x = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
    o.y = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
    o.z = (uint32_t)f32_to_bf16_rne(acc[4]) | ((uint32_t)f32_to_bf16_rne(acc[5]) << 16);
    o.w = (uint32_t)f32_to_bf16_rne(acc[6]) | ((uint32_t)f32_to_bf16_rne(acc[7]) << 16);
    *reinterpret_cast<uint4*>(out + (int64_t)t * H + c) = o;
}

int num_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

int persistent_grid(int64_t tiles_ub, int per_cu = 2) {
    int64_t g = std::min<int64_t>(tiles_ub, (int64_t)num_cus() * per_cu);
    if (g >= 8) g = (g + 7) / 8 * 8;
    return (int)std::max<int64_t>(g, 1);
}

// Scales through LDS where a row's scale bytes split into whole 16-byte
// pieces (K % 256 == 0) and the LDS allows: every tile height but 32 rows,
// whose three workgroups per CU would not fit the scale blocks beside their
// activation buffers.
template <int BM> constexpr bool gemm_sdma_fits() { return BM >= 64; }

template <bool GATEUP, int BM, int BK, int NW, bool SDMA>
moe_status launch_gemm_s(GemmParams P, int64_t slots, int E, hipStream_t s) {
    constexpr int BN = (GATEUP ? 32 : 64) * NW;
    P.ntn = P.N / BN;
    const int64_t tiles_ub = (slots / BM + std::min<int64_t>(E, slots)) * P.ntn;
    // activation double buffer, then the scale blocks' double buffer
    const size_t shmem = 2 * BM * (BK * 2 + 16) + (SDMA ? 2 * 64 * NW * 64 : 0);
    auto kern = &k_grouped_gemm<GATEUP, BM, BK, NW, SDMA>;
    if (allow_dynamic_lds(reinterpret_cast<const void*>(kern), shmem) != MOE_OK) return MOE_ERR_HIP;
    const char* name = GATEUP ? "gemm_gateup" : "gemm_down";
    MOE_LAUNCH(name, (k_grouped_gemm<GATEUP, BM, BK, NW, SDMA>),
               dim3(persistent_grid(tiles_ub, gemm_wg_per_cu<BM, NW>())), dim3(NW * kWave), shmem, s, P);
    return MOE_OK;
}

template <bool GATEUP, int BM, int BK, int NW>
moe_status launch_gemm(GemmParams P, int64_t slots, int E, hipStream_t s) {
    if constexpr (gemm_sdma_fits<BM>())
        if (P.K % 256 == 0) return launch_gemm_s<GATEUP, BM, BK, NW, true>(P, slots, E, s);
    return launch_gemm_s<GATEUP, BM, BK, NW, false>(P, slots, E, s);
}

// Row tile by the mean rows per touched expert.  A weight tile is decoded once
// per row tile, so tiles that hold a whole typical expert pay off even with
// padding: at 1K tokens, top-8 of 256 (about 32 rows per expert, many with
// 33-45) 64-row tiles take the layer from 1.61 to 1.32 ms against 32-row
// tiles; 128-row tiles (one workgroup per CU) take 2.38 ms.  The 64-row
// tiles use eight waves (twice the columns per tile, half the re-reads of
// the gathered activation rows) and 256-wide K stages (whole 128-byte weight
// lines per stage) where the shape allows.  Measured on MI355X at 1K tokens
// with tiles cut to their rows' subtiles and the decode interleaved with the
// MFMAs: gate/up 615 us with eight waves and 256-wide stages (four waves:
// 704 us, or 789 us with 128-wide stages), down 325 us (four waves with
// 128-wide stages: 357 us).
template <bool GATEUP>
moe_status launch_gemm_bm(const GemmParams& P, int64_t slots, int E, hipStream_t s) {
    const int64_t avg = slots / std::max<int64_t>(1, std::min<int64_t>(E, slots));
    if (avg <= 16) return launch_gemm<GATEUP, 32, 128, 4>(P, slots, E, s);
    if (avg <= 64) {
        if (GATEUP && P.K % 256 == 0 && P.N % 256 == 0) return launch_gemm<true, 64, 256, 8>(P, slots, E, s);
        if (!GATEUP && P.K % 256 == 0 && P.N % 512 == 0) return launch_gemm<false, 64, 256, 8>(P, slots, E, s);
        return launch_gemm<GATEUP, 64, 128, 4>(P, slots, E, s);
    }
    return launch_gemm<GATEUP, 128, 128, 4>(P, slots, E, s);
}

}  // namespace

moe_status launch_gateup_grouped(const FwdArgs& a, hipStream_t s) {
    const int64_t slots = (int64_t)a.T * a.k;
    GemmParams g{};
    g.a = a.x;
    g.sorted_slots = a.sorted_slots;
    g.topk = a.k;
    g.K = a.H;
    g.N = a.I;
    g.E = a.E;
    g.c0 = a.gate->codes; g.s0 = a.gate->scales; g.g0 = a.gate->global_scale;
    g.c1 = a.up->codes;   g.s1 = a.up->scales;   g.g1 = a.up->global_scale;
    g.counts = a.counts;
    g.offsets = a.offsets;
    g.out = a.h;
    g.gmul = a.xs;
    g.hf = a.hf;
    return launch_gemm_bm<true>(g, slots, a.E, s);
}

moe_status launch_down_grouped(const FwdArgs& a, hipStream_t s) {
    const int64_t slots = (int64_t)a.T * a.k;
    GemmParams d{};
    d.a = a.h;
    d.sorted_slots = a.sorted_slots;
    d.topk = a.k;
    d.K = a.I;
    d.N = a.H;
    d.E = a.E;
    d.c0 = a.down->codes; d.s0 = a.down->scales; d.g0 = a.down->global_scale;
    d.counts = a.counts;
    d.offsets = a.offsets;
    d.out = a.y;
    d.gmul = a.hs;
    d.hf = nullptr;
    return launch_gemm_bm<false>(d, slots, a.E, s);
}

moe_status launch_combine(const FwdArgs& a, hipStream_t s) {
    MOE_LAUNCH("combine", k_combine, dim3((a.H + 2047) / 2048, a.T), dim3(256), 0, s, (const uint16_t*)a.y, a.topk_w,
               a.slot_pos, a.T, a.H, a.k, a.out);
    return MOE_OK;
}

}  // namespace moe
