// Prefill-shape grouped GEMMs, software-pipelined through LDS.
//
// Same arithmetic as k_grouped_gemm (moe_prefill.hip): weights decode
// exactly to bf16 (E2M1 * E4M3), bf16 MFMA with fp32 accumulation, the FP32
// global scale in the epilogue, SwiGLU fused into the gate/up epilogue.  The
// difference is the tile, 128 rows x 512 weight columns (gate/up: 256 gate +
// 256 up), which halves the re-reads of the gathered activation rows per
// flop, and how the operands reach the matrix cores:
//   * every operand of a K stage (BK = 64) -- the tile's 128 activation
//     rows, the packed codes of its 512 weight columns and their E4M3 scales
//     -- goes from memory straight to LDS with gfx950 LDS-DMA
//     (global_load_lds), so no register holds data in flight and every wait
//     is an explicit vmcnt;
//   * a ring of kStages stages keeps kStages - 1 stages in flight while one
//     is computed, across tile boundaries (a workgroup walks its tiles as one
//     sequence of (tile, stage) steps);
//   * LDS layouts are XOR-swizzled in 16-byte units so that the MFMA
//     fragment reads (8 consecutive lanes, 8 consecutive rows or columns)
//     hit distinct banks;
//   * 16-row subtiles past the tile's last row skip their MFMAs, so a tile of
//     an expert with few tokens costs what its rows need.
// The K order inside a stage is permuted identically for both operands:
// lane group q of an MFMA takes k = 16 q + 8 s .. 16 q + 8 s + 7 at k-step
// s, so one 8-byte read gives a lane its 16 codes (one E4M3 group) for both
// k-steps.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kPT = 256;                        // threads (4 waves)
constexpr int kBM = 128;                        // rows per tile
constexpr int kBN = 512;                        // weight columns per tile (gate/up: 256 + 256)
constexpr int kNS = 8;                          // 16-column subtiles per wave (a wave owns kBN / 4 columns)
constexpr int kBK = 64;                         // K per stage
constexpr int kStages = 4;                      // LDS ring
constexpr int kAhead = kStages - 1;             // stages in flight while one is computed
constexpr int kABytes = kBM * kBK * 2;          // 16 KiB activations
constexpr int kBBytes = kBN * kBK / 2;          // 16 KiB codes
constexpr int kSBytes = kBN * kBK / 16;         // 2 KiB scales
constexpr int kStageBytes = kABytes + kBBytes + kSBytes;
constexpr int kMGroup = 8;                      // row tiles per scheduling group
// vector-memory operations one wave issues per stage: 4 activation, 4 code
// and 2 scale LDS-DMA
constexpr int kOpsPerStage = 10;

struct PipeParams {
    const uint16_t* a;          // gate/up: x [T][K]; down: h [T*k][K]
    const int32_t* sorted_slots;
    int topk;
    int K, N, E;
    const uint8_t *c0, *s0;     // gate (gate/up) or down
    const float* g0;
    const uint8_t *c1, *s1;     // up (gate/up only)
    const float* g1;
    const int32_t* counts;
    const int32_t* offsets;
    void* out;                  // gate/up: h bf16 [T*k][N]; down: y fp32 [T*k][N]
    int ntn;                    // column tiles per expert
};

struct Tile {
    int e, p0, rows, nt;
};

__device__ __forceinline__ bf16x8 decode8s(uint32_t word, float s) {
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

// Tile t of the launch: expert, first sorted row, rows, column tile.  Tiles
// are numbered expert by expert (prefix over experts in s_prefix) and, inside
// an expert, in groups of kMGroup row tiles x all column tiles.
__device__ __forceinline__ Tile pipe_tile(const PipeParams& P, const int* s_prefix, const int* s_cnt,
                                          const int* s_off, int t) {
    int lo = 0, hi = P.E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_prefix[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int e = lo, L = t - s_prefix[e], ne = s_cnt[e];
    const int mte = (ne + kBM - 1) / kBM, full = mte / kMGroup;
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
    Tile d;
    d.e = e;
    d.p0 = s_off[e] + mt * kBM;
    d.rows = min(kBM, ne - mt * kBM);
    d.nt = nt;
    return d;
}

// Wait until at most n (0 .. kAhead - 1 stages) of this wave's
// vector-memory operations are outstanding, then a workgroup barrier that
// also waits for this wave's LDS reads (the ring slot about to be refilled
// is no longer read).
__device__ __forceinline__ void stage_barrier(int stages_after) {
    switch (stages_after) {
        case 0: wait_vmem_at_most<0>(); break;
        case 1: wait_vmem_at_most<1 * kOpsPerStage>(); break;
        default: wait_vmem_at_most<2 * kOpsPerStage>(); break;
    }
    wait_lds_barrier();
}
static_assert(kAhead == 3, "stage_barrier covers up to two stages after the awaited one");

template <bool GATEUP>
__global__ void __launch_bounds__(kPT, 1) k_gemm_pipe(PipeParams P) {
    extern __shared__ __align__(16) uint8_t ring[];          // kStages x kStageBytes
    __shared__ int s_prefix[MOE_MAX_EXPERTS + 1];
    __shared__ int s_cnt[MOE_MAX_EXPERTS], s_off[MOE_MAX_EXPERTS];   // per expert: rows, first sorted row
    __shared__ __align__(16) int32_t s_rows[2][128];          // sorted-slot values of two tiles (gate/up)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lcol = lane & 15, kq = lane >> 4;

    // tiles per expert -> exclusive prefix (row tiles x column tiles)
    for (int e = tid; e < P.E; e += kPT) {
        const int c = P.counts[e];
        s_cnt[e] = c;
        s_off[e] = P.offsets[e];
        s_prefix[e] = ((c + kBM - 1) / kBM) * P.ntn;
    }
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

    // this workgroup's tiles: it * G + slot, slot spreading consecutive
    // tiles over the XCDs' L2s in contiguous runs
    const int G = gridDim.x;
    const int slot = (G & 7) == 0 ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : (int)blockIdx.x;
    const int ntiles = total > slot ? (total - slot + G - 1) / G : 0;
    const int nst = P.K / kBK;
    const int64_t nsteps = (int64_t)ntiles * nst;

    // per-lane sources of the tile being prefetched
    int64_t a_off[4];               // activation row byte offsets (4 rows per lane)
    const uint8_t* b_src[4];        // code column bases (4 DMA per stage)
    const uint8_t* s_src[2];        // scale column bases (2 DMA per stage)
    int pf_tile = -1;

    // gate/up: the sorted-slot values of tile j into s_rows[buf] (two dword
    // DMAs by wave 0; lanes past the tile's rows read its first slot)
#define MOE_PIPE_ROWS(j, buf)                                                                   \
    do {                                                                                        \
        if (GATEUP && wave == 0 && (j) < ntiles) {                                              \
            const Tile d_ = pipe_tile(P, s_prefix, s_cnt, s_off, (j) * G + slot);                             \
            _Pragma("unroll") for (int h_ = 0; h_ < 2; ++h_) {                                  \
                const int r_ = 64 * h_ + lane;                                                  \
                lds_dma4(P.sorted_slots + d_.p0 + (r_ < d_.rows ? r_ : 0),                      \
                         (lds_void*)&s_rows[buf][64 * h_]);                                     \
            }                                                                                   \
        }                                                                                       \
    } while (0)

    // sources of tile j for this lane's DMAs
#define MOE_PIPE_ENTER(j)                                                                       \
    do {                                                                                        \
        const Tile d_ = pipe_tile(P, s_prefix, s_cnt, s_off, (j) * G + slot);                                 \
        _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) {                                      \
            const int u_ = (wave * 4 + i_) * 64 + lane;                                         \
            const int row_ = min(u_ >> 3, d_.rows - 1);   /* past the tile: repeat its last row */ \
            const int64_t src_row_ = GATEUP ? (int64_t)(s_rows[(j) & 1][row_] / P.topk) : (int64_t)(d_.p0 + row_); \
            a_off[i_] = src_row_ * P.K * 2;                                                     \
        }                                                                                       \
        _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) {                                      \
            const int u_ = (wave * 4 + i_) * 64 + lane;                                         \
            const int col_ = u_ >> 1, chunk_ = (u_ & 1) ^ ((col_ >> 3) & 1);                    \
            const uint8_t* cb_ = GATEUP ? (col_ < kBN / 2 ? P.c0 : P.c1) : P.c0;                \
            const int64_t n_ = (int64_t)d_.e * P.N +                                            \
                               (GATEUP ? d_.nt * (kBN / 2) + (col_ & (kBN / 2 - 1)) : d_.nt * kBN + col_); \
            b_src[i_] = cb_ + n_ * (P.K / 2) + 16 * chunk_;                                     \
        }                                                                                       \
        _Pragma("unroll") for (int i_ = 0; i_ < 2; ++i_) {                                      \
            const int col_ = (wave * 2 + i_) * 64 + lane;                                       \
            const uint8_t* sb_ = GATEUP ? (col_ < kBN / 2 ? P.s0 : P.s1) : P.s0;                \
            const int64_t n_ = (int64_t)d_.e * P.N +                                            \
                               (GATEUP ? d_.nt * (kBN / 2) + (col_ & (kBN / 2 - 1)) : d_.nt * kBN + col_); \
            s_src[i_] = sb_ + n_ * (P.K / 16);                                                  \
        }                                                                                       \
        pf_tile = (j);                                                                          \
    } while (0)

    // the loads of step g (tile g / nst, stage g % nst) into its ring slot
#define MOE_PIPE_ISSUE(g)                                                                       \
    do {                                                                                        \
        const int j_ = (int)((g) / nst), st_ = (int)((g) - (int64_t)j_ * nst);                  \
        if (j_ != pf_tile) {                                                                    \
            if (GATEUP && nst <= kAhead) {  /* short K: the row table may still be in flight */ \
                wait_all_memory();                                                              \
                __builtin_amdgcn_s_barrier();                                                   \
            }                                                                                   \
            MOE_PIPE_ENTER(j_);                                                                 \
            MOE_PIPE_ROWS(j_ + 1, (j_ + 1) & 1);                                                \
        }                                                                                       \
        uint8_t* base_ = ring + (int)((g) % kStages) * kStageBytes;                             \
        const int k0_ = st_ * kBK;                                                              \
        _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) {                                      \
            const int u_ = (wave * 4 + i_) * 64 + lane;                                         \
            const int row_ = u_ >> 3, c_ = (u_ & 7) ^ (row_ & 7);                               \
            const uint8_t* src_ = reinterpret_cast<const uint8_t*>(P.a) + a_off[i_] + k0_ * 2 + 16 * c_; \
            lds_dma16(src_, (lds_void*)(base_ + (wave * 4 + i_) * 1024));                        \
        }                                                                                       \
        _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                        \
            lds_dma16(b_src[i_] + k0_ / 2, (lds_void*)(base_ + kABytes + (wave * 4 + i_) * 1024)); \
        _Pragma("unroll") for (int i_ = 0; i_ < 2; ++i_)                                        \
            lds_dma4(s_src[i_] + k0_ / 16, (lds_void*)(base_ + kABytes + kBBytes + (wave * 2 + i_) * 256)); \
    } while (0)

    // prologue: row tables of the first two tiles, then the first stages
    if (GATEUP) {
        MOE_PIPE_ROWS(0, 0);
        MOE_PIPE_ROWS(1, 1);
        wait_all_memory();
        __syncthreads();
    }
    for (int64_t g = 0; g < (nsteps < kAhead ? nsteps : (int64_t)kAhead); ++g) MOE_PIPE_ISSUE(g);

    // columns of this wave's subtiles within the tile's kBN: gate/up waves
    // own kBN / 8 gate and the same kBN / 8 up columns (SwiGLU pairs them)
    int colb[kNS];
#pragma unroll
    for (int ns = 0; ns < kNS; ++ns)
        colb[ns] = GATEUP ? (ns < kNS / 2 ? (kBN / 8) * wave + 16 * ns : kBN / 2 + (kBN / 8) * wave + 16 * (ns - kNS / 2))
                          : (kBN / 4) * wave + 16 * ns;

#pragma unroll 1
    for (int j = 0; j < ntiles; ++j) {
        const Tile cur = pipe_tile(P, s_prefix, s_cnt, s_off, j * G + slot);
        floatx4 acc[8][kNS];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int n = 0; n < kNS; ++n) acc[i][n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int st = 0; st < nst; ++st) {
            const int64_t g = (int64_t)j * nst + st;
            {
                const int64_t after = nsteps - 1 - g;
                stage_barrier(after < kAhead - 1 ? (int)after : kAhead - 1);
            }
            if (g + kAhead < nsteps) MOE_PIPE_ISSUE(g + kAhead);

            const uint8_t* base = ring + (int)(g % kStages) * kStageBytes;
            const uint8_t* Bs = base + kABytes;
            const uint8_t* Ss = Bs + kBBytes;
            uint2 cw[kNS];
            float sc[kNS];
#pragma unroll
            for (int ns = 0; ns < kNS; ++ns) {
                const int col = colb[ns] + lcol;
                cw[ns] = *reinterpret_cast<const uint2*>(Bs + col * 32 + 16 * ((kq >> 1) ^ ((col >> 3) & 1)) + 8 * (kq & 1));
                sc[ns] = e4m3_to_f32(Ss[col * 4 + kq]);
            }
            // the stage's activation fragments, both k-steps, up front
            bf16x8 af[2][8];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int ms = 0; ms < 8; ++ms) {
                    const int row = ms * 16 + lcol;
                    af[ks][ms] = *reinterpret_cast<const bf16x8*>(base + row * 128 + 16 * ((2 * kq + ks) ^ (row & 7)));
                }
            // column by column: the decode of the next column overlaps the
            // MFMAs of this one
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int ns = 0; ns < kNS; ++ns) {
                    const bf16x8 bf = decode8s(ks ? cw[ns].y : cw[ns].x, sc[ns]);
#pragma unroll
                    for (int ms = 0; ms < 8; ++ms)
                        acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks][ms], bf, acc[ms][ns], 0, 0, 0);
                }
            // issue order: each MFMA followed by two VALU instructions (the
            // next column's decode), so the matrix pipe never waits for it
#pragma unroll
            for (int i = 0; i < 2 * kNS * 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // two VALU
            }
        }

        // epilogue: lane holds rows 4 kq + i (i < 4) of each 16-row subtile, column lcol
        if (GATEUP) {
            const float gg = P.g0[cur.e], gu = P.g1[cur.e];
            uint16_t* h = reinterpret_cast<uint16_t*>(P.out);
#pragma unroll
            for (int ms = 0; ms < 8; ++ms)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = ms * 16 + kq * 4 + i;
                    if (r < cur.rows) {
#pragma unroll
                        for (int ns = 0; ns < kNS / 2; ++ns) {
                            const float av = gg * acc[ms][ns][i];
                            const float bv = gu * acc[ms][ns + kNS / 2][i];
                            const int col = cur.nt * (kBN / 2) + (kBN / 8) * wave + 16 * ns + lcol;
                            h[(int64_t)(cur.p0 + r) * P.N + col] = f32_to_bf16_rne(silu(av) * bv);
                        }
                    }
                }
        } else {
            const float gd = P.g0[cur.e];
            float* y = reinterpret_cast<float*>(P.out);
#pragma unroll
            for (int ms = 0; ms < 8; ++ms)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = ms * 16 + kq * 4 + i;
                    if (r < cur.rows) {
#pragma unroll
                        for (int ns = 0; ns < kNS; ++ns) {
                            const int col = cur.nt * kBN + (kBN / 4) * wave + 16 * ns + lcol;
                            y[(int64_t)(cur.p0 + r) * P.N + col] = gd * acc[ms][ns][i];
                        }
                    }
                }
        }
    }
#undef MOE_PIPE_ROWS
#undef MOE_PIPE_ENTER
#undef MOE_PIPE_ISSUE
}

int cu_count_pipe() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

template <bool GATEUP>
moe_status launch_pipe(const PipeParams& P, int64_t slots, hipStream_t s) {
    const size_t shmem = (size_t)kStages * kStageBytes;
    if (allow_dynamic_lds(reinterpret_cast<const void*>(&k_gemm_pipe<GATEUP>), shmem) != MOE_OK) return MOE_ERR_HIP;
    const int64_t tiles_ub = (slots / kBM + std::min<int64_t>(P.E, slots)) * P.ntn;
    int64_t g = std::min<int64_t>(tiles_ub, cu_count_pipe());
    if (g >= 8) g = g / 8 * 8;
    g = std::max<int64_t>(g, 1);
    MOE_LAUNCH(GATEUP ? "gemm_gateup" : "gemm_down", k_gemm_pipe<GATEUP>, dim3((unsigned)g), dim3(kPT), shmem, s, P);
    return MOE_OK;
}

}  // namespace

bool prefill_pipe_supported(int H, int I) { return H % kBN == 0 && I % (kBN / 2) == 0 && I % kBK == 0; }

moe_status launch_gateup_pipe(const FwdArgs& a, hipStream_t s) {
    PipeParams g{};
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
    g.ntn = a.I / (kBN / 2);
    return launch_pipe<true>(g, (int64_t)a.T * a.k, s);
}

moe_status launch_down_pipe(const FwdArgs& a, hipStream_t s) {
    PipeParams d{};
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
    d.ntn = a.H / kBN;
    return launch_pipe<false>(d, (int64_t)a.T * a.k, s);
}

}  // namespace moe
