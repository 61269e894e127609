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
//     (those in blocks of four stages) -- goes from memory straight to LDS
//     with gfx950 LDS-DMA (global_load_lds), so no register holds data in
//     flight and every wait is an explicit vmcnt;
//   * a ring of kStages stages keeps kStages - 1 stages in flight while one
//     is computed, across tile boundaries (a workgroup walks its tiles as one
//     sequence of (tile, stage) steps);
//   * eight waves, two per SIMD: each owns 64 weight columns for all 128
//     rows (128 accumulator registers), so the decode of one wave's codes
//     and its LDS reads overlap the other wave's MFMAs;
//   * LDS layouts are XOR-swizzled in 16-byte units so that the MFMA
//     fragment reads (consecutive lanes on consecutive rows or columns) hit
//     distinct banks.
// The K order inside a stage is permuted identically for both operands:
// lane group q of an MFMA takes k = 16 q + 8 s .. 16 q + 8 s + 7 at k-step
// s, so one 8-byte read gives a lane its 16 codes (one E4M3 group) for both
// k-steps.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kPT = 512;                        // threads: 8 waves, two per SIMD
constexpr int kWaves = kPT / 64;
constexpr int kBN = 512;                        // weight columns per tile (gate/up: 256 + 256)
constexpr int kNS = kBN / kWaves / 16;          // 16-column subtiles per wave (a wave owns 64 columns)
constexpr int kBK = 64;                         // K per stage
constexpr int kStages = 4;                      // LDS ring
constexpr int kAhead = kStages - 1;             // stages in flight while one is computed
// rows per tile, BM = 128 (experts of several hundred rows) or 64 (a few
// dozen): activation bytes of a stage and the ring layout depend on it
template <int BM> constexpr int a_bytes() { return BM * kBK * 2; }   // 16 / 8 KiB activations
constexpr int kBBytes = kBN * kBK / 2;          // 16 KiB codes
// The E4M3 scales travel in blocks of kSBlk stages: 16 bytes of each weight
// row (one 16-byte piece per lane), where one stage's 4 bytes per row would
// cost the load path one request per row for 4 bytes.  Two block buffers: a
// block is issued with its first stage, three stages ahead, when the buffer
// it replaces (two blocks back) is no longer read.
constexpr int kSBlk = 4;                        // stages per scale block
constexpr int kSRowBytes = kSBlk * kBK / 16;    // 16 bytes of a row's scales per block
constexpr int kSBlkBytes = kBN * kSRowBytes;    // 8 KiB
// the ring is three rings, one per operand, so that every LDS read of a
// stage is a per-stage base plus an immediate offset (all below 64 KiB)
constexpr int kARing = 0;
template <int BM> constexpr int b_ring() { return kStages * a_bytes<BM>(); }
template <int BM> constexpr int s_ring() { return b_ring<BM>() + kStages * kBBytes; }
template <int BM> constexpr int ring_bytes() { return s_ring<BM>() + 2 * kSBlkBytes; }
constexpr int kMGroup = 8;                      // row tiles per scheduling group
constexpr int64_t kPipeBM64MaxMeanRows = 96;    // mean rows per touched expert up to which tiles are 64 rows
#ifndef MOE_PIPE_DMA_WAVES
#define MOE_PIPE_DMA_WAVES 4
#endif
// Waves 0 .. kDmaWaves - 1 issue a stage's LDS-DMA operations: 1 KiB
// activation, code and (every kSBlk stages) scale runs.  With 4 (one per SIMD, the
// default) the other wave of each SIMD goes on with its MFMAs while its
// partner issues; all 8 issuing measured 6 % slower on MI355X.
constexpr int kDmaWaves = MOE_PIPE_DMA_WAVES;
template <int BM> constexpr int a_dma() { return a_bytes<BM>() / 1024 / kDmaWaves; }
constexpr int kBDma = kBBytes / 1024 / kDmaWaves;
constexpr int kSDma = kSBlkBytes / 1024 / kDmaWaves;
template <int BM> constexpr int ops_plain() { return a_dma<BM>() + kBDma; }   // a stage without a scale block
template <int BM> constexpr int ops_per_stage() { return ops_plain<BM>() + kSDma; }
constexpr int kDmaCols = kBN / kDmaWaves;       // weight columns one DMA wave brings in
static_assert(a_dma<128>() * kDmaWaves * 1024 == a_bytes<128>() && a_dma<64>() * kDmaWaves * 1024 == a_bytes<64>() &&
              kBDma * 32 == kDmaCols && kSDma * 64 == kDmaCols && kNS == 4, "stage split over the waves");
static_assert(ops_per_stage<64>() <= 8 && ops_per_stage<128>() <= 10, "DMA points per stage");
// point (0 .. 7: after which subtile's MFMAs) at which a DMA wave issues
// op j of a stage; with 8 DMA waves the second wave of each SIMD is offset
// so that the two do not stall on the load queue together
__device__ __forceinline__ constexpr int dma_point(int j, int wave) {
    return kDmaWaves == 4 ? (j < 6 ? j : (j < 8 ? j : j - 2)) : j + (wave >= 4 ? 3 : 0);
}

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
    void* out;                  // gate/up: h bf16 [T*k][N]; down: y bf16 [T*k][N]
    int ntn;                    // column tiles per expert
    float gmul;                 // multiplies the global scales (W4A4 input scale; 1 for W4A16)
    float* hf;                  // gate/up: fp32 h instead of bf16 into out, when set (W4A4)
};

struct Tile {
    int e, p0, rows, nt;
};

// 8 codes (one E2M1 nibble each, k order) times their E4M3 group scale, as
// bf16: the products are exact in bf16, so keeping the top half of each fp32
// product is exact too.
__device__ __forceinline__ bf16x8 decode8s(uint32_t word, float s) {
    const floatx2 p0 = e2m1x2_to_f32<0>(word);
    const floatx2 p1 = e2m1x2_to_f32<1>(word);
    const floatx2 p2 = e2m1x2_to_f32<2>(word);
    const floatx2 p3 = e2m1x2_to_f32<3>(word);
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(__float_as_uint(p0[1] * s), __float_as_uint(p0[0] * s), 0x07060302u);
    r[1] = __builtin_amdgcn_perm(__float_as_uint(p1[1] * s), __float_as_uint(p1[0] * s), 0x07060302u);
    r[2] = __builtin_amdgcn_perm(__float_as_uint(p2[1] * s), __float_as_uint(p2[0] * s), 0x07060302u);
    r[3] = __builtin_amdgcn_perm(__float_as_uint(p3[1] * s), __float_as_uint(p3[0] * s), 0x07060302u);
    return __builtin_bit_cast(bf16x8, r);
}

// LDS slot of 16-byte unit c of activation row r: c ^ a_swz(r).  A
// fragment read (16-byte lanes, rows r0 .. r0 + 15 of one unit) then hits
// distinct banks whether the LDS serves 8 or 16 such lanes per cycle: the
// swizzle differs across any 8 consecutive rows and across the 8 even (or
// odd) rows of 16.
__device__ __forceinline__ int a_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Tile t of the launch: expert, first sorted row, rows, column tile.  Tiles
// are numbered expert by expert (prefix over experts in s_prefix) and, inside
// an expert, in groups of kMGroup row tiles x all column tiles.
template <int BM>
__device__ __forceinline__ Tile pipe_tile(const PipeParams& P, const int* s_prefix, const int* s_cnt,
                                          const int* s_off, int t) {
    int lo = 0, hi = P.E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_prefix[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int e = lo, L = t - s_prefix[e], ne = s_cnt[e];
    const int mte = (ne + BM - 1) / BM, full = mte / kMGroup;
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
    d.p0 = s_off[e] + mt * BM;
    d.rows = min(BM, ne - mt * BM);
    d.nt = nt;
    return d;
}

// Before step g a DMA wave waits until only the operations of the steps
// issued after g (0 .. kAhead - 1 of them) are outstanding -- a step whose
// stage opens a scale block has kSDma more -- then every wave meets at a
// workgroup barrier that also waits for its LDS reads (the ring slot about
// to be refilled is no longer read).
template <int BM>
__device__ __forceinline__ void stage_barrier(bool dma_wave, int stages_after, int g) {
    if (dma_wave) {
        constexpr int P = ops_plain<BM>(), S = kSDma;
        const bool blk1 = ((g + 1) % kSBlk) == 0, blk2 = ((g + 2) % kSBlk) == 0;
        if (stages_after == 0) wait_vmem_at_most<0>();
        else if (stages_after == 1) {
            if (blk1) wait_vmem_at_most<P + S>();
            else wait_vmem_at_most<P>();
        } else {
            if (blk1 || blk2) wait_vmem_at_most<2 * P + S>();
            else wait_vmem_at_most<2 * P>();
        }
    }
    wait_lds_barrier();
}
static_assert(kAhead == 3, "stage_barrier covers up to two stages after the awaited one");

// One K stage of a wave's 128 x 64 block.  Per k-step the eight activation
// fragments are read once and each of the wave's four weight subtiles is
// decoded once and meets all of them; the decode of the next subtile is
// interleaved with the MFMAs of the current one.  Every 16-row subtile is
// computed, also past a short tile's last row: skipping them would need a
// second copy of the loop, and the two copies' accumulators would no longer
// stay in place.  dma(p), p = 0 .. 7, runs after the p-th subtile's MFMAs:
// a DMA wave issues part of a later stage's loads there, so a stall on a
// full load queue overlaps the MFMAs already issued and the other wave's.
// Lane offsets inside a stage's rings: activation fragment (k-step ks) of
// row lcol (16-row subtile ms adds ms * 2048), codes and scale of column
// lcol of the wave's first subtile (subtile ns adds cb[ns] columns).
struct LaneLds {
    int a[2], b, s;
};

template <bool GATEUP, int MS, class Dma>
__device__ __forceinline__ void stage_mfma(floatx4 (&acc)[MS][kNS], const uint8_t* as, const uint8_t* bs,
                                           const uint8_t* ss, const LaneLds& o, Dma&& dma) {
    // columns of the wave's subtiles relative to its first: gate/up waves
    // own 32 gate columns and the same 32 up columns (SwiGLU pairs them)
    constexpr int cb[kNS] = {0, 16, GATEUP ? kBN / 2 : 32, GATEUP ? kBN / 2 + 16 : 48};
    uint2 cw[kNS];
    float sc[kNS];
#pragma unroll
    for (int ns = 0; ns < kNS; ++ns) {
        cw[ns] = *reinterpret_cast<const uint2*>(bs + o.b + cb[ns] * 32);
        sc[ns] = e4m3_to_f32(ss[o.s + cb[ns] * kSRowBytes]);
    }
    bf16x8 bnext = decode8s(cw[0].x, sc[0]);
    // activation fragments: k-step 0 now, k-step 1 in two halves during the
    // k-step 0 MFMAs (after subtiles 1 and 2), so their LDS latency is hidden
    bf16x8 af[2][MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) af[0][ms] = *reinterpret_cast<const bf16x8*>(as + o.a[0] + ms * 2048);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int ns = 0; ns < kNS; ++ns) {
            const bf16x8 bf = bnext;
            const int nn = ns + 1 < kNS ? ns + 1 : 0;     // next subtile (of the next k-step after the last)
            if (ks == 0 || ns + 1 < kNS) {
                bnext = decode8s((ns + 1 < kNS ? ks : 1) ? cw[nn].y : cw[nn].x, sc[nn]);
                // keep the decode in this subtile's block: dma(p) below is a
                // branch, and the compiler would otherwise sink the decode
                // past it to its use, ahead of the next subtile's MFMAs
                u32x4 pin = __builtin_bit_cast(u32x4, bnext);
                asm volatile("" : "+v"(pin));
                bnext = __builtin_bit_cast(bf16x8, pin);
            }
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
                acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks][ms], bf, acc[ms][ns], 0, 0, 0);
            // each MFMA followed by its share of the next subtile's decode
            // (16 VALU instructions over the MS MFMAs), so the matrix pipe
            // does not wait for it
#pragma unroll
            for (int i = 0; i < MS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 16 / MS, 0);    // VALU
            }
            dma(ks * kNS + ns);
            if (ks == 0 && (ns == 1 || ns == 2)) {
#pragma unroll
                for (int h = 0; h < MS / 2; ++h) {
                    const int ms = (ns - 1) * (MS / 2) + h;
                    af[1][ms] = *reinterpret_cast<const bf16x8*>(as + o.a[1] + ms * 2048);
                }
            }
        }
    }
}

template <bool GATEUP, int BM>
__global__ void __launch_bounds__(kPT, 1) k_gemm_pipe(PipeParams P) {
    constexpr int MS = BM / 16;                               // 16-row subtiles
    constexpr int kABytes = a_bytes<BM>(), kADma = a_dma<BM>(), kOpsPerStage = ops_per_stage<BM>();
    constexpr int kBRing = b_ring<BM>(), kSRing = s_ring<BM>();
    extern __shared__ __align__(16) uint8_t ring[];          // activation, code and scale rings
    __shared__ int s_prefix[MOE_MAX_EXPERTS + 1];
    __shared__ int s_cnt[MOE_MAX_EXPERTS], s_off[MOE_MAX_EXPERTS];   // per expert: rows, first sorted row
    __shared__ __align__(16) int32_t s_rows[2][BM];           // sorted-slot values of two tiles (gate/up)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool dma_wave = wave < kDmaWaves;
    const int lcol = lane & 15, kq = lane >> 4;

    // tiles per expert -> exclusive prefix (row tiles x column tiles)
    for (int e = tid; e < P.E; e += kPT) {
        const int c = P.counts[e];
        s_cnt[e] = c;
        s_off[e] = P.offsets[e];
        s_prefix[e] = ((c + BM - 1) / BM) * P.ntn;
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
    const int nsteps = ntiles * nst;

    // DMA sources of the tile being prefetched: per-lane byte offsets of the
    // activation runs (row and 16-byte unit), and the wave-uniform bases of
    // its code and scale runs (their per-lane offsets never change)
    uint32_t a_vo[kADma];
    const uint8_t* b_base = nullptr;
    const uint8_t* s_base = nullptr;
    const uint32_t b_vo = (uint32_t)((lane >> 1) * (P.K / 2) + 16 * ((lane & 1) ^ ((lane >> 4) & 1)));
    const uint32_t s_vo = (uint32_t)(lane * (P.K / 16));   // scale row of the lane (16-byte piece)
    const int64_t b_step = (int64_t)32 * (P.K / 2), s_step = (int64_t)64 * (P.K / 16);
    // next (tile, stage) to prefetch, its ring slot and its step index
    int iss_j = 0, iss_st = 0, iss_slot = 0, iss_g = 0;

    // gate/up: the sorted-slot values of tile j into s_rows[buf] (two dword
    // DMAs by wave 0; lanes past the tile's rows read its first slot)
#define MOE_PIPE_ROWS(j, buf)                                                                   \
    do {                                                                                        \
        if (GATEUP && wave == 0 && (j) < ntiles) {                                              \
            const Tile d_ = pipe_tile<BM>(P, s_prefix, s_cnt, s_off, (j) * G + slot);               \
            _Pragma("unroll") for (int h_ = 0; h_ < BM / 64; ++h_) {                             \
                const int r_ = 64 * h_ + lane;                                                  \
                lds_dma4(P.sorted_slots + d_.p0 + (r_ < d_.rows ? r_ : 0),                      \
                         (lds_void*)&s_rows[buf][64 * h_]);                                     \
            }                                                                                   \
        }                                                                                       \
    } while (0)

    // sources of tile j for this wave's DMAs (DMA waves)
#define MOE_PIPE_ENTER(j)                                                                       \
    do {                                                                                        \
        const Tile d_ = pipe_tile<BM>(P, s_prefix, s_cnt, s_off, (j) * G + slot);                   \
        const int e_ = __builtin_amdgcn_readfirstlane(d_.e), nt_ = __builtin_amdgcn_readfirstlane(d_.nt); \
        const int rows_ = __builtin_amdgcn_readfirstlane(d_.rows), p0_ = __builtin_amdgcn_readfirstlane(d_.p0); \
        _Pragma("unroll") for (int i_ = 0; i_ < kADma; ++i_) {                                  \
            const int u_ = (wave * kADma + i_) * 64 + lane;                                     \
            const int row_ = min(u_ >> 3, rows_ - 1);   /* past the tile: repeat its last row */ \
            const int src_ = GATEUP ? s_rows[(j) & 1][row_] / P.topk : p0_ + row_;              \
            a_vo[i_] = (uint32_t)src_ * (uint32_t)(P.K * 2) + 16u * (uint32_t)((u_ & 7) ^ a_swz(u_ >> 3)); \
        }                                                                                       \
        /* first column of the wave's code / scale runs within the expert's matrix */         \
        const int64_t n0_ = (int64_t)e_ * P.N + (GATEUP ? nt_ * (kBN / 2) + (wave % (kDmaWaves / 2)) * kDmaCols \
                                                        : nt_ * kBN + wave * kDmaCols);         \
        b_base = (GATEUP && wave >= kDmaWaves / 2 ? P.c1 : P.c0) + n0_ * (P.K / 2);            \
        s_base = (GATEUP && wave >= kDmaWaves / 2 ? P.s1 : P.s0) + n0_ * (P.K / 16);           \
    } while (0)

    // the loads of the next (tile, stage) into its ring slot, by the DMA
    // waves: BEGIN sets up a new tile's sources, OP(p) issues op p (0 .. 3:
    // activation runs, 4 .. 7: code runs, 8, 9: scale runs of the block
    // that the stage opens, if it opens one), END moves on
#define MOE_PIPE_BEGIN()                                                                        \
    do {                                                                                        \
        if (iss_st == 0) {                                                                      \
            if (GATEUP && nst <= kAhead) {  /* short K: the row table may still be in flight */ \
                wait_all_memory();                                                              \
                __builtin_amdgcn_s_barrier();                                                   \
            }                                                                                   \
            MOE_PIPE_ENTER(iss_j);                                                              \
            MOE_PIPE_ROWS(iss_j + 1, (iss_j + 1) & 1);                                          \
        }                                                                                       \
    } while (0)
#define MOE_PIPE_OP(p)                                                                          \
    do {                                                                                        \
        const int k0_ = iss_st * kBK;                                                           \
        if ((p) < kADma) {                                                                      \
            const int i_ = (p);                                                                 \
            lds_dma16_sv(reinterpret_cast<const uint8_t*>(P.a) + k0_ * 2, a_vo[i_],             \
                         (lds_void*)(ring + kARing + iss_slot * kABytes + (wave * kADma + i_) * 1024)); \
        } else if ((p) < kADma + kBDma) {                                                       \
            const int i_ = (p) - kADma;                                                         \
            lds_dma16_sv(b_base + (i_ * b_step + k0_ / 2), b_vo,                                \
                         (lds_void*)(ring + kBRing + iss_slot * kBBytes + (wave * kBDma + i_) * 1024)); \
        } else if (iss_st % kSBlk == 0) {                                                       \
            const int i_ = (p) - kADma - kBDma;                                                 \
            lds_dma16_sv(s_base + (i_ * s_step + k0_ / 16), s_vo,                               \
                         (lds_void*)(ring + kSRing + ((iss_g / kSBlk) & 1) * kSBlkBytes +       \
                                     (wave * kSDma + i_) * 1024));                              \
        }                                                                                       \
    } while (0)
#define MOE_PIPE_END()                                                                          \
    do {                                                                                        \
        iss_slot = (iss_slot + 1) & (kStages - 1);                                              \
        ++iss_g;                                                                                \
        if (++iss_st == nst) {                                                                  \
            iss_st = 0;                                                                         \
            ++iss_j;                                                                            \
        }                                                                                       \
    } while (0)
    static_assert((kStages & (kStages - 1)) == 0, "ring slots wrap with a mask");

    // prologue: row tables of the first two tiles, then the first stages
    if (GATEUP) {
        MOE_PIPE_ROWS(0, 0);
        MOE_PIPE_ROWS(1, 1);
        wait_all_memory();
        __syncthreads();
    }
    if (dma_wave)
        for (int g = 0; g < (nsteps < kAhead ? nsteps : kAhead); ++g) {
            MOE_PIPE_BEGIN();
#pragma unroll
            for (int p = 0; p < kOpsPerStage; ++p) MOE_PIPE_OP(p);
            MOE_PIPE_END();
        }

    // this lane's LDS offsets inside a stage (see LaneLds); the wave's first
    // column is 32 w (gate/up: then 32 up columns at kBN / 2 + 32 w) or 64 w
    LaneLds lo;
    {
        const int col = (GATEUP ? 32 : 64) * wave + lcol;
        lo.a[0] = lcol * 128 + 16 * ((2 * kq) ^ a_swz(lcol));
        lo.a[1] = lcol * 128 + 16 * ((2 * kq + 1) ^ a_swz(lcol));
        lo.b = col * 32 + 16 * ((kq >> 1) ^ ((lcol >> 3) & 1)) + 8 * (kq & 1);
        lo.s = col * kSRowBytes + kq;
    }

    int g = 0;            // (tile, stage) step being computed
#pragma unroll 1
    for (int j = 0; j < ntiles; ++j) {
        const Tile cur = pipe_tile<BM>(P, s_prefix, s_cnt, s_off, j * G + slot);
        // the expert's global scales, by scalar loads: a vector load would be
        // ordered behind the DMA operations in flight, and one still counted
        // as pending across the stage loop makes the compiler wait for all
        // of them inside it
        const int e_cur = __builtin_amdgcn_readfirstlane(cur.e);
        const float g_a = ((const __attribute__((address_space(4))) float*)P.g0)[e_cur] * P.gmul;
        const float g_b = GATEUP ? ((const __attribute__((address_space(4))) float*)P.g1)[e_cur] * P.gmul : 0.0f;
        floatx4 acc[MS][kNS];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int n = 0; n < kNS; ++n) acc[i][n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int st = 0; st < nst; ++st, ++g) {
            {
                const int after = nsteps - 1 - g;
                stage_barrier<BM>(dma_wave, after < kAhead - 1 ? after : kAhead - 1, g);
            }
            // a DMA wave spreads stage g + kAhead's loads over this stage's MFMAs
            const bool issuing = dma_wave && g + kAhead < nsteps;
            if (issuing) MOE_PIPE_BEGIN();   /* before the first op: it may set up a new tile */
            const int rs = g & (kStages - 1);
            stage_mfma<GATEUP, MS>(acc, ring + kARing + rs * kABytes, ring + kBRing + rs * kBBytes,
                               ring + kSRing + ((g / kSBlk) & 1) * kSBlkBytes + (g % kSBlk) * (kBK / 16), lo,
                               [&](int p) {
                if (issuing) {
#pragma unroll
                    for (int j = 0; j < kOpsPerStage; ++j)
                        if (dma_point(j, wave) == p) MOE_PIPE_OP(j);
                }
            });
            if (issuing) MOE_PIPE_END();
        }

        // epilogue: lane holds rows 4 kq + i (i < 4) of each 16-row subtile, column lcol
        if (GATEUP) {
            const float gg = g_a, gu = g_b;
            uint16_t* h = reinterpret_cast<uint16_t*>(P.out);
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = ms * 16 + kq * 4 + i;
                    if (r < cur.rows) {
#pragma unroll
                        for (int ns = 0; ns < kNS / 2; ++ns) {
                            const float av = gg * acc[ms][ns][i];
                            const float bv = gu * acc[ms][ns + kNS / 2][i];
                            const int col = cur.nt * (kBN / 2) + 32 * wave + 16 * ns + lcol;
                            const int64_t idx = (int64_t)(cur.p0 + r) * P.N + col;
                            const float v = silu(av) * bv;
                            if (P.hf) P.hf[idx] = v;
                            else h[idx] = f32_to_bf16_rne(v);
                        }
                    }
                }
        } else {
            const float gd = g_a;
            uint16_t* y = reinterpret_cast<uint16_t*>(P.out);
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = ms * 16 + kq * 4 + i;
                    if (r < cur.rows) {
#pragma unroll
                        for (int ns = 0; ns < kNS; ++ns) {
                            const int col = cur.nt * kBN + 64 * wave + 16 * ns + lcol;
                            y[(int64_t)(cur.p0 + r) * P.N + col] = f32_to_bf16_rne(gd * acc[ms][ns][i]);
                        }
                    }
                }
        }
    }
#undef MOE_PIPE_ROWS
#undef MOE_PIPE_ENTER
#undef MOE_PIPE_BEGIN
#undef MOE_PIPE_OP
#undef MOE_PIPE_END
}

int cu_count_pipe() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

template <bool GATEUP, int BM>
moe_status launch_pipe_bm(const PipeParams& P, int64_t slots, hipStream_t s) {
    const size_t shmem = (size_t)ring_bytes<BM>();
    if (allow_dynamic_lds(reinterpret_cast<const void*>(&k_gemm_pipe<GATEUP, BM>), shmem) != MOE_OK)
        return MOE_ERR_HIP;
    const int64_t tiles_ub = (slots / BM + std::min<int64_t>(P.E, slots)) * P.ntn;
    int64_t g = std::min<int64_t>(tiles_ub, cu_count_pipe());
    if (g >= 8) g = g / 8 * 8;
    g = std::max<int64_t>(g, 1);
    MOE_LAUNCH(GATEUP ? "gemm_gateup" : "gemm_down", (k_gemm_pipe<GATEUP, BM>), dim3((unsigned)g), dim3(kPT), shmem, s,
               P);
    return MOE_OK;
}

// Row tile by the mean rows per touched expert: 64-row tiles hold a whole
// expert of a 1K-token prefill (about 32 rows, up to ~60) with half the
// padding of 128-row tiles.
template <bool GATEUP>
moe_status launch_pipe(const PipeParams& P, int64_t slots, hipStream_t s) {
    const int64_t avg = slots / std::max<int64_t>(1, std::min<int64_t>(P.E, slots));
    return avg <= kPipeBM64MaxMeanRows ? launch_pipe_bm<GATEUP, 64>(P, slots, s) : launch_pipe_bm<GATEUP, 128>(P, slots, s);
}

}  // namespace

// Shapes the kernels tile exactly; the activation DMAs address rows by a
// 32-bit byte offset from the activation base (x for gate/up, h for down).
bool prefill_pipe_supported(int64_t T, int k, int H, int I) {
    return H % kBN == 0 && I % (kBN / 2) == 0 && H % (kBK * kSBlk) == 0 && I % (kBK * kSBlk) == 0 &&
           T * H * 2 < (int64_t)1 << 32 &&
           T * k * I * 2 < (int64_t)1 << 32;
}

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
    g.gmul = a.xs;
    g.hf = a.hf;
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
    d.gmul = a.hs;
    d.hf = nullptr;
    return launch_pipe<false>(d, (int64_t)a.T * a.k, s);
}

}  // namespace moe
