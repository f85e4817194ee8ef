// gemm_bf16.hip -- tiled bf16 MFMA GEMM for the colwise and rowwise shards.
//
// Computes Y = epilogue(X . W^T) with X [M, K] and W [N, K] both K-contiguous
// (nn.Linear layout), fp32 accumulation on the CDNA4 matrix cores
// (v_mfma_f32_16x16x32_bf16), and a fused epilogue: + bias, GELU-tanh, store
// as bf16 (round to nearest even) or fp32.  The colwise shard of the
// Diffusers "Tensor parallelism" page (section "Colwise and rowwise") is this
// kernel on a row block of W; the rowwise shard is this kernel on a column
// block of W and X with an fp32 store and no bias (the partial sum).
//
// Design for gfx950:
//  * BM x BN output tile per workgroup: 256, 224 or 192 rows by 256 or 192
//    columns for many rows, 128 or 64 rows for a few hundred, whichever fills
//    the CUs best (pick_tile); up to 128 rows the split-K kernel
//    (gemm_narrow.hip) runs instead.  K step 64.
//  * The 192- to 256-row tiles run on 256 threads = 4 waves in a 2 x 2 grid,
//    one wave per SIMD, each owning (BM/2) x (BN/2) outputs as up to 8 x 8 MFMA
//    16x16 fp32 accumulators in the accumulation registers (mainloop4).  Per
//    k32 step a wave reads NXB + NWB fragments for NXB x NWB MFMAs (16 for 64
//    at 256 x 256), a third fewer LDS reads per flop than eight waves of
//    128 x 64.  The 64- and 128-row tiles run on 512 threads = 8 waves in a
//    2 x 4 grid, two per SIMD (mainloop).
//  * On dense random operands the part runs at its power limit (the clock
//    falls from 2.41 GHz on all-zero operands to 1.76 GHz on random ones at
//    the same MFMA-busy fraction), so energy per flop and the MFMA-busy
//    fraction under the cap set the speed.  The four-wave schedule writes out
//    every k32 step: MFMAs with the fragment reads and loads spread evenly
//    between them; bursts of loads left the single wave of a SIMD stalled on
//    issue.  The 16x16x32 form moves 20% fewer register bytes per flop than
//    32x32x16 (operand reads plus accumulator read and write) and measured
//    3-9% faster on every workload shape.
//  * Operands go HBM/L2 -> LDS by direct-to-LDS DMA (global_load_lds_dwordx4),
//    no VGPR staging: 2 stages x (X tile + W tile), at most 128 KiB of the
//    160 KiB LDS, 3 stages for the 224 x 192 and 192 x 192 tiles.  The 64- and
//    128-row tiles, whose MFMA work per k-tile is too short to cover the next
//    k-tile's loads, keep 3 or 4 stages (at most 144 KiB) and 2 or 3 k-tiles in
//    flight.
//  * Fragments are double-buffered in registers at k32 granularity: while
//    the MFMAs of one k32 step run, the fragments of the next step are read
//    from LDS.  The single barrier per k-tile sits before the second k32 step:
//    after it the next k-tile has landed and every wave has finished reading
//    the stage that the loads of the k-tile after next then overwrite, so the
//    loads run a whole k-tile ahead and no fragment read is exposed.
//  * LDS tiles are 64-element (128-byte) rows; the 16-byte chunk c of row r
//    is stored at position c ^ ((r >> 1) & 7).  A fragment read covers
//    16 rows of one chunk column per 16 lanes; under this swizzle each group
//    of lanes that the LDS serves together touches distinct banks.
//  * The W fragment is the MFMA "A" operand and the X fragment the "B"
//    operand, so each lane holds runs of four consecutive output columns of
//    one row.  The epilogue applies bias / GELU / SwiGLU / rounding, passes
//    each 16-row slice of a wave's tile through a private LDS area and stores
//    whole row segments: direct stores from the MFMA layout cover 16 rows x
//    16 B per instruction and wrote 1.64x the algorithmic bytes for an fp32
//    output when measured with the 32x32 layout.  The stores are
//    non-temporal.
//  * Workgroups are dealt round-robin to the 8 XCDs; the tile index is
//    remapped so each XCD gets a contiguous run of a grouped raster order,
//    which keeps its concurrent tiles on few X row-panels and W row-panels
//    (shared in that XCD's L2).
//  * Ragged M and N: loads clamp the row index to the last valid row (the
//    extra rows are computed and discarded), stores are masked.
#include "tp_internal.h"
#include <atomic>
#include <type_traits>

namespace tpl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define TPL_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// The tile shape is two template parameters, the 16-row MFMA blocks per wave NXB and the
// 16-column blocks per wave NWB.  Eight-wave tiles (2 x 4 waves): NXB = 4 or 2 (128 or 64
// rows) by NWB = 4 or 3 (256 or 192 columns).  Four-wave tiles (2 x 2 waves, mainloop4):
// NXB = 8, 7 or 6 (256, 224 or 192 rows) by NWB = 8 or 6 (256 or 192 columns).  pick_tile
// chooses the shape that fills the CUs best for the problem.
constexpr int BK = 64;
constexpr int kThreads = 512;     // 8 waves in a 2 (M) x 4 (N) grid
constexpr int kWavesN = 4;
constexpr int kWaves = kThreads / 64;

// An eight-wave tile; WM and WN (a wave's rows and columns) also serve the shared epilogue.
template <int NXB, int NWB>
struct Tile {
    static constexpr int XB = NXB;       // 16-row X blocks (16-row MFMA tiles) per wave
    static constexpr int WB = NWB;
    static constexpr int WM = 16 * NXB;  // rows of the output owned by one wave
    static constexpr int WN = 16 * NWB;  // columns of the output owned by one wave
    static constexpr int BM = 2 * WM;    // rows of the output tile
    static constexpr int BN = kWavesN * WN;  // columns of the output tile (weight rows)
    static constexpr int kDmaW = (BN * BK * 2) / (kThreads * 16);  // 16-byte DMAs per thread per W tile
    static constexpr int kXElems = BM * BK;
    static constexpr int kDmaX = BM / 64;  // one DMA instruction of the workgroup moves 64 rows
    static constexpr int kStageElems = (BM + BN) * BK;  // X tile + W tile
    // These tiles stream a weight panel for few rows and keep more k-tiles in flight:
    // 64 x 192 4 stages (128 KiB), 64 x 256 3 (120 KiB), 128 x 192 3 (120 KiB), 128 x 256 3
    // (144 KiB); a k loop shorter than the stages double buffers.
    static constexpr int kStages = NXB == 2 ? (NWB == 3 ? 4 : 3) : 3;
    static constexpr int kLdsElems = kStages * kStageElems;
};

struct GemmParams {
    const uint16_t *x;
    const uint16_t *w;
    const uint16_t *bias;
    void *y;
    int64_t ldx, ldw, ldy;
    int M, N, K;
    int tiles_m, tiles_n, group_m;
};

// Workgroups are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8).
// Renumber [0, total) so that each XCD's blocks get a contiguous run.
__device__ __forceinline__ int xcd_contiguous(int bid, int total)
{
    const int xcd = bid & 7;
    const int local = bid >> 3;
    const int per = (total + 7) >> 3;
    const int tall = total - (per - 1) * 8;  // XCDs that receive `per` blocks
    return xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
}

// Linear tile index -> (tile row, tile column), grouped raster: group_m tile
// rows at a time, column-major inside the group.
__device__ __forceinline__ void tile_of(int lin, const GemmParams &p, int &tm, int &tn)
{
    const int in_group = p.group_m * p.tiles_n;
    const int g = lin / in_group;
    const int first_m = g * p.group_m;
    const int gsz = min(p.tiles_m - first_m, p.group_m);
    const int r = lin - g * in_group;
    tm = first_m + r % gsz;
    tn = r / gsz;
}

// GELU, tanh form: g(v) = v/2 (1 + tanh(u)), u = sqrt(2/pi) (v + 0.044715 v^3).
// Uses 1 + tanh(u) = 2 / (1 + exp(-2u)), so g(v) = v / (1 + exp(-2u)), with
// exp(-2u) = 2^(v (a + b v^2)), a = -2 sqrt(2/pi) log2(e), b = 0.044715 a.
// The hardware exp2 and reciprocal (about 1 ulp each) replace the library
// exp and the IEEE divide: 7 instructions per element instead of about 19,
// which took 6% of a 4608 x 9216 x 6144 launch in the epilogue.  Both tails
// are exact limits (2^+inf gives v * 0 = -0, 2^-inf gives v).
__device__ __forceinline__ float gelu_tanh(float v)
{
    const float a = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
    const float b = 0.044715f * a;
    const float e = __builtin_amdgcn_exp2f(v * __builtin_fmaf(b, v * v, a));
    return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// One k32 step's operand fragments: per lane 8 bf16 of one row of each of
// the wave's NXB 16-row X blocks and NWB 16-row W blocks.
template <int NXB, int NWB>
struct Frags {
    bf16x8 x[NXB];
    bf16x8 w[NWB];
};

// Per-thread constants of the tile pipeline.
struct Ctx {
    int lane, wave, wave_m, wave_n;
    int dma_row, dma_chunk;       // DMA: row within a 64-row group, logical chunk
    int xrow_off, wrow_off;       // fragment row offsets inside an LDS tile
    int swz, kh;                  // fragment swizzle and k-quarter
};

template <int NXB, int NWB>
__device__ __forceinline__ Ctx make_ctx()
{
    Ctx c;
    const int tid = threadIdx.x;
    c.lane = tid & 63;
    c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    c.wave_m = c.wave / kWavesN;
    c.wave_n = c.wave % kWavesN;
    // DMA addressing.  Instruction j of wave w fills LDS chunks
    // [(8j + w) * 64, +64) of a 64-column tile: lane l lands at tile row
    // R = 64j + 8w + l/8, stored position l%8, so it must fetch logical chunk
    // (l%8) ^ ((R >> 1) & 7) = (l%8) ^ ((4 (w & 1) + l/16) & 7).
    c.dma_row = c.wave * 8 + (c.lane >> 3);
    c.dma_chunk = (c.lane & 7) ^ ((((c.wave & 1) << 2) + (c.lane >> 4)) & 7);
    // Fragment addressing: lane l reads row (l % 16) of a 16-row block,
    // 16-byte k-chunk (4 s + l / 16) for k32 step s, stored at position
    // chunk ^ ((row >> 1) & 7) = chunk ^ (((l % 16) >> 1) & 7).
    c.xrow_off = (c.wave_m * Tile<NXB, NWB>::WM + (c.lane & 15)) * BK;
    c.wrow_off = (c.wave_n * Tile<NXB, NWB>::WN + (c.lane & 15)) * BK;
    c.swz = (c.lane >> 1) & 7;
    c.kh = c.lane >> 4;
    return c;
}

// Waits until this wave's direct-to-LDS loads have written the LDS.  A
// barrier after it then publishes every wave's loads to the workgroup.  The
// compiler's own waits do not cover this in every loop shape: a k-step-32
// variant of this kernel compiled with no load wait before its barrier and read
// stale tiles.
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Waits until at most N of this wave's vector memory instructions are outstanding (they
// complete in issue order) and its LDS reads have returned: with N = the loads issued
// after a k-tile's, that k-tile has landed while the later ones stay in flight.
template <int N>
__device__ __forceinline__ void wait_dma_keep()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

// A workgroup barrier without the release fence of __syncthreads(), which would wait for
// every outstanding load, the ones meant to stay in flight included.  The caller waits
// for what must be complete first; the empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void barrier_only()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One 16-byte direct-to-LDS load per lane (global_load_lds_dwordx4): lane l
// writes dst + 16 l bytes.  Kept out of templates: the host pass of a
// template rejects the LDS address-space argument.
__device__ __forceinline__ void dma16(const char *src, uint16_t *dst)
{
    __builtin_amdgcn_global_load_lds(src, TPL_LDS(dst), 16, 0, 0);
}

// acc += X[m0 .. m0+BM-1, k] . Wt^T over k-tiles [kt0, kt1), where the BN
// rows of the W tile Wt are W[n0 .. n0+BN-1] (eight waves: the 64- and 128-row tiles).
// Rows past the end are clamped (computed and discarded).  Starts with a barrier, so the
// LDS may still be in use by the caller's previous tile when it is called.
template <int NXB, int NWB>
__device__ __forceinline__ void mainloop(const GemmParams &p, uint16_t *lds, const Ctx &c, int m0, int n0,
                                         int kt0, int kt1, f32x4 (&acc)[NXB][NWB])
{
    // Per-lane byte offsets (32-bit: operands are below 2 GiB) from
    // wave-uniform bases, so the DMA uses the scalar-base addressing form.
    const char *xbase = reinterpret_cast<const char *>(p.x) + (int64_t)kt0 * BK * 2;
    const char *wbase = reinterpret_cast<const char *>(p.w) + (int64_t)kt0 * BK * 2;
    typedef Tile<NXB, NWB> L;
    constexpr int WB = NWB, kDmaW = L::kDmaW;
    static_assert(kDmaW * kWaves * 512 == L::BN * BK, "the W DMAs cover the W tile exactly");
    static_assert(L::kDmaX * kWaves * 512 >= L::kXElems, "the X DMAs cover the X tile");
    uint32_t xoff[L::kDmaX], woff[kDmaW];
#pragma unroll
    for (int j = 0; j < L::kDmaX; ++j) {
        const int gm = min(m0 + j * (8 * kWaves) + c.dma_row, p.M - 1);
        xoff[j] = (uint32_t)(((int64_t)gm * p.ldx + c.dma_chunk * 8) * 2);
    }
#pragma unroll
    for (int j = 0; j < kDmaW; ++j) {
        // DMA instruction j fills tile rows 64 j + dma_row
        const int gn = min(n0 + j * (8 * kWaves) + c.dma_row, p.N - 1);
        woff[j] = (uint32_t)(((int64_t)gn * p.ldw + c.dma_chunk * 8) * 2);
    }
    auto issue = [&](int stage, int k0) {
        uint16_t *xs = lds + stage * L::kStageElems;
        uint16_t *ws = xs + L::kXElems;
        const char *xb = xbase + k0 * 2;
        const char *wb = wbase + k0 * 2;
#pragma unroll
        for (int j = 0; j < L::kDmaX; ++j)
            dma16(xb + xoff[j], xs + (j * kWaves + c.wave) * 512);
#pragma unroll
        for (int j = 0; j < kDmaW; ++j)
            dma16(wb + woff[j], ws + (j * kWaves + c.wave) * 512);
    };
    // The MFMAs run X block by X block, and the fragments are read in the order they use them.
    auto read_frags = [&](int stage, int s, Frags<NXB, NWB> &f) {
        const uint16_t *xs = lds + stage * L::kStageElems;
        const uint16_t *ws = xs + L::kXElems;
        const int cpos = ((s * 4 + c.kh) ^ c.swz) * 8;
#pragma unroll
        for (int i = 0; i < L::XB; ++i)
            f.x[i] = *reinterpret_cast<const bf16x8 *>(xs + c.xrow_off + i * 16 * BK + cpos);
#pragma unroll
        for (int j = 0; j < WB; ++j)
            f.w[j] = *reinterpret_cast<const bf16x8 *>(ws + c.wrow_off + j * 16 * BK + cpos);
    };
    auto mma = [&](const Frags<NXB, NWB> &f) {
#pragma unroll
        for (int i = 0; i < L::XB; ++i)
#pragma unroll
            for (int j = 0; j < WB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.w[j], f.x[i], acc[i][j], 0, 0, 0);
    };
    // Pipeline: stage t % 2 holds k-tile t; steps s = 0, 1 are its k32 slices.
    // TPL_STEP(read next, mma current) fixes the order of one step for the
    // scheduler: (MFMA, read) for each of the next step's fragments, then the
    // remaining MFMAs.
#define TPL_STEP(RD, MM) do { RD; MM;                                        \
        _Pragma("unroll") for (int g_ = 0; g_ < L::XB + WB; ++g_) {           \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                \
        }                                                                     \
        __builtin_amdgcn_sched_group_barrier(0x008, L::XB * WB - (L::XB + WB), 0); \
        __builtin_amdgcn_sched_barrier(0); } while (0)
    const int T = kt1 - kt0;
    Frags<NXB, NWB> f0, f1;
    if constexpr (L::kStages > 2) {
        if (T >= L::kStages) {
            // S stages, k-tile t in stage t % S.  All S are issued first; in iteration t,
            // once k-tile t + 1 has landed and every wave has read k-tile t, k-tile t + S
            // goes into k-tile t's stage, so S - 1 k-tiles stay in flight behind the one
            // being computed.
            constexpr int S = L::kStages;
            constexpr int kPer = L::kDmaX + kDmaW;  // DMA instructions per k-tile and wave
            static_assert((S - 1) * kPer <= 63, "the wait count fits vmcnt");
            __syncthreads();  // the LDS is free: the previous tile's reads are done
#pragma unroll
            for (int i = 0; i < S; ++i)
                issue(i, i * BK);
            wait_dma_keep<(S - 1) * kPer>();
            barrier_only();
            read_frags(0, 0, f0);
            int st = 0;
            for (int t = 0; t < T - 1; ++t) {
                const int nx = st == S - 1 ? 0 : st + 1;
                TPL_STEP(read_frags(st, 1, f1), mma(f0));
                if (t + S - 1 < T)
                    wait_dma_keep<(S - 2) * kPer>();  // k-tile t + 1 has landed
                else
                    wait_dma_keep<0>();
                barrier_only();
                if (t + S < T)
                    issue(st, (t + S) * BK);
                TPL_STEP(read_frags(nx, 0, f0), mma(f1));
                st = nx;
            }
            TPL_STEP(read_frags(st, 1, f1), mma(f0));
            mma(f1);
            __builtin_amdgcn_sched_barrier(0);
            return;
        }
    }
    __syncthreads();  // the LDS is free: the previous tile's reads are done
    issue(0, 0);
    wait_dma();
    __syncthreads();
    read_frags(0, 0, f0);
    if (T > 1)
        issue(1, BK);
    int t = 0;
    for (; t < T - 1; ++t) {
        const int st = t & 1;
        TPL_STEP(read_frags(st, 1, f1), mma(f0));
        wait_dma();
        __syncthreads();
        if (t + 2 < T)
            issue(st, (t + 2) * BK);
        TPL_STEP(read_frags(st ^ 1, 0, f0), mma(f1));
    }
    TPL_STEP(read_frags((T - 1) & 1, 1, f1), mma(f0));
    mma(f1);
    // Keep the epilogue's arithmetic out of the last MFMAs (interleaved with them, tiles at
    // the register limit spilled).
    __builtin_amdgcn_sched_barrier(0);
#undef TPL_STEP
}

// SiLU (Swish): v * sigmoid(v) = v / (1 + exp(-v)) = v / (1 + 2^(-v log2(e))),
// with the hardware exp2 and reciprocal as in gelu_tanh; both tails are exact
// limits (2^+inf gives -0, 2^-inf gives v).
__device__ __forceinline__ float silu(float v)
{
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * -1.4426950408889634f));
}

// Epilogue activations.
constexpr int kActNone = 0;
constexpr int kActGelu = 1;
constexpr int kActSwiglu = 2;  // W tile = interleaved [gate; up] 64-row blocks, see mainloop4

// Epilogue through LDS.  Lane l holds Y[m][n..n+3] for m = row base +
// 16 i + l%16 and n = column base + 16 j + 4 (l / 16).  For each of the
// wave's 16-row slices the wave writes its output values (after bias /
// activation / rounding) into a private LDS area with padded rows, then
// reads them back row-major and stores whole row segments.  A wave owns 16 NWB
// output columns, or 8 NWB with SwiGLU: there its blocks j < NWB / 2 hold the gate
// and j >= NWB / 2 the up projection of the same columns, and the output is
// silu(gate + b_gate) * (up + b_up), the bias being [b_gate; b_up] (2 N).
template <int NXB, int NWB, bool OUT_BF16, bool HAS_BIAS, int ACT>
__device__ __forceinline__ void epilogue(const GemmParams &p, uint16_t *lds, const Ctx &c, int m0, int n0,
                                         const f32x4 (&acc)[NXB][NWB])
{
    __syncthreads();  // every wave is done reading the operand stages
    typedef typename std::conditional<OUT_BF16, __bf16, float>::type OutT;
    constexpr bool kGated = ACT == kActSwiglu;
    static_assert(!kGated || NWB == 4 || NWB == 8, "the gated epilogue pairs NWB / 2 gate and up blocks");
    constexpr int WNO = kGated ? Tile<NXB, NWB>::WN / 2 : Tile<NXB, NWB>::WN;  // output columns per wave
    constexpr int JO = WNO / 16;               // 16-column output blocks per wave
    constexpr int kOutEs = sizeof(OutT);
    constexpr int kRowElems = WNO + 16 / kOutEs;  // one 16-byte pad per row
    OutT *stage = reinterpret_cast<OutT *>(lds) + c.wave * 16 * kRowElems;
    // The lane's terms are derived here from an opaque copy of the thread index, so the
    // compiler cannot keep them live through the main loop (at 256 registers the 256-row
    // tiles would spill them).
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int mrow = lane & 15;
    const int ncol = 4 * (lane >> 4);
    auto bias4 = [&](int e) {
        const bf16x4 bb = *reinterpret_cast<const bf16x4 *>(p.bias + e);
        return f32x4{(float)bb[0], (float)bb[1], (float)bb[2], (float)bb[3]};
    };
    constexpr int kVec = 16 / kOutEs;              // elements per 16-byte vector
    constexpr int kVecPerRow = WNO / kVec;
    // When a pass of 64 lanes covers whole rows, each lane keeps its row and column for
    // every pass; otherwise (48 output columns per wave) a lane's position moves per pass.
    constexpr bool kWholeRows = 64 % kVecPerRow == 0;
    constexpr int kRowsPerPass = kWholeRows ? 64 / kVecPerRow : 1;
    constexpr int kPasses = (16 * kVecPerRow + 63) / 64;
    const int rd_row = lane / kVecPerRow;
    const int rd_vec = lane % kVecPerRow;
    const int64_t lane_off = (int64_t)rd_row * p.ldy + rd_vec * kVec;
#pragma unroll
    for (int i = 0; i < NXB; ++i) {
#pragma unroll
        for (int j = 0; j < JO; ++j) {
            const int n = n0 + c.wave_n * WNO + j * 16 + ncol;  // N % 16 == 0: n < N covers n + 3
            f32x4 v = acc[i][j];
            if (HAS_BIAS && n < p.N)
                v = v + bias4(n);
            if (ACT == kActGelu) {
                v[0] = gelu_tanh(v[0]);
                v[1] = gelu_tanh(v[1]);
                v[2] = gelu_tanh(v[2]);
                v[3] = gelu_tanh(v[3]);
            }
            if (kGated) {
                f32x4 u = acc[i][j + NWB / 2];
                if (HAS_BIAS && n < p.N)
                    u = u + bias4(p.N + n);
                v[0] = silu(v[0]) * u[0];
                v[1] = silu(v[1]) * u[1];
                v[2] = silu(v[2]) * u[2];
                v[3] = silu(v[3]) * u[3];
            }
            OutT *dst = stage + mrow * kRowElems + j * 16 + ncol;
            if (OUT_BF16)
                *reinterpret_cast<bf16x4 *>(dst) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
            else
                *reinterpret_cast<f32x4 *>(dst) = v;
        }
        // Row r + rd_row of the slice: the row's base and bound are wave-uniform, the lane's
        // offset is fixed, so no per-row lane value stays live across the unrolled passes.
        const int mbase = m0 + c.wave_m * Tile<NXB, NWB>::WM + i * 16;
        OutT *ybase = reinterpret_cast<OutT *>(p.y) + n0 + c.wave_n * WNO;
        if constexpr (kWholeRows) {
            const bool col_ok = n0 + c.wave_n * WNO + rd_vec * kVec < p.N;
#pragma unroll
            for (int r = 0; r < 16; r += kRowsPerPass) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(stage + (r + rd_row) * kRowElems + rd_vec * kVec);
                // Non-temporal stores: about 1% faster than ordinary ones over a DiT block's
                // GEMMs, with the same fetched and written bytes.
                if (rd_row < p.M - (mbase + r) && col_ok)
                    __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(ybase + (int64_t)(mbase + r) * p.ldy + lane_off));
            }
        } else {
#pragma unroll
            for (int q = 0; q < kPasses; ++q) {
                const int e = lane + 64 * q;        // vector e of the slice: row e / kVecPerRow
                const int row = e / kVecPerRow;
                const int vec = e - row * kVecPerRow;
                if (row < 16) {
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(stage + row * kRowElems + vec * kVec);
                    if (row < p.M - mbase && n0 + c.wave_n * WNO + vec * kVec < p.N)
                        __builtin_nontemporal_store(
                            v, reinterpret_cast<f32x4 *>(ybase + (int64_t)(mbase + row) * p.ldy + vec * kVec));
                }
            }
        }
    }
}

template <int NXB, int NWB>
__device__ __forceinline__ void zero(f32x4 (&acc)[NXB][NWB])
{
#pragma unroll
    for (int i = 0; i < NXB; ++i)
#pragma unroll
        for (int j = 0; j < NWB; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// ---- Four-wave tiles: the 192-, 224- and 256-row tiles of the plain, bias and GELU epilogues.
//
// 256 threads = 4 waves in a 2 x 2 grid, one wave per SIMD, each owning (16 NXB) x (16 NWB)
// outputs (NWB = 8 or 6: 256- or 192-column tiles) as NXB x NWB MFMA accumulators, up to 256
// registers, held in the accumulation registers: each MFMA is written out with its
// accumulator tied to those registers ("+a"), so the compiler never moves an accumulator
// between register files inside the loop (it did, hundreds of moves per k-tile, when it
// chose the registers itself).  Per wave and k32 step the fragment reads fall to
// NXB + NWB for NXB x NWB MFMAs (12 for 32 MFMAs with eight waves of 128 x 64, 16 for 64
// here), so the LDS serves a third fewer reads per flop.
//
// With one wave per SIMD nothing hides an instruction the wave spends not issuing MFMAs,
// so the order of each k32 step is written out (the MFMAs clobber memory, which pins every
// load between them): MFMA q, then, if q is a multiple of RS, the next fragment read, and if
// q is 1 more than a multiple of DS, the next load of the k-tile after next.  The reads and
// loads are spread evenly over the step.  Issued in bursts after the first MFMAs instead,
// the same kernel measured 3-9% slower than the eight-wave tiles; spread, and with the loads
// in their scalar-base form (dma16_sbase), it measured 1-13% faster on every shape of the
// DiT block (bit-identical outputs); packing the loads into half of each step instead cost
// 7%.  LDS layout, swizzle and epilogue are those of the eight-wave kernel, and so is the
// pipeline of two LDS stages with one barrier per k-tile before its second k32 step.  The
// 224 x 192 and 192 x 192 tiles fit three stages in the 160 KiB of LDS: a k-tile's loads
// then spread over a whole k-tile and have twice as long to land (4608 x 4608 x 6144: 5%
// faster than with two stages).
constexpr int kThreads4 = 256;
constexpr int kWaves4 = kThreads4 / 64;

// One 16-byte direct-to-LDS load per lane in its scalar-base form: a wave-uniform base
// address plus the lane's 32-bit byte offset, with the LDS address of the wave's 1 KiB
// destination in M0 (lane l writes 16 l bytes after it).  The builtin forms a 64-bit lane
// address with two VALU instructions per load, which the single wave of a SIMD issues
// between its MFMAs.  The load writes no register; the caller waits for it with an explicit
// vmcnt wait before the barrier that publishes its data.  No other code of the kernel uses
// M0, so clobbering it here is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_sbase(const char *base, uint32_t off, uint16_t *dst)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t *)dst;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(off), "s"(base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// acc += X[m0 .. m0 + BM - 1, :] . W[n0 .. n0 + BN - 1, :]^T over all of K, four waves.
// Rows past the end are clamped (computed and discarded).
template <int NXB, int NWB, int S, bool GATED>
__device__ __forceinline__ void mainloop4(const GemmParams &p, uint16_t *lds, const Ctx &c, int m0, int n0,
                                          f32x4 (&acc)[NXB][NWB])
{
    static_assert(!GATED || NWB == 8, "the gated tile pairs four gate and four up blocks per wave");
    constexpr int WM = 16 * NXB, WN = 16 * NWB, BM = 2 * WM, BN = 2 * WN;
    constexpr int kDmaX = BM / 32, kDmaW = BN / 32, kDma = kDmaX + kDmaW;  // per lane and k-tile
    constexpr int kXElems = BM * BK, kStageElems = (BM + BN) * BK;
    constexpr int kMfma = NXB * NWB, kReads = NXB + NWB;
    constexpr int RS = kMfma / kReads, DS = kMfma / kDma;
    static_assert(RS >= 1 && DS >= 1 && (kReads - 1) * RS < kMfma && 1 % DS + (kDma - 1) * DS < kMfma,
                  "the reads and loads of a k32 step fit between its MFMAs");
    // DMA: instruction j of wave w fills LDS chunks [(4 j + w) * 64, +64) of a 64-column tile:
    // lane l lands at tile row 32 j + 8 w + l / 8, stored position l % 8, so it fetches logical
    // chunk (l % 8) ^ ((row >> 1) & 7) = (l % 8) ^ ((4 (w & 1) + l / 16) & 7).
    const int dma_row = c.wave * 8 + (c.lane >> 3);
    const int dma_chunk = (c.lane & 7) ^ ((((c.wave & 1) << 2) + (c.lane >> 4)) & 7);
    // Fragments: lane l reads row l % 16 of a 16-row block, chunk (4 s + l / 16) ^ swz.
    const int xrow_off = (c.wave_m * WM + (c.lane & 15)) * BK;
    const int wrow_off = (c.wave_n * WN + (c.lane & 15)) * BK;
    const int swz = (c.lane >> 1) & 7;
    const int kh = c.lane >> 4;
    uint32_t xoff[kDmaX], woff[kDmaW];
#pragma unroll
    for (int j = 0; j < kDmaX; ++j) {
        const int gm = min(m0 + 32 * j + dma_row, p.M - 1);
        xoff[j] = (uint32_t)(((int64_t)gm * p.ldx + dma_chunk * 8) * 2);
    }
#pragma unroll
    for (int j = 0; j < kDmaW; ++j) {
        // GATED: tile row 128 q + 64 h + i is W[h N + n0 + 64 q + i], so wave column q's blocks
        // 0-3 hold the gate rows and blocks 4-7 the up rows of outputs n0 + 64 q + [0, 64).
        const int gn = GATED ? ((j >> 1) & 1) * p.N + min(n0 + 64 * (j >> 2) + 32 * (j & 1) + dma_row, p.N - 1)
                             : min(n0 + 32 * j + dma_row, p.N - 1);
        woff[j] = (uint32_t)(((int64_t)gn * p.ldw + dma_chunk * 8) * 2);
    }
    const char *xbase = reinterpret_cast<const char *>(p.x);
    const char *wbase = reinterpret_cast<const char *>(p.w);
    auto dma = [&](int d, int stage, int k0) {  // load d of k-tile k0 / 64 into `stage`
        uint16_t *xs = lds + stage * kStageElems;
        if (d < kDmaX)
            dma16_sbase(xbase + k0 * 2, xoff[d], xs + (d * kWaves4 + c.wave) * 512);
        else
            dma16_sbase(wbase + k0 * 2, woff[d - kDmaX], xs + kXElems + ((d - kDmaX) * kWaves4 + c.wave) * 512);
    };
    // read r of a k32 step: the X fragments first, then the W fragments (the next step's
    // first MFMAs use W block 0 with every X block)
    auto read = [&](int r, int stage, int s, Frags<NXB, NWB> &f) {
        const uint16_t *xs = lds + stage * kStageElems;
        const int cpos = ((s * 4 + kh) ^ swz) * 8;
        if (r < NXB)
            f.x[r] = *reinterpret_cast<const bf16x8 *>(xs + xrow_off + r * 16 * BK + cpos);
        else
            f.w[r - NXB] = *reinterpret_cast<const bf16x8 *>(xs + kXElems + wrow_off + (r - NXB) * 16 * BK + cpos);
    };
    // One k32 step on `cur`; READS: the next step's fragments (stage rstage, k32 step rs) into
    // `nxt`; loads [D0, D0 + DN) of the k-tile at dk0 into stage dstage, spread evenly.
    auto step_part = [&](const Frags<NXB, NWB> &cur, Frags<NXB, NWB> &nxt, auto READS, auto D0, auto DN, int rstage,
                         int rs, int dstage, int dk0) {
        constexpr int d0 = decltype(D0)::value, dn = decltype(DN)::value;
        constexpr int ds = dn > 0 ? kMfma / dn : 1;
#pragma unroll
        for (int q = 0; q < kMfma; ++q) {
            const int j = q / NXB, i = q % NXB;  // W block by W block
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                         : "+a"(acc[i][j])
                         : "v"(cur.w[j]), "v"(cur.x[i])
                         : "memory");
            if constexpr (dn > 0) {
                if (q % ds == 1 % ds && q / ds < dn)
                    dma(d0 + q / ds, dstage, dk0);
            }
            if constexpr (decltype(READS)::value) {
                if (q % RS == 0 && q / RS < kReads)
                    read(q / RS, rstage, rs, nxt);
            }
        }
    };
    auto step = [&](const Frags<NXB, NWB> &cur, Frags<NXB, NWB> &nxt, auto READS, auto DMA, int rstage, int rs,
                    int dstage, int dk0) {
        step_part(cur, nxt, READS, std::integral_constant<int, 0>{},
                  std::integral_constant<int, decltype(DMA)::value ? kDma : 0>{}, rstage, rs, dstage, dk0);
    };
    using Yes = std::true_type;
    using No = std::false_type;
    const int T = p.K / BK;
    Frags<NXB, NWB> f0, f1;
    // Every iteration t computes k-tile t: step 0 on f0 while the step-1 fragments are read,
    // the barrier (k-tile t + 1 landed, k-tile t read by every wave), step 1 on f1 while the
    // next k-tile's step-0 fragments are read.  Past the last k-tile the loads repeat it into
    // a stage that is never read again, and the last iteration reads fragments it does not
    // use, so all iterations are the same one loop body: the compiler then has no reason to
    // move an accumulator between registers between the MFMAs, where such a move could read a
    // result before the MFMA has written it (the MFMAs are opaque to its hazard checks).
    auto kt = [&](int u) { return min(u, T - 1) * BK; };
    if constexpr (S == 3) {
        // Three stages: k-tile u goes into stage u % 3, its first kH loads in step 1 of
        // iteration u - 3, the rest in step 0 of iteration u - 2, so the loads of a k-tile are
        // spread over a whole k-tile and land by the barrier of iteration u - 1; at that
        // barrier only k-tile t + 2's loads may still be outstanding.
        constexpr int kH = kDma / 2;
        using I0 = std::integral_constant<int, 0>;
        using IH = std::integral_constant<int, kH>;
        using IR = std::integral_constant<int, kDma - kH>;
#pragma unroll
        for (int d = 0; d < kDma; ++d)
            dma(d, 0, 0);
#pragma unroll
        for (int d = 0; d < kDma; ++d)
            dma(d, 1, kt(1));
#pragma unroll
        for (int d = 0; d < kH; ++d)
            dma(d, 2, kt(2));
        wait_dma_keep<kDma + kH>();
        barrier_only();
#pragma unroll
        for (int r = 0; r < kReads; ++r)
            read(r, 0, 0, f0);
        int s0 = 0, s1 = 1, s2 = 2;  // stages of k-tiles t, t + 1, t + 2
        int t = 0;
        do {
            step_part(f0, f1, Yes{}, IH{}, IR{}, s0, 1, s2, kt(t + 2));
            wait_dma_keep<kDma>();
            barrier_only();
            step_part(f1, f0, Yes{}, I0{}, IH{}, s1, 0, s0, kt(t + 3));
            const int sn = s0;
            s0 = s1;
            s1 = s2;
            s2 = sn;
        } while (++t < T);
    } else {
        // Two stages: stage t % 2 holds k-tile t; step 1 loads k-tile t + 2 into it.
#pragma unroll
        for (int d = 0; d < kDma; ++d)
            dma(d, 0, 0);
#pragma unroll
        for (int d = 0; d < kDma; ++d)
            dma(d, 1, kt(1));
        wait_dma_keep<kDma>();
        barrier_only();
#pragma unroll
        for (int r = 0; r < kReads; ++r)
            read(r, 0, 0, f0);
        int t = 0;
        do {
            const int st = t & 1;
            step(f0, f1, Yes{}, No{}, st, 1, 0, 0);
            wait_dma_keep<0>();
            barrier_only();
            step(f1, f0, Yes{}, Yes{}, st ^ 1, 0, st, kt(t + 2));
        } while (++t < T);
    }
    wait_dma();  // the repeated loads of the last k-tile, before the epilogue reuses the LDS
    // The last MFMAs' results must be written before they are read as ordinary values; the
    // empty statements keep every read of an accumulator after the wait.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < NXB; ++i)
#pragma unroll
        for (int j = 0; j < NWB; ++j)
            asm volatile("" : "+a"(acc[i][j]));
}

// One (32 NXB) x (32 NWB) output tile per workgroup of four waves.
template <int NXB, int NWB, bool OUT_BF16, bool HAS_BIAS, int ACT>
__global__ __launch_bounds__(kThreads4) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm4_bf16_nt_kernel(GemmParams p)
{
    static_assert(NXB >= 6 && NXB <= 8 && (NWB == 6 || NWB == 8), "192-256 rows by 192 or 256 columns");
    constexpr bool kGated = ACT == kActSwiglu;
    constexpr int BM = 32 * NXB, BN = 32 * NWB;
    constexpr int kTileCols = kGated ? BN / 2 : BN;  // SwiGLU: 128 gate and 128 up weight rows
    // three stages where they fit in the 160 KiB of LDS (224 x 192 and 192 x 192 tiles)
    constexpr int S = 3 * (BM + BN) * BK * 2 <= 160 * 1024 ? 3 : 2;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[S * (BM + BN) * BK];
    Ctx c;
    c.lane = threadIdx.x & 63;
    c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    c.wave_m = c.wave >> 1;
    c.wave_n = c.wave & 1;
    int tm, tn;
    tile_of(xcd_contiguous(blockIdx.x, p.tiles_m * p.tiles_n), p, tm, tn);
    f32x4 acc[NXB][NWB];
    zero<NXB, NWB>(acc);
    mainloop4<NXB, NWB, S, kGated>(p, lds, c, tm * BM, tn * kTileCols, acc);
    epilogue<NXB, NWB, OUT_BF16, HAS_BIAS, ACT>(p, lds, c, tm * BM, tn * kTileCols, acc);
}

template <int NXB, int NWB, bool OUT_BF16, bool HAS_BIAS, int ACT>
hipError_t launch_tm4(GemmParams gp, hipStream_t stream)
{
    const int tile_cols = ACT == kActSwiglu ? 16 * NWB : 32 * NWB;
    gp.tiles_n = (gp.N + tile_cols - 1) / tile_cols;
    gp.tiles_m = (gp.M + 32 * NXB - 1) / (32 * NXB);
    gp.group_m = gp.tiles_m < 8 ? gp.tiles_m : 8;
    hipLaunchKernelGGL((gemm4_bf16_nt_kernel<NXB, NWB, OUT_BF16, HAS_BIAS, ACT>), dim3(gp.tiles_m * gp.tiles_n),
                       dim3(kThreads4), 0, stream, gp);
    return hipGetLastError();
}

// One BM x BN output tile per workgroup of eight waves (the 64- and 128-row tiles).
template <int NXB, int NWB, bool OUT_BF16, bool HAS_BIAS, int ACT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_nt_kernel(GemmParams p)
{
    typedef Tile<NXB, NWB> L;
    static_assert(ACT != kActSwiglu, "the gated epilogue runs on the four-wave tiles");
    static_assert(NXB == 2 || NXB == 4, "64- and 128-row tiles");
    __shared__ __attribute__((aligned(1024))) uint16_t lds[L::kLdsElems];
    const Ctx c = make_ctx<NXB, NWB>();
    int tm, tn;
    tile_of(xcd_contiguous(blockIdx.x, p.tiles_m * p.tiles_n), p, tm, tn);
    f32x4 acc[NXB][NWB];
    zero<NXB, NWB>(acc);
    mainloop<NXB, NWB>(p, lds, c, tm * L::BM, tn * L::BN, 0, p.K / BK, acc);
    epilogue<NXB, NWB, OUT_BF16, HAS_BIAS, ACT>(p, lds, c, tm * L::BM, tn * L::BN, acc);
}

template <int NXB, int NWB, bool OUT_BF16, bool HAS_BIAS, int ACT>
hipError_t launch_tm(GemmParams gp, hipStream_t stream)
{
    typedef Tile<NXB, NWB> L;
    gp.tiles_n = (gp.N + L::BN - 1) / L::BN;
    gp.tiles_m = (gp.M + L::BM - 1) / L::BM;
    gp.group_m = gp.tiles_m < 8 ? gp.tiles_m : 8;
    hipLaunchKernelGGL((gemm_bf16_nt_kernel<NXB, NWB, OUT_BF16, HAS_BIAS, ACT>), dim3(gp.tiles_m * gp.tiles_n),
                       dim3(kThreads), 0, stream, gp);
    return hipGetLastError();
}

// nxb x nwb in the eight-wave tile's terms (16-row blocks per wave, 32 nxb rows by 64 nwb
// columns).  The 192- to 256-row tiles of the plain, bias and GELU epilogues run on four
// waves (nwb = 4 or 3 becomes 8 or 6 column blocks per wave); the 64- and 128-row tiles and
// SwiGLU run on eight.
template <bool OUT_BF16, bool HAS_BIAS, int ACT>
hipError_t launch_variant(const GemmParams &gp, int nxb, int nwb, hipStream_t stream)
{
    if constexpr (ACT != kActSwiglu) {
        if (nxb == 2)
            return nwb == 3 ? launch_tm<2, 3, OUT_BF16, HAS_BIAS, ACT>(gp, stream)
                            : launch_tm<2, 4, OUT_BF16, HAS_BIAS, ACT>(gp, stream);
        if (nxb == 4)
            return nwb == 3 ? launch_tm<4, 3, OUT_BF16, HAS_BIAS, ACT>(gp, stream)
                            : launch_tm<4, 4, OUT_BF16, HAS_BIAS, ACT>(gp, stream);
        if (nwb == 3) {
            switch (nxb) {
            case 6: return launch_tm4<6, 6, OUT_BF16, HAS_BIAS, ACT>(gp, stream);
            case 7: return launch_tm4<7, 6, OUT_BF16, HAS_BIAS, ACT>(gp, stream);
            default: return launch_tm4<8, 6, OUT_BF16, HAS_BIAS, ACT>(gp, stream);
            }
        }
        switch (nxb) {
        case 6: return launch_tm4<6, 8, OUT_BF16, HAS_BIAS, ACT>(gp, stream);
        case 7: return launch_tm4<7, 8, OUT_BF16, HAS_BIAS, ACT>(gp, stream);
        default: return launch_tm4<8, 8, OUT_BF16, HAS_BIAS, ACT>(gp, stream);
        }
    } else {
        (void)nwb;  // SwiGLU tiles are 256 weight rows = 128 outputs wide
        switch (nxb) {
        case 6: return launch_tm4<6, 8, OUT_BF16, HAS_BIAS, ACT>(gp, stream);
        case 7: return launch_tm4<7, 8, OUT_BF16, HAS_BIAS, ACT>(gp, stream);
        default: return launch_tm4<8, 8, OUT_BF16, HAS_BIAS, ACT>(gp, stream);
        }
    }
}


// Tile shape: the one with the least cost = (rounds of tiles over the CUs) x (tile area)
// x (cost per flop of the shape).  The per-flop factors were measured in the bench step,
// where the part runs at its power limit and every byte moved from L2 to LDS costs clock:
// against 256 x 256, a 224 x 256 tile costs 2.5% more per flop, 192 x 256 5%, 256 x 192
// 8%, 224 x 192 12% and 192 x 192 27%.  Ties go to the earlier (larger) shape.  Examples
// on 256 CUs: 4608 x 2304 x 6144 takes 252 tiles of 224 x 192 (one round), 4608 x 4608 x
// 6144 504 of them, 4608 x 9216 x 6144 756 of 224 x 256, and rowwise 4608 x 6144 x K 504 of
// 224 x 256 at every K.  With the four-wave tiles the choice matched the fastest four-wave
// tile on each of these shapes within 1% (a sweep of every shape, back to back); with the
// eight-wave tiles a short k loop had favoured 256-row tiles, since a tile's start and store
// outweighed the finer quantization.
// 64- and 128-row tiles (plain epilogues only) serve a few hundred rows, where the larger
// tiles leave CUs idle.  Their factors, 1.30 (128 x 256), 1.45 (128 x 192), 1.97 (64 x 256)
// and 2.2 (64 x 192), are fitted to back-to-back runs of every tile shape on 256 to 1536 rows
// of a 9216 x 6144 weight and three smaller products, where the choice then matched the
// fastest shape on every one: 256 rows take 64 x 192 tiles (61.7 us against 99.6 in
// 192 x 192), 512 rows 128 x 192 (74.0 against 104.9), 768 rows 128 x 256 (88.6 against
// 112.3), 1024 rows 224 x 192.
struct TileChoice {
    int nxb, nwb;
};

TileChoice pick_tile(int M, int N, int K, bool gated, int cus)
{
    struct Cand {
        int nxb, nwb;
        double per_flop;
    };
    static const Cand kCands[10] = {{8, 4, 1.0},  {7, 4, 1.025}, {6, 4, 1.05}, {8, 3, 1.08},
                                    {7, 3, 1.12}, {6, 3, 1.27},  {4, 4, 1.30}, {4, 3, 1.45},
                                    {2, 4, 1.97}, {2, 3, 2.2}};
    TileChoice best{8, 4};
    double best_cost = -1;
    for (const Cand &cd : kCands) {
        if (gated && (cd.nwb != 4 || cd.nxb < 6))
            continue;
        const int bm = 32 * cd.nxb;
        const int cols = cd.nwb == 4 ? (gated ? 128 : 256) : 192;
        const int64_t tiles = (int64_t)((M + bm - 1) / bm) * ((N + cols - 1) / cols);
        if (tiles > ((int64_t)1 << 22))
            continue;  // the launch's thread count must stay below 2^32 (256 x 256 always fits)
        const double cost = (double)((tiles + cus - 1) / cus) * bm * (64 * cd.nwb) * cd.per_flop;
        if (best_cost < 0 || cost < best_cost) {
            best = TileChoice{cd.nxb, cd.nwb};
            best_cost = cost;
        }
    }
    return best;
}

}  // namespace

// Compute units of the current device (cached per device).
int cu_count()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

void gemm_tile_shape(const LinearProblem &pr, int *rows, int *cols)
{
    const TileChoice tc = pick_tile((int)pr.M, (int)pr.N, (int)pr.K, pr.swiglu, cu_count());
    *rows = 32 * tc.nxb;
    *cols = tc.nwb == 4 ? (pr.swiglu ? 128 : 256) : 192;
}

hipError_t launch_gemm(const LinearProblem &pr, hipStream_t stream)
{
    GemmParams gp;
    gp.x = pr.x;
    gp.w = pr.w;
    gp.bias = pr.bias;
    gp.y = pr.y;
    gp.ldx = pr.ldx;
    gp.ldw = pr.ldw;
    gp.ldy = pr.ldy;
    gp.M = (int)pr.M;
    gp.N = (int)pr.N;
    gp.K = (int)pr.K;
    const int act = pr.swiglu ? kActSwiglu : (pr.gelu ? kActGelu : kActNone);
    const TileChoice tc = pick_tile(gp.M, gp.N, gp.K, pr.swiglu, cu_count());
    const int nxb = tc.nxb, nwb = tc.nwb;
    const bool bias = pr.bias != nullptr;
    const int sel = (pr.out_bf16 ? 6 : 0) + (bias ? 3 : 0);
    switch (sel + act) {
    case 0: return launch_variant<false, false, 0>(gp, nxb, nwb, stream);
    case 1: return launch_variant<false, false, 1>(gp, nxb, nwb, stream);
    case 2: return launch_variant<false, false, 2>(gp, nxb, nwb, stream);
    case 3: return launch_variant<false, true, 0>(gp, nxb, nwb, stream);
    case 4: return launch_variant<false, true, 1>(gp, nxb, nwb, stream);
    case 5: return launch_variant<false, true, 2>(gp, nxb, nwb, stream);
    case 6: return launch_variant<true, false, 0>(gp, nxb, nwb, stream);
    case 7: return launch_variant<true, false, 1>(gp, nxb, nwb, stream);
    case 8: return launch_variant<true, false, 2>(gp, nxb, nwb, stream);
    case 9: return launch_variant<true, true, 0>(gp, nxb, nwb, stream);
    case 10: return launch_variant<true, true, 1>(gp, nxb, nwb, stream);
    default: return launch_variant<true, true, 2>(gp, nxb, nwb, stream);
    }
}

}  // namespace tpl
