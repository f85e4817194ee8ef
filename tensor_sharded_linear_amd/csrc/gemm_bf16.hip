// gemm_bf16.hip -- tiled bf16 MFMA GEMM for the colwise and rowwise shards.
//
// Computes Y = epilogue(X . W^T) with X [M, K] and W [N, K] both K-contiguous
// (nn.Linear layout), fp32 accumulation on the CDNA4 matrix cores
// (v_mfma_f32_32x32x16_bf16), and a fused epilogue: + bias, GELU-tanh, store
// as bf16 (round to nearest even) or fp32.  The colwise shard of the
// Diffusers "Tensor parallelism" page (section "Colwise and rowwise") is this
// kernel on a row block of W; the rowwise shard is this kernel on a column
// block of W and X with an fp32 store and no bias (the partial sum).
//
// Design for gfx950:
//  * 256 x 256 output tile per workgroup, K step 64, 256 threads = 4 waves in
//    a 2 x 2 grid; each wave owns a 128 x 128 sub-tile held as 4 x 4 MFMA
//    32x32 fp32 accumulators (v_mfma_f32_32x32x16_bf16), 256 accumulator
//    registers per lane (the AGPR file), one wave per SIMD.  A 128 x 128 wave
//    tile needs 64 flop per byte read from LDS, a third less LDS traffic per
//    flop than 128 x 64.
//  * Operands go HBM/L2 -> LDS by direct-to-LDS DMA (global_load_lds_dwordx4),
//    no VGPR staging, double-buffered: 2 stages x (X tile + W tile) x 32 KiB =
//    128 KiB of the 160 KiB LDS.
//  * Fragments are double-buffered in registers at k16 granularity: while the
//    16 MFMAs of one k16 step run, the 8 fragments of the next step are read
//    from LDS.  The single barrier per k-tile sits before the last k16 step:
//    after it the next k-tile has landed and every wave has finished reading
//    the stage that the DMA for the k-tile after next then overwrites, so the
//    DMA runs a whole k-tile ahead and no fragment read is exposed.
//  * LDS tiles are 64-element (128-byte) rows; the 16-byte chunk c of row r is
//    stored at position c ^ (r & 7), so the eight lanes that read one
//    16-byte column of a fragment hit eight different bank groups.
//  * The W fragment is the MFMA "A" operand and the X fragment the "B"
//    operand, so each lane holds runs of four consecutive output columns of
//    one row.  The epilogue applies bias / GELU / rounding, passes each
//    32-row slice of a wave's tile through a private LDS area and stores
//    whole row segments (4 rows x 256 B fp32, 8 rows x 128 B bf16 per
//    instruction): direct stores from the MFMA layout cover 32 rows x 32 B
//    and measured 1.64x the algorithmic write bytes for an fp32 output.
//  * Workgroups are dealt round-robin to the 8 XCDs; the tile index is
//    remapped so each XCD gets a contiguous run of a grouped raster order,
//    which keeps its concurrent tiles on few X row-panels and W row-panels
//    (shared in that XCD's L2).
//  * Ragged M and N: loads clamp the row index to the last valid row (the
//    extra rows are computed and discarded), stores are masked.
#include "tp_internal.h"
#include <type_traits>

namespace tpl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define TPL_LDS(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kThreads = 512;     // 8 waves in a 2 (M) x 4 (N) grid
constexpr int kWavesN = 4;
constexpr int kWaves = kThreads / 64;
constexpr int WM = 128;           // rows of the output owned by one wave
constexpr int WN = 64;            // columns of the output owned by one wave
constexpr int TM = WM / 32;       // 32-row MFMA tiles per wave
constexpr int TN = WN / 32;       // 32-column MFMA tiles per wave
constexpr int kDmaPerOperand = (BM * BK * 2) / (kThreads * 16);  // 16-byte DMAs per thread per tile
constexpr int kTileElems = BM * BK;          // one operand tile (BM == BN)
constexpr int kStageElems = 2 * kTileElems;  // X tile + W tile
constexpr int kLdsElems = 2 * kStageElems;   // double buffered: 128 KiB

struct GemmParams {
    const uint16_t *x;
    const uint16_t *w;
    const uint16_t *bias;
    void *y;
    int64_t ldx, ldw, ldy;
    int M, N, K;
    int tiles_m, tiles_n, group_m;
};

// Block index -> (tile row, tile column).  See the file header.
__device__ __forceinline__ void tile_coords(int bid, const GemmParams &p, int &tm, int &tn)
{
    const int total = p.tiles_m * p.tiles_n;
    const int xcd = bid & 7;
    const int local = bid >> 3;
    const int per = (total + 7) >> 3;
    const int tall = total - (per - 1) * 8;  // XCDs that receive `per` blocks
    const int lin = xcd < tall ? xcd * per + local
                               : tall * per + (xcd - tall) * (per - 1) + local;
    const int in_group = p.group_m * p.tiles_n;
    const int g = lin / in_group;
    const int first_m = g * p.group_m;
    const int gsz = min(p.tiles_m - first_m, p.group_m);
    const int r = lin - g * in_group;
    tm = first_m + r % gsz;
    tn = r / gsz;
}

// GELU, tanh form: g(v) = v/2 (1 + tanh(u)), u = sqrt(2/pi) (v + 0.044715 v^3).
// Uses 1 + tanh(u) = 2 / (1 + exp(-2u)), so g(v) = v / (1 + exp(-2u)); both
// tails are exact limits (exp -> inf gives -0, exp -> 0 gives v).
__device__ __forceinline__ float gelu_tanh(float v)
{
    const float kSqrt2OverPi = 0.7978845608028654f;
    const float u = kSqrt2OverPi * (v + 0.044715f * v * v * v);
    return v / (1.0f + __expf(-2.0f * u));
}

// One k16 step's operand fragments: per lane 8 bf16 of one row of each of
// the wave's four 32-row X blocks and four 32-row W blocks.
struct Frags {
    bf16x8 x[TM];
    bf16x8 w[TN];
};

template <bool OUT_BF16, bool HAS_BIAS, bool GELU>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_nt_kernel(GemmParams p)
{
    __shared__ __attribute__((aligned(1024))) uint16_t lds[kLdsElems];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_coords(blockIdx.x, p, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    // DMA addressing.  Instruction j of wave w fills LDS chunks
    // [(4j + w) * 64, +64) of a 256x64 tile: lane l lands at tile row
    // 32j + 8w + l/8, stored position l%8, i.e. logical chunk (l%8) ^ (l/8).
    const int dma_row = wave * 8 + (lane >> 3);
    const int dma_chunk = (lane & 7) ^ ((((wave & 1) << 2) + (lane >> 4)) & 7);
    const uint16_t *xsrc[kDmaPerOperand];
    const uint16_t *wsrc[kDmaPerOperand];
#pragma unroll
    for (int j = 0; j < kDmaPerOperand; ++j) {
        const int r = j * (8 * kWaves) + dma_row;
        const int gm = min(m0 + r, p.M - 1);
        const int gn = min(n0 + r, p.N - 1);
        xsrc[j] = p.x + (int64_t)gm * p.ldx + dma_chunk * 8;
        wsrc[j] = p.w + (int64_t)gn * p.ldw + dma_chunk * 8;
    }

    // Fragment addressing: lane l reads row (l % 32) of a 32-row block,
    // 16-byte k-chunk (2 s + l / 32) for k16 step s; the row's low 3 bits
    // equal l % 8.
    const int wave_m = wave / kWavesN;
    const int wave_n = wave % kWavesN;
    const int xrow_off = (wave_m * WM + (lane & 31)) * BK;
    const int wrow_off = (wave_n * WN + (lane & 31)) * BK;
    const int swz = (lane >> 1) & 7;
    const int kh = lane >> 5;
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.f;
    auto issue = [&](int stage, int k0) {
        uint16_t *xs = lds + stage * kStageElems;
        uint16_t *ws = xs + kTileElems;
#pragma unroll
        for (int j = 0; j < kDmaPerOperand; ++j)
            __builtin_amdgcn_global_load_lds(xsrc[j] + k0, TPL_LDS(xs + (j * kWaves + wave) * 512), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < kDmaPerOperand; ++j)
            __builtin_amdgcn_global_load_lds(wsrc[j] + k0, TPL_LDS(ws + (j * kWaves + wave) * 512), 16, 0, 0);
    };
    auto read_frags = [&](int stage, int s, Frags &f) {
        const uint16_t *xs = lds + stage * kStageElems;
        const uint16_t *ws = xs + kTileElems;
        const int cpos = ((s * 2 + kh) ^ swz) * 8;
#pragma unroll
        for (int i = 0; i < TM; ++i)
            f.x[i] = *reinterpret_cast<const bf16x8 *>(xs + xrow_off + i * 32 * BK + cpos);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            f.w[j] = *reinterpret_cast<const bf16x8 *>(ws + wrow_off + j * 32 * BK + cpos);
    };
    auto mma = [&](const Frags &f) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[j], f.x[i], acc[i][j], 0, 0, 0);
    };
    // Pipeline: stage t % 2 holds k-tile t; steps s = 0..3 are its k16 slices.
    // Each step issues the next step's 6 fragment reads interleaved with its
    // first MFMAs (2 reads, 1 MFMA, three times, then 5 MFMAs), so the reads
    // land while the step's remaining MFMAs run.
#define TPL_STEP(RD, MM) do { RD; MM;                                    \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                \
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                \
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                \
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                \
        __builtin_amdgcn_sched_group_barrier(0x008, 5, 0);                \
        __builtin_amdgcn_sched_barrier(0); } while (0)
    const int T = p.K / BK;
    Frags f0, f1;
    issue(0, 0);
    __syncthreads();
    read_frags(0, 0, f0);
    if (T > 1)
        issue(1, BK);
    for (int t = 0; t < T - 1; ++t) {
        const int st = t & 1;
        TPL_STEP(read_frags(st, 1, f1), mma(f0));
        TPL_STEP(read_frags(st, 2, f0), mma(f1));
        TPL_STEP(read_frags(st, 3, f1), mma(f0));
        __syncthreads();
        if (t + 2 < T)
            issue(st, (t + 2) * BK);
        TPL_STEP(read_frags(st ^ 1, 0, f0), mma(f1));
    }
    TPL_STEP(read_frags((T - 1) & 1, 1, f1), mma(f0));
    TPL_STEP(read_frags((T - 1) & 1, 2, f0), mma(f1));
    TPL_STEP(read_frags((T - 1) & 1, 3, f1), mma(f0));
    mma(f1);
#undef TPL_STEP

    // Epilogue through LDS.  Lane l holds Y[m][n..n+3] for m = row base +
    // 32 i + l%32 and n = column base + 32 j + 8 q + 4 (l / 32).  For each of
    // the wave's four 32-row slices the wave writes its 32 x 64 values (after
    // bias / GELU / rounding) into a private LDS area with padded rows, then
    // reads them back row-major and stores whole row segments: 4 rows x 256 B
    // (fp32) or 8 rows x 128 B (bf16) per store instruction.
    __syncthreads();  // every wave is done reading the operand stages
    typedef typename std::conditional<OUT_BF16, __bf16, float>::type OutT;
    constexpr int kOutEs = sizeof(OutT);
    constexpr int kRowElems = WN + 16 / kOutEs;                 // 64 + one 16-byte pad
    OutT *stage = reinterpret_cast<OutT *>(lds) + wave * 32 * kRowElems;
    const int mrow = lane & 31;
    const int ncol = 4 * (lane >> 5);
    f32x4 bj[TN][4];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bj[j][q] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int n = n0 + wave_n * WN + j * 32 + q * 8 + ncol;
            if (HAS_BIAS && n < p.N) {
                const bf16x4 bb = *reinterpret_cast<const bf16x4 *>(p.bias + n);
                bj[j][q] = f32x4{(float)bb[0], (float)bb[1], (float)bb[2], (float)bb[3]};
            }
        }
    constexpr int kVec = 16 / kOutEs;              // elements per 16-byte vector
    constexpr int kVecPerRow = WN / kVec;          // 16 (fp32) or 8 (bf16)
    constexpr int kRowsPerPass = 64 / kVecPerRow;  // 4 (fp32) or 8 (bf16)
    const int rd_row = lane / kVecPerRow;
    const int rd_vec = lane % kVecPerRow;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f32x4 v = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                if (HAS_BIAS)
                    v = v + bj[j][q];
                if (GELU) {
                    v[0] = gelu_tanh(v[0]);
                    v[1] = gelu_tanh(v[1]);
                    v[2] = gelu_tanh(v[2]);
                    v[3] = gelu_tanh(v[3]);
                }
                OutT *dst = stage + mrow * kRowElems + j * 32 + q * 8 + ncol;
                if (OUT_BF16)
                    *reinterpret_cast<bf16x4 *>(dst) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
                else
                    *reinterpret_cast<f32x4 *>(dst) = v;
            }
        const int mbase = m0 + wave_m * WM + i * 32;
        const int ncol0 = n0 + wave_n * WN + rd_vec * kVec;
#pragma unroll
        for (int r = 0; r < 32; r += kRowsPerPass) {
            const int row = r + rd_row;
            const int m = mbase + row;
            const f32x4 v = *reinterpret_cast<const f32x4 *>(stage + row * kRowElems + rd_vec * kVec);
            if (m < p.M && ncol0 < p.N)
                *reinterpret_cast<f32x4 *>(reinterpret_cast<OutT *>(p.y) + (int64_t)m * p.ldy + ncol0) = v;
        }
    }
}

template <bool OUT_BF16, bool HAS_BIAS, bool GELU>
hipError_t launch_variant(const GemmParams &gp, hipStream_t stream)
{
    const dim3 grid(gp.tiles_m * gp.tiles_n);
    const dim3 block(kThreads);
    hipLaunchKernelGGL((gemm_bf16_nt_kernel<OUT_BF16, HAS_BIAS, GELU>), grid, block, 0, stream, gp);
    return hipGetLastError();
}

}  // namespace

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
    gp.tiles_m = (int)((pr.M + BM - 1) / BM);
    gp.tiles_n = (int)((pr.N + BN - 1) / BN);
    gp.group_m = gp.tiles_m < 8 ? gp.tiles_m : 8;
    const bool bias = pr.bias != nullptr;
    const int sel = (pr.out_bf16 ? 4 : 0) | (bias ? 2 : 0) | (pr.gelu ? 1 : 0);
    switch (sel) {
    case 0: return launch_variant<false, false, false>(gp, stream);
    case 1: return launch_variant<false, false, true>(gp, stream);
    case 2: return launch_variant<false, true, false>(gp, stream);
    case 3: return launch_variant<false, true, true>(gp, stream);
    case 4: return launch_variant<true, false, false>(gp, stream);
    case 5: return launch_variant<true, false, true>(gp, stream);
    case 6: return launch_variant<true, true, false>(gp, stream);
    default: return launch_variant<true, true, true>(gp, stream);
    }
}

}  // namespace tpl
