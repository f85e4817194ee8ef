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
//  * 256 x 256 output tile per workgroup, K step 64, 512 threads = 8 waves in a
//    2 (M) x 4 (N) grid; each wave owns a 128 x 64 sub-tile held as 8 x 4
//    MFMA 16x16 fp32 accumulators (128 accumulator registers per lane).
//  * Operands go HBM/L2 -> LDS by direct-to-LDS DMA (global_load_lds_dwordx4),
//    no VGPR staging, double-buffered: 2 stages x (X tile + W tile) x 32 KiB =
//    128 KiB of the 160 KiB LDS.  The DMA for step t+1 is issued before the
//    MFMAs of step t.
//  * LDS tiles are 64-element (128-byte) rows; the 16-byte chunk c of row r is
//    stored at position c ^ (r & 7), so the eight lanes that read one
//    16-byte column of a fragment hit eight different bank groups.
//  * The W fragment is the MFMA "A" operand and the X fragment the "B"
//    operand, so each lane ends up holding four consecutive output columns of
//    one row: the epilogue stores 16-byte (fp32) / 8-byte (bf16) vectors.
//  * Workgroups are dealt round-robin to the 8 XCDs; the tile index is
//    remapped so each XCD gets a contiguous run of a grouped raster order,
//    which keeps its concurrent tiles on few X row-panels and W row-panels
//    (shared in that XCD's L2).
//  * Ragged M and N: loads clamp the row index to the last valid row (the
//    extra rows are computed and discarded), stores are masked.
#include "tp_internal.h"

namespace tpl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define TPL_LDS(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kThreads = 512;
constexpr int kWavesN = 4;
constexpr int WM = 128;           // rows of the output owned by one wave
constexpr int WN = 64;            // columns of the output owned by one wave
constexpr int FM = WM / 16;       // 16-row MFMA fragments per wave
constexpr int FN = WN / 16;       // 16-column MFMA fragments per wave
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

__device__ __forceinline__ void wait_dma_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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

template <bool OUT_BF16, bool HAS_BIAS, bool GELU>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_nt_kernel(GemmParams p)
{
    __shared__ __attribute__((aligned(1024))) uint16_t lds[kLdsElems];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    int tm, tn;
    tile_coords(blockIdx.x, p, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    // DMA addressing.  Instruction j of wave w fills LDS chunks
    // [(8j + w) * 64, +64) of a 256x64 tile: lane l lands at tile row
    // 64j + 8w + l/8, stored position l%8, i.e. logical chunk (l%8) ^ (l/8).
    const int dma_row = wave * 8 + (lane >> 3);
    const int dma_chunk = (lane & 7) ^ (lane >> 3);
    const uint16_t *xsrc[4];
    const uint16_t *wsrc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = j * 64 + dma_row;
        const int gm = min(m0 + r, p.M - 1);
        const int gn = min(n0 + r, p.N - 1);
        xsrc[j] = p.x + (int64_t)gm * p.ldx + dma_chunk * 8;
        wsrc[j] = p.w + (int64_t)gn * p.ldw + dma_chunk * 8;
    }

    auto issue = [&](int stage, int k0) {
        uint16_t *xs = lds + stage * kStageElems;
        uint16_t *ws = xs + kTileElems;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_global_load_lds(xsrc[j] + k0, TPL_LDS(xs + (j * 8 + wave) * 512), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_global_load_lds(wsrc[j] + k0, TPL_LDS(ws + (j * 8 + wave) * 512), 16, 0, 0);
    };

    // Fragment addressing: lane l reads row (l % 16) of a 16-row fragment,
    // 16-byte k-chunk (4 kk + l / 16); the row's low 3 bits equal l % 8.
    const int wave_m = wave / kWavesN;
    const int wave_n = wave % kWavesN;
    const int xrow_off = (wave_m * WM + (lane & 15)) * BK;
    const int wrow_off = (wave_n * WN + (lane & 15)) * BK;
    const int swz = lane & 7;
    const int kq = lane >> 4;

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int T = p.K / BK;
    issue(0, 0);
    wait_dma_all();
    __syncthreads();

    for (int t = 0; t < T; ++t) {
        if (t + 1 < T)
            issue((t + 1) & 1, (t + 1) * BK);
        const uint16_t *xs = lds + (t & 1) * kStageElems;
        const uint16_t *ws = xs + kTileElems;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int cpos = ((kk * 4 + kq) ^ swz) * 8;
            bf16x8 xf[FM], wf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                xf[i] = *reinterpret_cast<const bf16x8 *>(xs + xrow_off + i * 16 * BK + cpos);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                wf[j] = *reinterpret_cast<const bf16x8 *>(ws + wrow_off + j * 16 * BK + cpos);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
        }
        wait_dma_all();
        __syncthreads();
    }

    // Epilogue: lane holds Y[m][n .. n+3], m = row base + 16 i + l%16,
    // n = column base + 16 j + 4 (l / 16).
    const int mb = m0 + wave_m * WM + (lane & 15);
    const int nb = n0 + wave_n * WN + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = nb + j * 16;
        if (n >= p.N)
            continue;  // N % 16 == 0: a fragment's 16 columns are all in or all out
        f32x4 b = f32x4{0.f, 0.f, 0.f, 0.f};
        if (HAS_BIAS) {
            const bf16x4 bb = *reinterpret_cast<const bf16x4 *>(p.bias + n);
            b = f32x4{(float)bb[0], (float)bb[1], (float)bb[2], (float)bb[3]};
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = mb + i * 16;
            if (m >= p.M)
                continue;
            f32x4 v = acc[i][j];
            if (HAS_BIAS)
                v = v + b;
            if (GELU) {
                v[0] = gelu_tanh(v[0]);
                v[1] = gelu_tanh(v[1]);
                v[2] = gelu_tanh(v[2]);
                v[3] = gelu_tanh(v[3]);
            }
            if (OUT_BF16) {
                bf16x4 o = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
                *reinterpret_cast<bf16x4 *>(reinterpret_cast<uint16_t *>(p.y) + (int64_t)m * p.ldy + n) = o;
            } else {
                *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.y) + (int64_t)m * p.ldy + n) = v;
            }
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
