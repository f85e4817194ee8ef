// gemm_narrow.hip -- split-K MFMA kernel for linear layers with few rows.
//
// Between the weight-streaming kernel's row limit and 128 rows (a small batch of
// tokens: a short text stream, the tiny MLP's 64 tokens, adaLN inputs past the
// weight-streaming kernel's limit), Y = X . W^T moves the whole weight for 2 M
// flops per weight element, so the weight stream, not the matrix cores, sets
// the time.  The tiled GEMM's 192-row tiles would be mostly padding and give
// only N / 192 workgroups for 256 CUs (9216 x 6144 weight: 97-103 us at 7 to
// 128 rows).  Here instead:
//
//  * a workgroup of 4 waves owns all M rows, as MB = ceil(M / 16) <= 8 blocks
//    of 16 (6 for 5 blocks, 8 for 7), and a run of output columns (weight rows) sized so that every CU
//    streams about the same number of weight lines: 9216 columns on 256 CUs
//    give 256 runs of 36 (three 16-row weight blocks, the last one partial),
//    where fixed 32-column runs (288 workgroups) left 32 CUs with two and took
//    29 us at 7 rows instead of 22.5; with SwiGLU a run is up to 16 gate rows
//    and the matching up rows of the packed weight;
//  * its waves split K in steps of 64, dealt round-robin (wave w takes steps
//    w, w + 4, ...), so the 4 waves read neighbouring 128-byte pieces of each
//    row;
//  * every load covers whole 128-byte lines, 8 lanes per line: the L1 issues
//    one L2 request per line it is asked for and keeps a limited number in
//    flight per CU, so lanes that each fetched their own MFMA fragment (16 rows
//    x 64 bytes per load) halved the bytes per request and held the weight
//    stream at 2.4-2.7 TB/s (7 rows, 32-column runs: 47 us against 28 us);
//  * a wave passes each step's lines through its own LDS area (one 2 KiB
//    16 x 64 tile per block, XOR-swizzled) into the fragment layout of
//    v_mfma_f32_16x16x32_bf16, the weight as the A operand;
//  * D steps of loads are in flight per wave (6, 4, 3 or 2 as the weight and
//    activation blocks number 2, 3, 4 or more): no load sits in a conditional block (rows past the end are
//    clamped to the last row, steps past the end to the last step, and the
//    extra data is discarded) and the loads go out in step order, so the
//    compiler's in-order load counting keeps all D in flight;
//  * the 4 waves' fp32 partial tiles meet in LDS and are added in wave order,
//    so each output is the same sum whatever N is; one (block, lane) item per
//    thread then applies bias, GELU or SwiGLU and rounding, and stores the 4
//    consecutive columns its lane holds.
//
// Every workgroup reads all of X (M x K) besides its weight rows, so the
// activation's share of the requests grows with M: 9216 x 6144 takes 22.5 us at
// 7 rows, 31 us at 64 and 46 us at 128 (the weight alone at 8 TB/s: 14 us).
// Beyond 128 rows the activation's re-reads would outweigh the weight, and the
// tiled kernel takes over.
#include "tp_internal.h"
#include <type_traits>

namespace tpl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxRows = 48;      // weight rows per workgroup (3 blocks of 16)
constexpr int kMaxGatedRows = 16; // gate rows (and as many up rows) per workgroup

constexpr int kActNone = 0;
constexpr int kActGelu = 1;
constexpr int kActSwiglu = 2;

struct NarrowParams {
    const uint16_t *x;
    const uint16_t *w;
    const uint16_t *bias;
    void *y;
    int64_t ldx, ldw, ldy;
    int M, N, K;
    int rows;  // output columns (weight rows) per workgroup, a multiple of 4
};

// GELU, tanh form, as in the tiled kernel: g(v) = v / (1 + exp(-2u)),
// u = sqrt(2/pi) (v + 0.044715 v^3), with exp(-2u) = 2^(v (a + b v^2)) on the
// hardware exp2 and the reciprocal.
__device__ __forceinline__ float gelu_tanh(float v)
{
    const float a = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
    const float b = 0.044715f * a;
    const float e = __builtin_amdgcn_exp2f(v * __builtin_fmaf(b, v * v, a));
    return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// SiLU as in the tiled kernel: v / (1 + 2^(-v log2(e))).
__device__ __forceinline__ float silu(float v)
{
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * -1.4426950408889634f));
}

__device__ __forceinline__ f32x4 bias4(const uint16_t *b, int n)
{
    const bf16x4 bb = *reinterpret_cast<const bf16x4 *>(b + n);
    return f32x4{(float)bb[0], (float)bb[1], (float)bb[2], (float)bb[3]};
}

// Steps (64 k each) whose loads are in flight per wave: 8 (NB + MB) registers per step.
// From 8 blocks on (up to 3 weight and 8 activation blocks) one step, the registers of a
// second going to the accumulators; the other waves of the CU keep the loads going.
template <int MB, int NB>
constexpr int depth()
{
    return (NB + MB) <= 2 ? 6 : ((NB + MB) == 3 ? 4 : ((NB + MB) == 4 ? 3 : ((NB + MB) <= 7 ? 2 : 1)));
}

// LDS: during the k loop each wave's transpose area (one 2 KiB tile of 16 rows x 64 k per
// block), after it the waves' partial sums (one 16 x 16 fp32 tile per output block).
template <int MB, int NB>
struct NarrowLds {
    union {
        bf16x8 xpose[kWaves][NB + MB][128];
        f32x4 red[kWaves][MB * NB][64];
    };
};

// NB 16-row weight blocks cover the workgroup's p.rows weight rows (gated: block 0 the
// gate rows, block 1 the matching up rows, p.rows <= 16).
template <int MB, int NB, int ACT, bool OUT_BF16, bool HAS_BIAS>
__global__ __launch_bounds__(kThreads) void gemm_narrow_kernel(NarrowParams p)
{
    constexpr bool kGated = ACT == kActSwiglu;
    static_assert(!kGated || NB == 2, "the gated form pairs one gate and one up block");
    constexpr int kNB = NB;
    constexpr int D = depth<MB, NB>();
    __shared__ NarrowLds<MB, NB> lds;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * p.rows;
    const int n_end = min(n0 + p.rows, p.N);  // a multiple of 4
    // Steps of 64 k, dealt round-robin: wave w takes steps w, w + 4, ..., so at any time the
    // 4 waves read neighbouring 128-byte pieces of each row.
    const int steps = ((p.K >> 6) - wave + kWaves - 1) / kWaves;

    // Each load covers 8 rows x 128 bytes of a 16-row block: lane l fetches 16-byte chunk
    // l % 8 of row l / 8 (load h = 0) or 8 + l / 8 (h = 1), so every 8 lanes read one whole
    // 128-byte line.  The L1 sends one request per line it is asked for; with fewer lanes
    // per line (each lane loading its MFMA fragment directly: 16 rows x 64 bytes per load)
    // it sent 64-byte requests, and the number of requests it keeps in flight per CU held
    // the weight stream to well under half the rate.  Weight rows of block j:
    // n0 + 16 j + 8 h + l / 8 (gated: block 0 the gate rows n0 + ..., block 1 the up rows
    // N + n0 + ...), clamped to the workgroup's last row; activation rows of block i:
    // 16 i + 8 h + l / 8, clamped to the last row.  Clamped rows repeat a line that the
    // same load already asks for, which costs no extra request.
    const int lrow = lane >> 3, lchunk = lane & 7;
    const int kofs = wave * 64 + 8 * lchunk;
    const bf16x8 *wp[kNB][2];
    const bf16x8 *xp[MB][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
            const int r = kGated ? j * p.N + min(n0 + 8 * h + lrow, n_end - 1)
                                 : min(n0 + 16 * j + 8 * h + lrow, n_end - 1);
            wp[j][h] = reinterpret_cast<const bf16x8 *>(p.w + (int64_t)r * p.ldw + kofs);
        }
#pragma unroll
        for (int i = 0; i < MB; ++i)
            xp[i][h] = reinterpret_cast<const bf16x8 *>(p.x + (int64_t)min(16 * i + 8 * h + lrow, p.M - 1) * p.ldx +
                                                        kofs);
    }
    // The wave's transpose area: per block, 16 rows x 8 chunks of 16 bytes, chunk c of row
    // r at slot 8 r + (c ^ (r & 7)), so that the writes (8 chunks of one row per 8 lanes) and
    // the fragment reads (chunk 4 s + l / 16 of row l % 16, 8 rows per 8 lanes) hit distinct
    // banks.
    const int fr = lane & 15;
    int wslot[2], rslot[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        wslot[h] = 8 * (8 * h + lrow) + (lchunk ^ lrow);
        rslot[h] = 8 * fr + ((4 * h + (lane >> 4)) ^ (fr & 7));
    }

    f32x4 acc[MB][kNB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (steps > 0) {
        bf16x8 wb[D][kNB][2], xb[D][MB][2];
        // Step s of the wave starts 4 x 64 elements (32 vectors) after step s - 1.
        auto load = [&](int u, int s) {
            const int o = min(s, steps - 1) * (8 * kWaves);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int j = 0; j < kNB; ++j)
                    wb[u][j][h] = __builtin_nontemporal_load(wp[j][h] + o);
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    xb[u][i][h] = xp[i][h][o];
            }
        };
        // Step u's lines pass through the wave's LDS area into the MFMA fragment layout:
        // for k32 half s, lane l holds k = 32 s + 8 (l / 16) .. + 8 of row l % 16 of each block.
        auto mma = [&](int u) {
            bf16x8(*t)[128] = lds.xpose[wave];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int j = 0; j < kNB; ++j)
                    t[j][wslot[h]] = wb[u][j][h];
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    t[kNB + i][wslot[h]] = xb[u][i][h];
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                bf16x8 fw[kNB], fx[MB];
#pragma unroll
                for (int j = 0; j < kNB; ++j)
                    fw[j] = t[j][rslot[s]];
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    fx[i] = t[kNB + i][rslot[s]];
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int j = 0; j < kNB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[j], fx[i], acc[i][j], 0, 0, 0);
            }
        };
        // The loads are issued in step order, here and in the loop, and the scheduling
        // barriers keep them so: the compiler counts outstanding loads in issue order, so
        // waiting for step s then waits for nothing issued after it.  (With the prologue's
        // loads reordered, the loop's first wait covered every load in flight.)
#pragma unroll
        for (int u = 0; u < D; ++u) {
            load(u, u);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Whole groups of D steps: the MFMAs of a step, then the loads of the step D later
        // into the registers they freed.  The last group's loads re-read the wave's last
        // step (clamped) where the steps run out; the tail below discards them.
        const int groups = steps / D;
        for (int g = 0; g < groups; ++g) {
#pragma unroll
            for (int u = 0; u < D; ++u) {
                mma(u);
                load(u, (g + 1) * D + u);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        const int rest = steps - groups * D;
#pragma unroll
        for (int u = 0; u < D - 1; ++u)
            if (u < rest)
                mma(u);
    }

    __syncthreads();  // every wave is done with its transpose area
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j)
            lds.red[wave][i * kNB + j][lane] = acc[i][j];
    __syncthreads();

    typedef typename std::conditional<OUT_BF16, __bf16, float>::type OutT;
    // Item (block, l): lane l of every wave holds Y[16 i + l % 16][n .. n + 3],
    // n = column base + 16 j + 4 (l / 16).  n and n_end are multiples of 4, so n < n_end
    // covers n + 3.
    constexpr int kItems = (kGated ? MB : MB * kNB) * 64;
    for (int e = threadIdx.x; e < kItems; e += kThreads) {
        const int l = e & 63;
        const int blk = kGated ? (e >> 6) * kNB : e >> 6;
        const int m = 16 * (blk / kNB) + (l & 15);
        const int n = n0 + 16 * (blk % kNB) + 4 * (l >> 4);
        f32x4 v = lds.red[0][blk][l];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            v += lds.red[w][blk][l];
        if (m >= p.M || n >= n_end)
            continue;
        if (HAS_BIAS)
            v += bias4(p.bias, n);
        if (ACT == kActGelu) {
            v[0] = gelu_tanh(v[0]);
            v[1] = gelu_tanh(v[1]);
            v[2] = gelu_tanh(v[2]);
            v[3] = gelu_tanh(v[3]);
        }
        if (kGated) {
            f32x4 u = lds.red[0][blk + 1][l];
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
                u += lds.red[w][blk + 1][l];
            if (HAS_BIAS)
                u += bias4(p.bias, p.N + n);
            v[0] = silu(v[0]) * u[0];
            v[1] = silu(v[1]) * u[1];
            v[2] = silu(v[2]) * u[2];
            v[3] = silu(v[3]) * u[3];
        }
        OutT *dst = reinterpret_cast<OutT *>(p.y) + (int64_t)m * p.ldy + n;
        if (OUT_BF16)
            *reinterpret_cast<bf16x4 *>(dst) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        else
            *reinterpret_cast<f32x4 *>(dst) = v;
    }
}

template <int MB, int NB, int ACT, bool OUT_BF16, bool HAS_BIAS>
hipError_t launch_mb(const NarrowParams &np, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_narrow_kernel<MB, NB, ACT, OUT_BF16, HAS_BIAS>), dim3((np.N + np.rows - 1) / np.rows),
                       dim3(kThreads), 0, stream, np);
    return hipGetLastError();
}

template <int NB, int ACT, bool OUT_BF16, bool HAS_BIAS>
hipError_t launch_nb(const NarrowParams &np, hipStream_t stream)
{
    switch ((np.M + 15) / 16) {
    case 1: return launch_mb<1, NB, ACT, OUT_BF16, HAS_BIAS>(np, stream);
    case 2: return launch_mb<2, NB, ACT, OUT_BF16, HAS_BIAS>(np, stream);
    case 3: return launch_mb<3, NB, ACT, OUT_BF16, HAS_BIAS>(np, stream);
    case 4: return launch_mb<4, NB, ACT, OUT_BF16, HAS_BIAS>(np, stream);
    case 5:
    case 6: return launch_mb<6, NB, ACT, OUT_BF16, HAS_BIAS>(np, stream);
    default: return launch_mb<8, NB, ACT, OUT_BF16, HAS_BIAS>(np, stream);
    }
}

template <int ACT, bool OUT_BF16, bool HAS_BIAS>
hipError_t launch_act(const NarrowParams &np, hipStream_t stream)
{
    if constexpr (ACT == kActSwiglu) {
        return launch_nb<2, ACT, OUT_BF16, HAS_BIAS>(np, stream);
    } else {
        switch ((np.rows + 15) / 16) {
        case 1: return launch_nb<1, ACT, OUT_BF16, HAS_BIAS>(np, stream);
        case 2: return launch_nb<2, ACT, OUT_BF16, HAS_BIAS>(np, stream);
        default: return launch_nb<3, ACT, OUT_BF16, HAS_BIAS>(np, stream);
        }
    }
}

template <bool OUT_BF16, bool HAS_BIAS>
hipError_t launch_out(const NarrowParams &np, int act, hipStream_t stream)
{
    switch (act) {
    case kActGelu: return launch_act<kActGelu, OUT_BF16, HAS_BIAS>(np, stream);
    case kActSwiglu: return launch_act<kActSwiglu, OUT_BF16, HAS_BIAS>(np, stream);
    default: return launch_act<kActNone, OUT_BF16, HAS_BIAS>(np, stream);
    }
}

// Weight rows per workgroup.  The CUs share the weight stream; a CU's time goes with the
// lines it requests: its workgroups' weight rows plus, for each workgroup, the activation
// rows (every workgroup reads all of X; an activation line, served from L2, costs about
// 0.6 of a weight line from HBM).  Workgroups beyond one per CU run on the same CUs, so the
// cost of a choice is ceil(workgroups / CUs) x (rows + 0.6 M) (gated: 2 rows per output).
// Rows are a multiple of 4 (the epilogue stores 4 columns per lane), at most 48 (16 gated).
// Ties go to more rows per workgroup (fewer activation re-reads).  9216 outputs on 256 CUs
// take 36 rows: 256 workgroups, one per CU; 32 rows per workgroup left 32 CUs with two.
int pick_rows(int64_t M, int64_t N, bool gated, int cus)
{
    const int max_rows = gated ? kMaxGatedRows : kMaxRows;
    const double x_cost = 0.6 * (double)M;
    int best = 4;
    double best_cost = -1;
    for (int rows = 4; rows <= max_rows; rows += 4) {
        const int64_t wgs = (N + rows - 1) / rows;
        const int64_t rounds = (wgs + cus - 1) / cus;
        const double cost = (double)rounds * ((gated ? 2 : 1) * rows + x_cost);
        if (best_cost < 0 || cost <= best_cost) {
            best = rows;
            best_cost = cost;
        }
    }
    return best;
}

}  // namespace

bool narrow_supports(const LinearProblem &pr)
{
    if (pr.M < 1 || pr.M > kNarrowMaxM)
        return false;
    // One 256-thread workgroup per run: the launch's thread count must stay below 2^32.
    const int rows = pick_rows(pr.M, pr.N, pr.swiglu, cu_count());
    return (pr.N + rows - 1) / rows <= ((int64_t)1 << 23);
}

void narrow_tile_shape(const LinearProblem &pr, int *rows, int *cols)
{
    const int mb = (int)((pr.M + 15) / 16);
    *rows = 16 * (mb == 5 ? 6 : (mb == 7 ? 8 : mb));  // the instance launch_nb picks
    *cols = pick_rows(pr.M, pr.N, pr.swiglu, cu_count());
}

hipError_t launch_narrow(const LinearProblem &pr, hipStream_t stream)
{
    if (!narrow_supports(pr))
        return hipErrorInvalidValue;  // the caller checks narrow_supports()
    NarrowParams np;
    np.x = pr.x;
    np.w = pr.w;
    np.bias = pr.bias;
    np.y = pr.y;
    np.ldx = pr.ldx;
    np.ldw = pr.ldw;
    np.ldy = pr.ldy;
    np.M = (int)pr.M;
    np.N = (int)pr.N;
    np.K = (int)pr.K;
    np.rows = pick_rows(pr.M, pr.N, pr.swiglu, cu_count());
    const int act = pr.swiglu ? kActSwiglu : (pr.gelu ? kActGelu : kActNone);
    if (pr.out_bf16)
        return pr.bias ? launch_out<true, true>(np, act, stream) : launch_out<true, false>(np, act, stream);
    return pr.bias ? launch_out<false, true>(np, act, stream) : launch_out<false, false>(np, act, stream);
}

}  // namespace tpl
