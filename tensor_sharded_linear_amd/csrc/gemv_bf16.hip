// gemv_bf16.hip -- weight-streaming kernel for skinny linear layers (M <= 16).
//
// The adaLN modulation projection reads a handful of conditioning vectors
// (one per sample) and a large weight; the Diffusers "Tensor parallelism"
// page (section "What to leave out") singles it out as the one large
// standalone projection.  With M of 1..16 the work is a matrix-vector product
// bound by how fast the weight streams from HBM, so it gets its own kernel:
//
//  * the M activation rows are staged once per workgroup in LDS (bf16);
//  * each wave takes whole weight rows n (grid-stride over rows), the 64 lanes
//    read consecutive 16-byte chunks of the row (1 KiB per instruction, fully
//    coalesced), several chunks in flight per lane;
//  * per chunk and activation row, four v_dot2_f32_bf16 accumulate in fp32;
//  * a butterfly over the 64 lanes reduces each row's M sums; lanes 0..M-1
//    apply bias / GELU-tanh and store.
#include "tp_internal.h"

namespace tpl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 6;  // 16-byte chunks in flight per lane per batch

struct GemvParams {
    const uint16_t *x;
    const uint16_t *w;
    const uint16_t *bias;
    void *y;
    int64_t ldx, ldw, ldy;
    int M, N, K;
};

__device__ __forceinline__ float gelu_tanh(float v)
{
    const float kSqrt2OverPi = 0.7978845608028654f;
    const float u = kSqrt2OverPi * (v + 0.044715f * v * v * v);
    return v / (1.0f + __expf(-2.0f * u));
}

__device__ __forceinline__ float dot8(const bf16x8 &a, const bf16x8 &b, float acc)
{
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[0], a[1]}, bf16x2{b[0], b[1]}, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[2], a[3]}, bf16x2{b[2], b[3]}, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[4], a[5]}, bf16x2{b[4], b[5]}, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[6], a[7]}, bf16x2{b[6], b[7]}, acc, false);
    return acc;
}

template <int BMAX, bool OUT_BF16, bool HAS_BIAS, bool GELU>
__global__ __launch_bounds__(kThreads) void gemv_bf16_kernel(GemvParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // [M][K]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nch = p.K >> 3;  // 16-byte chunks per row (K % 64 == 0)

    // Stage the activation rows.
    for (int idx = tid; idx < p.M * nch; idx += kThreads) {
        const int b = idx / nch;
        const int c = idx - b * nch;
        *reinterpret_cast<bf16x8 *>(xs + b * p.K + c * 8) =
            *reinterpret_cast<const bf16x8 *>(p.x + (int64_t)b * p.ldx + c * 8);
    }
    __syncthreads();

    const int wave_stride = gridDim.x * kWaves;
    for (int n = blockIdx.x * kWaves + wave; n < p.N; n += wave_stride) {
        const uint16_t *wr = p.w + (int64_t)n * p.ldw;
        float acc[BMAX];
#pragma unroll
        for (int b = 0; b < BMAX; ++b)
            acc[b] = 0.f;
        for (int c0 = 0; c0 < nch; c0 += 64 * kUnroll) {
            bf16x8 wv[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int c = c0 + u * 64 + lane;
                if (c < nch)
                    wv[u] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(wr + c * 8));
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int c = c0 + u * 64 + lane;
                if (c < nch) {
#pragma unroll
                    for (int b = 0; b < BMAX; ++b) {
                        if (b < p.M) {
                            const bf16x8 xv = *reinterpret_cast<const bf16x8 *>(xs + b * p.K + c * 8);
                            acc[b] = dot8(wv[u], xv, acc[b]);
                        }
                    }
                }
            }
        }
        // Butterfly reduction over the wave: every lane ends with the row totals.
#pragma unroll
        for (int b = 0; b < BMAX; ++b) {
            if (b < p.M) {
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1)
                    acc[b] += __shfl_xor(acc[b], off, 64);
            }
        }
        if (lane < p.M) {
            float v = 0.f;
#pragma unroll
            for (int b = 0; b < BMAX; ++b)
                if (b == lane)
                    v = acc[b];
            if (HAS_BIAS)
                v += (float)(*reinterpret_cast<const __bf16 *>(p.bias + n));
            if (GELU)
                v = gelu_tanh(v);
            if (OUT_BF16)
                *reinterpret_cast<__bf16 *>(reinterpret_cast<uint16_t *>(p.y) + (int64_t)lane * p.ldy + n) = (__bf16)v;
            else
                reinterpret_cast<float *>(p.y)[(int64_t)lane * p.ldy + n] = v;
        }
    }
}

template <int BMAX, bool OUT_BF16, bool HAS_BIAS, bool GELU>
hipError_t launch_variant(const GemvParams &gp, hipStream_t stream)
{
    const size_t lds = (size_t)gp.M * gp.K * sizeof(uint16_t);
    auto kern = gemv_bf16_kernel<BMAX, OUT_BF16, HAS_BIAS, GELU>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    int blocks = (gp.N + kWaves - 1) / kWaves;
    // Persistent-style grid: a few workgroups per CU, rows strided over waves,
    // so the activation rows are staged into LDS only a few times per CU.
    const int cap = 256 * 2;
    if (blocks > cap)
        blocks = cap;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), lds, stream, gp);
    return hipGetLastError();
}

template <int BMAX>
hipError_t launch_bmax(const GemvParams &gp, bool out_bf16, bool bias, bool gelu, hipStream_t s)
{
    const int sel = (out_bf16 ? 4 : 0) | (bias ? 2 : 0) | (gelu ? 1 : 0);
    switch (sel) {
    case 0: return launch_variant<BMAX, false, false, false>(gp, s);
    case 1: return launch_variant<BMAX, false, false, true>(gp, s);
    case 2: return launch_variant<BMAX, false, true, false>(gp, s);
    case 3: return launch_variant<BMAX, false, true, true>(gp, s);
    case 4: return launch_variant<BMAX, true, false, false>(gp, s);
    case 5: return launch_variant<BMAX, true, false, true>(gp, s);
    case 6: return launch_variant<BMAX, true, true, false>(gp, s);
    default: return launch_variant<BMAX, true, true, true>(gp, s);
    }
}

}  // namespace

hipError_t launch_gemv(const LinearProblem &pr, hipStream_t stream)
{
    GemvParams gp;
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
    const bool bias = pr.bias != nullptr;
    if (pr.M <= 4)
        return launch_bmax<4>(gp, pr.out_bf16, bias, pr.gelu, stream);
    return launch_bmax<16>(gp, pr.out_bf16, bias, pr.gelu, stream);
}

}  // namespace tpl
