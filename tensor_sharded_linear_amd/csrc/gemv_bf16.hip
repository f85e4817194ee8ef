// gemv_bf16.hip -- weight-streaming kernel for skinny linear layers (M <= 5).
//
// The adaLN modulation projection reads a handful of conditioning vectors
// (one per sample) and a large weight; the Diffusers "Tensor parallelism"
// page (section "What to leave out") singles it out as the one large
// standalone projection.  With M of 1..5 the work is a matrix-vector product
// bound by how fast the weight streams from HBM, so it gets its own kernel:
//
//  * one persistent 512-thread workgroup per CU stages the M activation rows
//    in LDS once (bf16, M * K * 2 bytes); its staging loads are all issued
//    before the first is stored, and before the wave's first weight row, so
//    they cost one memory round trip and the row stays in flight meanwhile;
//  * each wave takes whole weight rows n (strided over all waves of the
//    grid); its 64 lanes read consecutive 16-byte chunks of the row (1 KiB per
//    instruction, fully coalesced, non-temporal), the whole row in one batch;
//  * the loads of the wave's next row are issued before the current row is
//    reduced, so every wave keeps a row (K * 2 bytes) in flight while it
//    computes.  That holds only while no load sits in a conditional block
//    (below); with the last rows guarded inside the loop the compiler's waits
//    kept one row in flight, and a cold 9216 x 6144 weight with 4 rows took
//    21.2 us instead of 19.3 (36864 x 1536: 22.5 instead of 18.7);
//  * per chunk and activation row, four v_dot2_f32_bf16 accumulate in fp32;
//    a butterfly over the 64 lanes (DPP inside 16-lane rows, shuffles across
//    rows) reduces each row's M sums, and lanes 0..M-1 apply bias / GELU-tanh
//    and store.
#include "tp_internal.h"

namespace tpl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

struct GemvParams {
    const uint16_t *x;
    const uint16_t *w;
    const uint16_t *bias;
    void *y;
    int64_t ldx, ldw, ldy;
    int M, N, K;
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

__device__ __forceinline__ float dot8(const bf16x8 &a, const bf16x8 &b, float acc)
{
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[0], a[1]}, bf16x2{b[0], b[1]}, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[2], a[3]}, bf16x2{b[2], b[3]}, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[4], a[5]}, bf16x2{b[4], b[5]}, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[6], a[7]}, bf16x2{b[6], b[7]}, acc, false);
    return acc;
}

// Sum over the 64 lanes of a wave.  Inside each 16-lane row the butterfly
// uses DPP lane swizzles (VALU, no LDS round trip): swap neighbours, swap
// pairs, mirror each 8-lane half, mirror the row.  The two cross-row steps use
// lane shuffles.  Every lane ends with the total.
__device__ __forceinline__ float wave_sum(float v)
{
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

// NIT = 16-byte chunks per lane per row = ceil(K / 512); B = activation rows.
// The activations sit in LDS with a row pitch of K + 8: each row is followed by
// a zero chunk.  Lanes whose chunk index runs past the row re-read the weight
// row's last chunk and pair it with their activation row's zero chunk, so
// neither the loads nor the dot products branch per lane.  The epilogue options (bias,
// GELU, output dtype) are uniform runtime flags: they act once per row.
//
// No global load sits in a conditional block.  The compiler counts outstanding
// loads per wave statically; a load that may or may not have been issued forces
// it to assume the smaller count, and a wait for one row then also waits for the
// next row's loads, which leaves one row in flight instead of two.  So the
// staging loads clamp their index, every row load (and the row's bias) is for a
// row that exists, and the last one or two rows of a wave are peeled out of the
// loop instead of guarded inside it.  The bias is loaded before the row's chunks,
// so waiting for it does not wait for them.
template <int NIT, int B>
__global__ __launch_bounds__(kThreads) void gemv_bf16_kernel(GemvParams p, int out_bf16, int gelu, int wave_major)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // [B][K + 8], zeros in the last 8
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nch = p.K >> 3;  // 16-byte chunks per row (K % 64 == 0)
    constexpr int UB = B >= 8 ? 1 : 8 / B;  // chunks per LDS batch (8 vectors)
    constexpr int kStage = (B * NIT * 64 + kThreads - 1) / kThreads;  // staging loads per thread
    constexpr int kStage1 = kStage < 8 ? kStage : 8;  // of which issued before the first row

    const int pitch = p.K + 8;  // LDS row pitch of the activations
    auto wch = [&](int u) { return min(u * 64 + lane, nch - 1) * 8; };
    auto xch = [&](int u) { return u * 64 + lane < nch ? (u * 64 + lane) * 8 : p.K; };

    const int stride = gridDim.x * kWaves;
    // This wave's first row.  When the rows do not divide evenly over the waves, the waves
    // that take one row more are spread over all workgroups (wave-major numbering) instead
    // of filling the first ones: 9216 rows on 2048 waves, 1 or 2 activation rows, 4% faster
    // cold.  With an even division the workgroup-major order (each workgroup's waves on
    // neighbouring rows) measured 1-3% faster.
    const int first = wave_major ? wave * gridDim.x + blockIdx.x : blockIdx.x * kWaves + wave;
    const int cnt = first < p.N ? (p.N - first + stride - 1) / stride : 0;  // its rows
    const uint16_t *bias_src = p.bias ? p.bias : p.w;  // a valid address either way
    const int lane_out = lane < B ? lane : B - 1;      // lanes past B repeat row B-1's store
    bf16x8 ra[NIT], rb[NIT];
    uint16_t ba = 0, bb = 0;

#define TPL_LOAD_ROW(i, r, bv)                                                               \
    do {                                                                                     \
        const int n_ = min(first + (i) * stride, p.N - 1);                                    \
        const uint16_t *src_ = p.w + (int64_t)n_ * p.ldw;                                     \
        bv = bias_src[n_];                                                                   \
        _Pragma("unroll") for (int u = 0; u < NIT; ++u)                                      \
            r[u] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(src_ + wch(u))); \
        __builtin_amdgcn_sched_barrier(0);                                                   \
    } while (0)

#define TPL_FINISH_ROW(i, r, bv)                                                             \
    do {                                                                                     \
        const int n_ = first + (i) * stride;                                                  \
        float acc_[B];                                                                       \
        _Pragma("unroll") for (int b = 0; b < B; ++b) acc_[b] = 0.f;                         \
        _Pragma("unroll") for (int u0 = 0; u0 < NIT; u0 += UB) {                             \
            bf16x8 xv_[UB][B];                                                               \
            _Pragma("unroll") for (int u = 0; u < UB; ++u)                                   \
                _Pragma("unroll") for (int b = 0; b < B; ++b)                                \
                    if (u0 + u < NIT)                                                        \
                        xv_[u][b] = *reinterpret_cast<const bf16x8 *>(xs + b * pitch + xch(u0 + u)); \
            _Pragma("unroll") for (int u = 0; u < UB; ++u)                                   \
                _Pragma("unroll") for (int b = 0; b < B; ++b)                                \
                    if (u0 + u < NIT)                                                        \
                        acc_[b] = dot8(r[u0 + u], xv_[u][b], acc_[b]);                        \
            __builtin_amdgcn_sched_barrier(0);                                               \
        }                                                                                    \
        _Pragma("unroll") for (int b = 0; b < B; ++b) acc_[b] = wave_sum(acc_[b]);           \
        float v_ = acc_[0];                                                                  \
        _Pragma("unroll") for (int b = 1; b < B; ++b) if (b == lane_out) v_ = acc_[b];       \
        if (p.bias) v_ += (float)__builtin_bit_cast(__bf16, bv);                             \
        if (gelu) v_ = gelu_tanh(v_);                                                        \
        if (out_bf16)                                                                        \
            *reinterpret_cast<__bf16 *>(reinterpret_cast<uint16_t *>(p.y) + (int64_t)lane_out * p.ldy + n_) = (__bf16)v_; \
        else                                                                                 \
            reinterpret_cast<float *>(p.y)[(int64_t)lane_out * p.ldy + n_] = v_;             \
    } while (0)

    // The staging loads go first: their LDS stores then wait for them alone, while the
    // first row's loads stay in flight across the barrier.
    {
        const int last = B * nch - 1;
        auto stage_load = [&](int i) {
            const int idx = min(tid + i * kThreads, last);
            const int bb_ = idx / nch;
            return *reinterpret_cast<const bf16x8 *>(p.x + (int64_t)bb_ * p.ldx + (idx - bb_ * nch) * 8);
        };
        auto stage_store = [&](int i, const bf16x8 &v) {
            const int idx = tid + i * kThreads;
            if (idx <= last) {
                const int bb_ = idx / nch;
                *reinterpret_cast<bf16x8 *>(xs + bb_ * pitch + (idx - bb_ * nch) * 8) = v;
            }
        };
        bf16x8 stg[kStage1];
#pragma unroll
        for (int i = 0; i < kStage1; ++i)
            stg[i] = stage_load(i);
        TPL_LOAD_ROW(0, ra, ba);  // a wave without rows loads row N - 1 and returns below
#pragma unroll
        for (int i = 0; i < kStage1; ++i)
            stage_store(i, stg[i]);
        // Many activation rows: the rest one at a time (these waits include the first row).
#pragma unroll
        for (int i = kStage1; i < kStage; ++i)
            stage_store(i, stage_load(i));
    }
    if (tid < B)
        *reinterpret_cast<bf16x8 *>(xs + tid * pitch + p.K) = bf16x8{};
    __syncthreads();
    if (cnt == 0)
        return;

    // Two rows in flight per wave: one is reduced while the next loads.
    int i = 0;
    for (; i + 2 < cnt; i += 2) {
        TPL_LOAD_ROW(i + 1, rb, bb);
        TPL_FINISH_ROW(i, ra, ba);
        TPL_LOAD_ROW(i + 2, ra, ba);
        TPL_FINISH_ROW(i + 1, rb, bb);
    }
    if (i + 2 == cnt) {
        TPL_LOAD_ROW(i + 1, rb, bb);
        TPL_FINISH_ROW(i, ra, ba);
        TPL_FINISH_ROW(i + 1, rb, bb);
    } else {
        TPL_FINISH_ROW(i, ra, ba);
    }
#undef TPL_LOAD_ROW
#undef TPL_FINISH_ROW
}

template <int NIT, int B>
hipError_t launch_variant(const GemvParams &gp, bool out_bf16, bool gelu, hipStream_t stream)
{
    // At most 5 rows of 6144 + 8 (or 2 of 8192 + 8) elements: within the 64 KiB of dynamic
    // LDS a launch gets without raising the limit.
    const size_t lds = (size_t)B * (gp.K + 8) * sizeof(uint16_t);
    auto kern = gemv_bf16_kernel<NIT, B>;
    // One persistent workgroup per CU (256 CUs), fewer if there are fewer rows.
    int blocks = (gp.N + kWaves - 1) / kWaves;
    if (blocks > 256)
        blocks = 256;
    const int wave_major = gp.N % (blocks * kWaves) != 0;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), lds, stream, gp, (int)out_bf16, (int)gelu, wave_major);
    return hipGetLastError();
}

// Chunk counts with a kernel instance: a row of K elements takes the smallest
// one >= ceil(K / 512), so the lanes that re-read a row's last chunk make up
// less than one iteration.
constexpr int kNits[] = {1, 2, 3, 4, 6, 8, 12, 16};

int chunk_iters(int64_t K)
{
    const int nit = (int)((K / 8 + 63) / 64);
    for (int n : kNits)
        if (nit <= n)
            return n;
    return 0;
}

// Largest row count this kernel takes, per chunk count: 5, where the split-K
// MFMA kernel takes over (measured back to back on three rotating weights:
// 4 rows x 9216 x 6144 19.4 us here against 23.0 there, 6 rows 22.4 against
// 21.9, 8 rows x 9216 x 4096 16.2 against 14.5); 2 at 16 chunks, where the row
// buffers and activation batch of more rows would not fit the 256-register
// budget of two waves per SIMD.
constexpr int max_rows(int nit) { return nit <= 12 ? 5 : 2; }

template <int NIT, int B>
hipError_t launch_if_fits(const GemvParams &gp, bool out_bf16, bool gelu, hipStream_t s)
{
    if constexpr (B <= max_rows(NIT))
        return launch_variant<NIT, B>(gp, out_bf16, gelu, s);
    return hipErrorInvalidValue;  // excluded by gemv_supports()
}

template <int NIT>
hipError_t launch_rows(const GemvParams &gp, bool out_bf16, bool gelu, hipStream_t s)
{
    switch (gp.M) {
    case 1: return launch_if_fits<NIT, 1>(gp, out_bf16, gelu, s);
    case 2: return launch_if_fits<NIT, 2>(gp, out_bf16, gelu, s);
    case 3: return launch_if_fits<NIT, 3>(gp, out_bf16, gelu, s);
    case 4: return launch_if_fits<NIT, 4>(gp, out_bf16, gelu, s);
    default: return launch_if_fits<NIT, 5>(gp, out_bf16, gelu, s);
    }
}

}  // namespace

bool gemv_supports(int64_t M, int64_t K)
{
    if (M < 1 || M > kSkinnyMaxM || K > kSkinnyMaxK || M * (K + 8) * 2 > kSkinnyMaxLdsBytes)
        return false;
    return M <= max_rows(chunk_iters(K));
}

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
    switch (chunk_iters(gp.K)) {
    case 1: return launch_rows<1>(gp, pr.out_bf16, pr.gelu, stream);
    case 2: return launch_rows<2>(gp, pr.out_bf16, pr.gelu, stream);
    case 3: return launch_rows<3>(gp, pr.out_bf16, pr.gelu, stream);
    case 4: return launch_rows<4>(gp, pr.out_bf16, pr.gelu, stream);
    case 6: return launch_rows<6>(gp, pr.out_bf16, pr.gelu, stream);
    case 8: return launch_rows<8>(gp, pr.out_bf16, pr.gelu, stream);
    case 12: return launch_rows<12>(gp, pr.out_bf16, pr.gelu, stream);
    case 16: return launch_rows<16>(gp, pr.out_bf16, pr.gelu, stream);
    default: return hipErrorInvalidValue;  // K > kSkinnyMaxK, excluded by gemv_supports()
    }
}

}  // namespace tpl
