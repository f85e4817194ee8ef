// combine.hip -- the layer-boundary SUM of rowwise partials on one device.
//
// Diffusers "Tensor parallelism" page: rowwise ranks each produce a partial
// sum and one AllReduce at the block boundary rebuilds the output (opening
// definition; "Colwise and rowwise", pairing rule).  With every rank's partial
// buffer on one device the reduction is this kernel:
//   out = ((p_0 + p_1) + ... + p_{P-1}) + bias
// in fp32, in ascending part order (a fixed order makes the result unique and
// reproducible), the bias added once, one rounding to the output dtype.
// HBM-bound: each thread owns four consecutive columns of R rows and issues
// all R * P 16-byte loads before summing.  The kernel is templated on a bound
// PMAX >= P so that its registers match P, and takes R = 2 rows for P <= 4 to
// keep enough loads in flight.  The output is stored non-temporally (whole
// 16-byte vectors of consecutive columns): left dirty in the caches, it was
// written back during the kernels that followed, and those ran slower (the
// GEMMs by 1%, the CONCAT by 4%).
#include "tp_internal.h"

namespace tpl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

template <int PMAX, bool OUT_BF16, bool HAS_BIAS>
__global__ __launch_bounds__(kThreads) void combine_sum_kernel(SumProblem a)
{
    constexpr int R = PMAX <= 4 ? 2 : 1;  // rows per thread
    const int64_t ng = (a.N + 3) >> 2;    // 4-column groups per row
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (g >= ng)
        return;
    const int64_t c = g * 4;
    for (int64_t r0 = (int64_t)blockIdx.y * R; r0 < a.M; r0 += (int64_t)gridDim.y * R) {
        if (c + 4 <= a.N) {
            f32x4 v[R][PMAX];
#pragma unroll
            for (int rr = 0; rr < R; ++rr)
#pragma unroll
                for (int p = 0; p < PMAX; ++p)
                    if (r0 + rr < a.M && p < a.num_parts)
                        v[rr][p] = __builtin_nontemporal_load(
                            reinterpret_cast<const f32x4 *>(a.parts[p] + (r0 + rr) * a.ld_part + c));
#pragma unroll
            for (int rr = 0; rr < R; ++rr) {
                const int64_t row = r0 + rr;
                if (row >= a.M)
                    break;
                f32x4 s = v[rr][0];
#pragma unroll
                for (int p = 1; p < PMAX; ++p)
                    if (p < a.num_parts)
                        s = s + v[rr][p];
                if (HAS_BIAS) {
                    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(a.bias + c);
                    s = s + f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
                }
                const int64_t o = row * a.ld_out + c;
                if (OUT_BF16) {
                    const bf16x4 r = bf16x4{(__bf16)s[0], (__bf16)s[1], (__bf16)s[2], (__bf16)s[3]};
                    __builtin_nontemporal_store(r, reinterpret_cast<bf16x4 *>(reinterpret_cast<uint16_t *>(a.out) + o));
                } else {
                    __builtin_nontemporal_store(s, reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.out) + o));
                }
            }
        } else {
            for (int rr = 0; rr < R && r0 + rr < a.M; ++rr) {
                const int64_t row = r0 + rr;
                for (int64_t cc = c; cc < a.N; ++cc) {
                    float s = a.parts[0][row * a.ld_part + cc];
                    for (int p = 1; p < a.num_parts; ++p)
                        s = s + a.parts[p][row * a.ld_part + cc];
                    if (HAS_BIAS)
                        s = s + (float)(*reinterpret_cast<const __bf16 *>(a.bias + cc));
                    const int64_t o = row * a.ld_out + cc;
                    if (OUT_BF16)
                        *reinterpret_cast<__bf16 *>(reinterpret_cast<uint16_t *>(a.out) + o) = (__bf16)s;
                    else
                        reinterpret_cast<float *>(a.out)[o] = s;
                }
            }
        }
    }
}

template <int PMAX>
void launch_pmax(const SumProblem &p, dim3 grid, hipStream_t stream)
{
    constexpr int R = PMAX <= 4 ? 2 : 1;
    const int64_t gy = (p.M + R - 1) / R;
    grid.y = (unsigned)(gy < 65535 ? gy : 65535);
    const dim3 block(kThreads);
    const bool bias = p.bias != nullptr;
    if (p.out_bf16) {
        if (bias)
            hipLaunchKernelGGL((combine_sum_kernel<PMAX, true, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((combine_sum_kernel<PMAX, true, false>), grid, block, 0, stream, p);
    } else {
        if (bias)
            hipLaunchKernelGGL((combine_sum_kernel<PMAX, false, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((combine_sum_kernel<PMAX, false, false>), grid, block, 0, stream, p);
    }
}

}  // namespace

hipError_t launch_combine_sum(const SumProblem &p, hipStream_t stream)
{
    const int64_t ng = (p.N + 3) / 4;
    const dim3 grid((unsigned)((ng + kThreads - 1) / kThreads), 1);
    if (p.num_parts <= 2)
        launch_pmax<2>(p, grid, stream);
    else if (p.num_parts <= 4)
        launch_pmax<4>(p, grid, stream);
    else if (p.num_parts <= 8)
        launch_pmax<8>(p, grid, stream);
    else
        launch_pmax<16>(p, grid, stream);
    return hipGetLastError();
}

}  // namespace tpl
