// index_copy.hip -- bit-exact strided copies for the index work of the path.
//
// Every index operation of the tensor-parallel path is a set of 2-D
// rectangles copied verbatim (Diffusers "Tensor parallelism" page):
//   * colwise shard slice ("Colwise and rowwise"): one block of whole rows;
//   * rowwise shard slice: one column block of every row;
//   * packed / head-aligned fused-QKV slice ("Fused projections"): one row
//     block per packed block;
//   * concat of colwise output slices (the one-device AllGather): one column
//     block per (rank, packed block).
// The host turns each request into a list of segments; this kernel moves
// them.  HBM-bound: each workgroup owns rows of one segment and its threads
// sweep a row with the widest vector (16, 8, 4 or 2 bytes) that every address,
// stride and row length of the launch allows.
#include "tp_internal.h"

namespace tpl {
namespace {

constexpr int kThreads = 256;

struct CopyArgs {
    CopySegment seg[kMaxSegmentsPerLaunch];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int VEC> struct VecType;
template <> struct VecType<16> { typedef u32x4 T; };
template <> struct VecType<8> { typedef u32x2 T; };
template <> struct VecType<4> { typedef uint32_t T; };
template <> struct VecType<2> { typedef uint16_t T; };

template <int VEC>
__global__ __launch_bounds__(kThreads) void copy_segments_kernel(CopyArgs a)
{
    typedef typename VecType<VEC>::T V;
    const CopySegment s = a.seg[blockIdx.y];
    const int64_t nv = s.row_bytes / VEC;
    for (int64_t r = blockIdx.x; r < s.rows; r += gridDim.x) {
        const V *src = reinterpret_cast<const V *>(s.src + r * s.src_ld);
        V *dst = reinterpret_cast<V *>(s.dst + r * s.dst_ld);
        for (int64_t v = threadIdx.x; v < nv; v += kThreads)
            dst[v] = __builtin_nontemporal_load(src + v);
    }
}

}  // namespace

hipError_t launch_copy_segments(const CopySegment *segs, int nseg, hipStream_t stream)
{
    for (int base = 0; base < nseg; base += kMaxSegmentsPerLaunch) {
        const int cnt = nseg - base < kMaxSegmentsPerLaunch ? nseg - base : kMaxSegmentsPerLaunch;
        CopyArgs a;
        uint64_t bits = 0;
        int64_t max_rows = 0;
        for (int i = 0; i < cnt; ++i) {
            const CopySegment &s = segs[base + i];
            a.seg[i] = s;
            bits |= (uint64_t)(uintptr_t)s.src | (uint64_t)(uintptr_t)s.dst | (uint64_t)s.src_ld |
                    (uint64_t)s.dst_ld | (uint64_t)s.row_bytes;
            if (s.rows > max_rows)
                max_rows = s.rows;
        }
        if (max_rows == 0)
            continue;
        // Rows per segment: enough workgroups to cover the chip several times.
        int64_t gx = max_rows < 4096 ? max_rows : 4096;
        const dim3 grid((unsigned)gx, (unsigned)cnt);
        const dim3 block(kThreads);
        if ((bits & 15) == 0)
            hipLaunchKernelGGL(copy_segments_kernel<16>, grid, block, 0, stream, a);
        else if ((bits & 7) == 0)
            hipLaunchKernelGGL(copy_segments_kernel<8>, grid, block, 0, stream, a);
        else if ((bits & 3) == 0)
            hipLaunchKernelGGL(copy_segments_kernel<4>, grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL(copy_segments_kernel<2>, grid, block, 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace tpl
