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
//
// Stores are ordinary ones.  Strided destinations (CONCAT: column blocks of
// each output row, whose ends fall inside 128-byte lines) need them so the L2
// merges the pieces that neighbouring segments write into the same lines
// (non-temporal stores there measured 13% slower).  Contiguous destinations
// (shard slices, the QKV split) reach 79-83% of HBM peak cold with ordinary
// stores against 69-76% with non-temporal ones (kernel durations of single
// calls after the Infinity Cache is evicted, 226 MB slices); the non-temporal
// form left the GEMMs after the slices in a bench step 0.5% faster, which does
// not make up for it.
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

// Rows of at most kThreads / 2 vectors are short: a row-by-row sweep would
// leave at least half of the workgroup idle.
__host__ __device__ inline bool short_rows(int64_t nv) { return nv > 0 && nv <= kThreads / 2; }

// Rows per block of the short-row sweep: kThreads / gcd(n, kThreads) for n
// vectors per row (kThreads is a power of two), so that a block is a whole
// number of passes of the workgroup.
__host__ __device__ inline int short_row_block(int n)
{
    int tz = 0;
    while (tz < 8 && ((n >> tz) & 1) == 0)
        ++tz;
    return kThreads >> tz;
}

template <int VEC>
__global__ __launch_bounds__(kThreads) void copy_segments_kernel(CopyArgs a)
{
    typedef typename VecType<VEC>::T V;
    const CopySegment s = a.seg[blockIdx.y];
    const int64_t nv = s.row_bytes / VEC;
    if (short_rows(nv)) {
        // Short rows (the tp 8 pieces of a packed CONCAT, 1.5 KiB): the
        // workgroup takes blocks of rb rows and sweeps each block's rb * nv
        // vectors as one range.
        const int n = (int)nv;
        const int rb = short_row_block(n);
        for (int64_t r0 = (int64_t)blockIdx.x * rb; r0 < s.rows; r0 += (int64_t)gridDim.x * rb) {
            const int rows = (int)min((int64_t)rb, s.rows - r0);
            for (int f = threadIdx.x; f < rows * n; f += kThreads) {
                const int q = f / n;
                const int v = f - q * n;
                const V t = __builtin_nontemporal_load(reinterpret_cast<const V *>(s.src + (r0 + q) * s.src_ld) + v);
                reinterpret_cast<V *>(s.dst + (r0 + q) * s.dst_ld)[v] = t;
            }
        }
        return;
    }
    for (int64_t r = blockIdx.x; r < s.rows; r += gridDim.x) {
        const V *src = reinterpret_cast<const V *>(s.src + r * s.src_ld);
        V *dst = reinterpret_cast<V *>(s.dst + r * s.dst_ld);
        for (int64_t v = threadIdx.x; v < nv; v += kThreads) {
            dst[v] = __builtin_nontemporal_load(src + v);
        }
    }
}

}  // namespace

hipError_t launch_copy_segments(const CopySegment *segs, int nseg, hipStream_t stream)
{
    for (int base = 0; base < nseg; base += kMaxSegmentsPerLaunch) {
        const int cnt = nseg - base < kMaxSegmentsPerLaunch ? nseg - base : kMaxSegmentsPerLaunch;
        CopyArgs a;
        uint64_t bits = 0;
        for (int i = 0; i < cnt; ++i) {
            const CopySegment &s = segs[base + i];
            a.seg[i] = s;
            bits |= (uint64_t)(uintptr_t)s.src | (uint64_t)(uintptr_t)s.dst | (uint64_t)s.src_ld |
                    (uint64_t)s.dst_ld | (uint64_t)s.row_bytes;
        }
        const int vec = (bits & 15) == 0 ? 16 : (bits & 7) == 0 ? 8 : (bits & 3) == 0 ? 4 : 2;
        // Workgroups per segment: one per row, or one per block of short rows;
        // the largest count over the segments, capped so that the grid still
        // covers the chip several times.
        int64_t max_groups = 0;
        for (int i = 0; i < cnt; ++i) {
            const CopySegment &s = segs[base + i];
            const int64_t nv = s.row_bytes / vec;
            int64_t groups = nv > 0 ? s.rows : 0;
            if (short_rows(nv)) {
                const int rb = short_row_block((int)nv);
                groups = (s.rows + rb - 1) / rb;
            }
            if (groups > max_groups)
                max_groups = groups;
        }
        if (max_groups == 0)
            continue;
        int64_t gx = max_groups < 4096 ? max_groups : 4096;
        const dim3 grid((unsigned)gx, (unsigned)cnt);
        const dim3 block(kThreads);
        switch (vec) {
        case 16: hipLaunchKernelGGL((copy_segments_kernel<16>), grid, block, 0, stream, a); break;
        case 8: hipLaunchKernelGGL((copy_segments_kernel<8>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((copy_segments_kernel<4>), grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL((copy_segments_kernel<2>), grid, block, 0, stream, a); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace tpl
