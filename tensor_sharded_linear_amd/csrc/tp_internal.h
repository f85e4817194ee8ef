// tp_internal.h -- declarations shared by the kernel files and the C-ABI layer
// of libtp_linear.so.  Everything here is internal; the public contract is
// include/tp_linear.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpl {

// The calling thread's message for the last non-OK status (tp_last_error()).
constexpr int kLastErrorBytes = 512;
char *last_error_buffer();

// Problem description of one linear-layer launch: Y = epilogue(X . W^T).
// X [M, K] bf16 (row stride ldx), W [N, K] bf16 (row stride ldw), Y [M, N]
// (row stride ldy) in bf16 or fp32, optional bias [N] bf16, optional GELU-tanh.
struct LinearProblem {
    const uint16_t *x;
    int64_t ldx;
    const uint16_t *w;
    int64_t ldw;
    const uint16_t *bias;  // nullptr: no bias
    void *y;
    int64_t ldy;
    int64_t M, N, K;
    bool out_bf16;
    bool gelu;
    bool swiglu = false;  // W holds 2N rows [gate; up]; y = silu(x gate^T + b_g) * (x up^T + b_u)
};

// Compute units of the current device (cached per device; 256 without a device).
int cu_count();

// Tiled MFMA GEMM (M > kNarrowMaxM).  Requires K % 64 == 0, N % 16 == 0.
hipError_t launch_gemm(const LinearProblem &p, hipStream_t stream);
// Output tile launch_gemm picks for p on the current device: rows 256, 224, 192, 128 or 64,
// columns 256 or 192 (128 outputs with SwiGLU).
void gemm_tile_shape(const LinearProblem &p, int *rows, int *cols);

// Weight-streaming kernel for skinny M (the adaLN modulation shape): each wave
// holds whole weight rows of up to kSkinnyMaxK elements in registers, and the
// M activation rows are staged in at most kSkinnyMaxLdsBytes of LDS.
// gemv_supports() says whether (M, K) fits; other requests use the split-K or
// the tiled kernel.
constexpr int64_t kSkinnyMaxM = 5;
constexpr int64_t kSkinnyMaxK = 8192;
constexpr int64_t kSkinnyMaxLdsBytes = 64 * 1024;
bool gemv_supports(int64_t M, int64_t K);
hipError_t launch_gemv(const LinearProblem &p, hipStream_t stream);

// Split-K MFMA kernel for few rows (M <= kNarrowMaxM) that the weight-streaming
// kernel does not take: all M rows and 32 output columns (16 with SwiGLU) per
// workgroup, K split across its waves.  Same requirements as the tiled kernel.
constexpr int64_t kNarrowMaxM = 128;
bool narrow_supports(const LinearProblem &p);
void narrow_tile_shape(const LinearProblem &p, int *rows, int *cols);
hipError_t launch_narrow(const LinearProblem &p, hipStream_t stream);

// Bit-exact strided copies: `rows` rows of `row_bytes` bytes each.
struct CopySegment {
    const char *src;
    char *dst;
    int64_t src_ld;  // bytes between source rows
    int64_t dst_ld;  // bytes between destination rows
    int64_t rows;
    int64_t row_bytes;
};
constexpr int kMaxSegmentsPerLaunch = 32;
hipError_t launch_copy_segments(const CopySegment *segs, int nseg, hipStream_t stream);

// SUM combine: out = ((p0 + p1) + ... ) + bias, fp32 adds, fp32 or bf16 out.
constexpr int kMaxParts = 16;
struct SumProblem {
    const float *parts[kMaxParts];
    int num_parts;
    int64_t ld_part;  // elements
    void *out;
    int64_t ld_out;   // elements
    const uint16_t *bias;
    int64_t M, N;
    bool out_bf16;
};
hipError_t launch_combine_sum(const SumProblem &p, hipStream_t stream);

}  // namespace tpl
