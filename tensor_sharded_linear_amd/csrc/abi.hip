// abi.hip -- the extern "C" entry points of libtp_linear.so (include/tp_linear.h).
//
// Each entry point validates every argument before touching the device, turns
// the request into kernel launches (tiled MFMA GEMM, split-K MFMA kernel for
// up to 128 rows, skinny weight-streaming kernel, bit-exact segment copies, SUM
// combine) on the caller's stream, and
// reports errors through a status code plus a thread-local message.  Nothing
// is allocated and no state is kept between calls.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "tp_internal.h"
#include "tp_linear.h"

namespace {

thread_local char g_msg[tpl::kLastErrorBytes] = "";

__attribute__((format(printf, 2, 3))) tp_status fail(tp_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
    return s;
}

tp_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess)
        return TP_OK;
    return fail(TP_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int elem_size(tp_dtype d) { return d == TP_BF16 ? 2 : (d == TP_F32 ? 4 : 0); }

constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr int64_t kMaxOperandBytes = (int64_t)1 << 31;
// Row strides above 2^31 elements are rejected, so that no offset product overflows.
constexpr int64_t kMaxLd = (int64_t)1 << 31;
// Output tiles of one tiled-GEMM launch (each a 512-thread workgroup): the
// launch's thread count must stay below 2^32.
constexpr int64_t kMaxTiles = (int64_t)1 << 22;
constexpr int kMaxBlocks = 16;

// Common checks of the two compute entry points.  Returns TP_OK when the
// call should proceed (M > 0), or the status to return.
tp_status check_linear(const char *fn, const void *x, int64_t ldx, const void *w, int64_t ldw,
                       const void *bias, const void *y, int64_t ldy, int y_es, int64_t M,
                       int64_t N, int64_t K, bool *noop)
{
    *noop = false;
    if (M < 0 || N <= 0 || K <= 0)
        return fail(TP_ERR_INVALID_ARG, "%s: need M >= 0, N > 0, K > 0 (got M=%lld N=%lld K=%lld)", fn,
                    (long long)M, (long long)N, (long long)K);
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return fail(TP_ERR_UNSUPPORTED, "%s: dimensions above 2^30 are not supported", fn);
    if (ldx > kMaxLd || ldw > kMaxLd || ldy > kMaxLd)
        return fail(TP_ERR_UNSUPPORTED, "%s: row strides above 2^31 elements are not supported", fn);
    if (K % 64 != 0)
        return fail(TP_ERR_UNSUPPORTED, "%s: K=%lld must be a multiple of 64", fn, (long long)K);
    if (N % 16 != 0)
        return fail(TP_ERR_UNSUPPORTED, "%s: N=%lld must be a multiple of 16", fn, (long long)N);
    if (ldx < K || ldx % 8 != 0)
        return fail(TP_ERR_INVALID_ARG, "%s: ldx=%lld must be >= K=%lld and a multiple of 8", fn,
                    (long long)ldx, (long long)K);
    if (ldw < K || ldw % 8 != 0)
        return fail(TP_ERR_INVALID_ARG, "%s: ldw=%lld must be >= K=%lld and a multiple of 8", fn,
                    (long long)ldw, (long long)K);
    if (ldy < N || (ldy * y_es) % 16 != 0)
        return fail(TP_ERR_INVALID_ARG, "%s: ldy=%lld must be >= N=%lld and a multiple of 16 bytes", fn,
                    (long long)ldy, (long long)N);
    // The kernels address each operand by 32-bit byte offsets from its base.
    if (((N - 1) * ldw + K) * 2 >= kMaxOperandBytes || (M > 0 && ((M - 1) * ldx + K) * 2 >= kMaxOperandBytes))
        return fail(TP_ERR_UNSUPPORTED, "%s: an operand spans 2 GiB or more", fn);
    if ((M + 191) / 192 * ((N + 255) / 256) > kMaxTiles)
        return fail(TP_ERR_UNSUPPORTED, "%s: an output of %lld x %lld needs more than 2^22 tiles", fn,
                    (long long)M, (long long)N);
    if (!w || !aligned(w, 16))
        return fail(TP_ERR_INVALID_ARG, "%s: weight pointer is null or not 16-byte aligned", fn);
    if (bias && !aligned(bias, 8))
        return fail(TP_ERR_INVALID_ARG, "%s: bias pointer is not 8-byte aligned", fn);
    if (M == 0) {
        *noop = true;
        return TP_OK;
    }
    if (!x || !aligned(x, 16))
        return fail(TP_ERR_INVALID_ARG, "%s: activation pointer is null or not 16-byte aligned", fn);
    if (!y || !aligned(y, 16))
        return fail(TP_ERR_INVALID_ARG, "%s: output pointer is null or not 16-byte aligned", fn);
    return TP_OK;
}

tp_status run_linear(const char *fn, const tpl::LinearProblem &p, hipStream_t stream)
{
    // The weight-streaming kernel has no gated epilogue: SwiGLU with few rows takes the
    // split-K kernel.
    hipError_t e;
    if (!p.swiglu && tpl::gemv_supports(p.M, p.K))
        e = tpl::launch_gemv(p, stream);
    else if (tpl::narrow_supports(p))
        e = tpl::launch_narrow(p, stream);
    else
        e = tpl::launch_gemm(p, stream);
    return hip_status(e, fn);
}

// Checks a packed-block description against a dimension and the tp degree.
tp_status check_blocks(const char *fn, const int64_t *blocks, int nb, int64_t dim, int P,
                       int64_t *unit_out)
{
    if (nb < 1 || nb > kMaxBlocks)
        return fail(TP_ERR_INVALID_ARG, "%s: num_blocks=%d must be in [1, %d]", fn, nb, kMaxBlocks);
    int64_t sum = 0;
    for (int i = 0; i < nb; ++i) {
        if (blocks[i] < 1 || blocks[i] > kMaxDim)
            return fail(TP_ERR_INVALID_ARG, "%s: blocks[%d]=%lld must be a positive integer", fn, i,
                        (long long)blocks[i]);
        sum += blocks[i];
    }
    if (dim % sum != 0)
        return fail(TP_ERR_NOT_DIVISIBLE, "%s: sum(blocks)=%lld does not divide the packed dim %lld", fn,
                    (long long)sum, (long long)dim);
    const int64_t unit = dim / sum;
    for (int i = 0; i < nb; ++i)
        if ((blocks[i] * unit) % P != 0)
            return fail(TP_ERR_NOT_DIVISIBLE,
                        "%s: packed block %d (%lld of %lld) is not divisible by tp_degree=%d", fn, i,
                        (long long)(blocks[i] * unit), (long long)dim, P);
    *unit_out = unit;
    return TP_OK;
}

}  // namespace

char *tpl::last_error_buffer() { return g_msg; }

extern "C" {

const char *tp_last_error(void) { return g_msg; }

tp_status tp_linear_colwise(const void *x, int64_t ldx, const void *w_shard, int64_t ldw,
                            const void *bias, void *y, int64_t ldy, tp_dtype y_dtype, tp_act act,
                            int64_t M, int64_t n_shard, int64_t K, hipStream_t stream)
{
    const char *fn = "tp_linear_colwise";
    g_msg[0] = 0;
    if (y_dtype != TP_BF16 && y_dtype != TP_F32)
        return fail(TP_ERR_INVALID_ARG, "%s: y_dtype must be TP_BF16 or TP_F32", fn);
    if (act != TP_ACT_NONE && act != TP_ACT_GELU_TANH && act != TP_ACT_SWIGLU)
        return fail(TP_ERR_INVALID_ARG, "%s: act must be TP_ACT_NONE, TP_ACT_GELU_TANH or TP_ACT_SWIGLU", fn);
    bool noop;
    tp_status s = check_linear(fn, x, ldx, w_shard, ldw, bias, y, ldy, elem_size(y_dtype), M, n_shard,
                               K, &noop);
    if (s != TP_OK)
        return s;
    // SwiGLU reads 2 n_shard weight rows (and bias entries): [gate; up].
    if (act == TP_ACT_SWIGLU && ((2 * n_shard - 1) * ldw + K) * 2 >= kMaxOperandBytes)
        return fail(TP_ERR_UNSUPPORTED, "%s: an operand spans 2 GiB or more", fn);
    if (noop)
        return s;
    tpl::LinearProblem p;
    p.x = (const uint16_t *)x;
    p.ldx = ldx;
    p.w = (const uint16_t *)w_shard;
    p.ldw = ldw;
    p.bias = (const uint16_t *)bias;
    p.y = y;
    p.ldy = ldy;
    p.M = M;
    p.N = n_shard;
    p.K = K;
    p.out_bf16 = y_dtype == TP_BF16;
    p.gelu = act == TP_ACT_GELU_TANH;
    p.swiglu = act == TP_ACT_SWIGLU;
    return run_linear(fn, p, stream);
}

tp_status tp_linear_tile_shape(int64_t M, int64_t N, int64_t K, tp_act act, int64_t *tile_rows,
                               int64_t *tile_cols)
{
    const char *fn = "tp_linear_tile_shape";
    g_msg[0] = 0;
    if (!tile_rows || !tile_cols)
        return fail(TP_ERR_INVALID_ARG, "%s: tile_rows and tile_cols must be non-null", fn);
    if (act != TP_ACT_NONE && act != TP_ACT_GELU_TANH && act != TP_ACT_SWIGLU)
        return fail(TP_ERR_INVALID_ARG, "%s: act must be TP_ACT_NONE, TP_ACT_GELU_TANH or TP_ACT_SWIGLU", fn);
    if (M < 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return fail(TP_ERR_INVALID_ARG, "%s: need 0 <= M, 0 < N, 0 < K, all at most 2^30", fn);
    tpl::LinearProblem p{};
    p.M = M;
    p.N = N;
    p.K = K;
    p.gelu = act == TP_ACT_GELU_TANH;
    p.swiglu = act == TP_ACT_SWIGLU;
    if (!p.swiglu && tpl::gemv_supports(M, K)) {
        *tile_rows = *tile_cols = 0;
        return TP_OK;
    }
    int rows = 0, cols = 0;
    if (tpl::narrow_supports(p))
        tpl::narrow_tile_shape(p, &rows, &cols);
    else
        tpl::gemm_tile_shape(p, &rows, &cols);
    *tile_rows = rows;
    *tile_cols = cols;
    return TP_OK;
}

tp_status tp_linear_rowwise(const void *x_shard, int64_t ldx, const void *w_shard, int64_t ldw,
                            float *partial, int64_t ldp, int64_t M, int64_t N, int64_t k_shard,
                            hipStream_t stream)
{
    const char *fn = "tp_linear_rowwise";
    g_msg[0] = 0;
    bool noop;
    tp_status s = check_linear(fn, x_shard, ldx, w_shard, ldw, nullptr, partial, ldp, 4, M, N, k_shard,
                               &noop);
    if (s != TP_OK || noop)
        return s;
    tpl::LinearProblem p;
    p.x = (const uint16_t *)x_shard;
    p.ldx = ldx;
    p.w = (const uint16_t *)w_shard;
    p.ldw = ldw;
    p.bias = nullptr;
    p.y = partial;
    p.ldy = ldp;
    p.M = M;
    p.N = N;
    p.K = k_shard;
    p.out_bf16 = false;
    p.gelu = false;
    return run_linear(fn, p, stream);
}

tp_status tp_linear_rowwise_split_input(const void *x_full, int64_t ldx, int64_t k_full, const void *w_shard,
                                        int64_t ldw, float *partial, int64_t ldp, int64_t M, int64_t N,
                                        int tp_degree, int rank, hipStream_t stream)
{
    const char *fn = "tp_linear_rowwise_split_input";
    g_msg[0] = 0;
    if (tp_degree < 1)
        return fail(TP_ERR_INVALID_ARG, "%s: tp_degree=%d must be >= 1", fn, tp_degree);
    if (rank < 0 || rank >= tp_degree)
        return fail(TP_ERR_INVALID_ARG, "%s: rank=%d outside [0, %d)", fn, rank, tp_degree);
    if (k_full <= 0 || k_full > kMaxDim)
        return fail(TP_ERR_INVALID_ARG, "%s: k_full=%lld must be in [1, 2^30]", fn, (long long)k_full);
    if (k_full % tp_degree != 0)
        return fail(TP_ERR_NOT_DIVISIBLE, "%s: tp_degree=%d does not divide k_full=%lld", fn, tp_degree,
                    (long long)k_full);
    const int64_t k_shard = k_full / tp_degree;
    if (ldx < k_full)
        return fail(TP_ERR_INVALID_ARG, "%s: ldx=%lld must be >= k_full=%lld", fn, (long long)ldx,
                    (long long)k_full);
    // The rank's slice of the replicated input: a column offset into x_full.
    const void *x_r = x_full ? (const void *)((const uint16_t *)x_full + rank * k_shard) : nullptr;
    bool noop;
    tp_status s = check_linear(fn, x_r, ldx, w_shard, ldw, nullptr, partial, ldp, 4, M, N, k_shard, &noop);
    if (s != TP_OK || noop)
        return s;
    tpl::LinearProblem p;
    p.x = (const uint16_t *)x_r;
    p.ldx = ldx;
    p.w = (const uint16_t *)w_shard;
    p.ldw = ldw;
    p.bias = nullptr;
    p.y = partial;
    p.ldy = ldp;
    p.M = M;
    p.N = N;
    p.K = k_shard;
    p.out_bf16 = false;
    p.gelu = false;
    return run_linear(fn, p, stream);
}

tp_status tp_fused_qkv_split(const void *w_qkv, const void *b_qkv, void *w_shard, void *b_shard,
                             int64_t num_heads, int64_t head_dim, int64_t K, tp_dtype dtype,
                             int tp_degree, int rank, hipStream_t stream)
{
    const char *fn = "tp_fused_qkv_split";
    g_msg[0] = 0;
    const int es = elem_size(dtype);
    if (!es)
        return fail(TP_ERR_INVALID_ARG, "%s: dtype must be TP_BF16 or TP_F32", fn);
    if (tp_degree < 1)
        return fail(TP_ERR_INVALID_ARG, "%s: tp_degree=%d must be >= 1", fn, tp_degree);
    if (rank < 0 || rank >= tp_degree)
        return fail(TP_ERR_INVALID_ARG, "%s: rank=%d outside [0, %d)", fn, rank, tp_degree);
    if (num_heads < 1 || head_dim < 1 || K < 1 || num_heads > kMaxDim || head_dim > kMaxDim || K > kMaxDim)
        return fail(TP_ERR_INVALID_ARG, "%s: num_heads, head_dim and K must be in [1, 2^30]", fn);
    if (3 * num_heads * head_dim > kMaxDim)
        return fail(TP_ERR_UNSUPPORTED, "%s: a fused weight of more than 2^30 rows is not supported", fn);
    if (num_heads % tp_degree != 0)
        return fail(TP_ERR_NOT_DIVISIBLE, "%s: tp_degree=%d does not divide num_heads=%lld", fn, tp_degree,
                    (long long)num_heads);
    if (!w_qkv || !w_shard || !aligned(w_qkv, 4) || !aligned(w_shard, 4))
        return fail(TP_ERR_INVALID_ARG, "%s: weight pointers must be non-null and 4-byte aligned", fn);
    if ((b_qkv == nullptr) != (b_shard == nullptr))
        return fail(TP_ERR_INVALID_ARG, "%s: pass both bias pointers or neither", fn);
    if (b_qkv && (!aligned(b_qkv, 4) || !aligned(b_shard, 4)))
        return fail(TP_ERR_INVALID_ARG, "%s: bias pointers must be 4-byte aligned", fn);

    const int64_t rows_per = num_heads / tp_degree * head_dim;  // rows of one of Q/K/V on this rank
    const int64_t full_per = num_heads * head_dim;
    tpl::CopySegment segs[6];
    int n = 0;
    for (int which = 0; which < 3; ++which) {
        const int64_t src_row = which * full_per + rank * rows_per;
        const int64_t dst_row = which * rows_per;
        segs[n++] = tpl::CopySegment{(const char *)w_qkv + src_row * K * es, (char *)w_shard + dst_row * K * es,
                                     K * es, K * es, rows_per, K * es};
        if (b_qkv)
            segs[n++] = tpl::CopySegment{(const char *)b_qkv + src_row * es, (char *)b_shard + dst_row * es,
                                         0, 0, 1, rows_per * es};
    }
    return hip_status(tpl::launch_copy_segments(segs, n, stream), fn);
}

tp_status tp_partial_combine(const void *const *parts, int num_parts, int64_t ld_part, void *out,
                             int64_t ld_out, tp_dtype in_dtype, tp_dtype out_dtype, tp_combine mode,
                             const void *bias, const int64_t *blocks, int num_blocks, int64_t M,
                             int64_t n_part, hipStream_t stream)
{
    const char *fn = "tp_partial_combine";
    g_msg[0] = 0;
    if (num_parts < 1 || num_parts > tpl::kMaxParts)
        return fail(TP_ERR_INVALID_ARG, "%s: num_parts=%d must be in [1, %d]", fn, num_parts, tpl::kMaxParts);
    if (!parts)
        return fail(TP_ERR_INVALID_ARG, "%s: parts (host array) is null", fn);
    if (M < 0 || n_part < 1 || M > kMaxDim || n_part > kMaxDim)
        return fail(TP_ERR_INVALID_ARG, "%s: need 0 <= M <= 2^30 and 1 <= n_part <= 2^30", fn);
    if (ld_part > kMaxLd || ld_out > kMaxLd)
        return fail(TP_ERR_UNSUPPORTED, "%s: row strides above 2^31 elements are not supported", fn);
    if (mode == TP_COMBINE_SUM) {
        if (in_dtype != TP_F32)
            return fail(TP_ERR_INVALID_ARG, "%s: SUM combines fp32 partials (in_dtype must be TP_F32)", fn);
        if (out_dtype != TP_F32 && out_dtype != TP_BF16)
            return fail(TP_ERR_INVALID_ARG, "%s: out_dtype must be TP_F32 or TP_BF16", fn);
        if (blocks || num_blocks)
            return fail(TP_ERR_INVALID_ARG, "%s: SUM takes no blocks", fn);
        if (ld_part < n_part || ld_part % 4 != 0)
            return fail(TP_ERR_INVALID_ARG, "%s: ld_part=%lld must be >= n_part and a multiple of 4", fn,
                        (long long)ld_part);
        const int oes = elem_size(out_dtype);
        if (ld_out < n_part || (ld_out * oes) % 16 != 0)
            return fail(TP_ERR_INVALID_ARG, "%s: ld_out=%lld must be >= n_part and a multiple of 16 bytes", fn,
                        (long long)ld_out);
        if (bias && !aligned(bias, 8))
            return fail(TP_ERR_INVALID_ARG, "%s: bias must be 8-byte aligned", fn);
        if (M == 0)
            return TP_OK;
        if (!out || !aligned(out, 16))
            return fail(TP_ERR_INVALID_ARG, "%s: out is null or not 16-byte aligned", fn);
        tpl::SumProblem p;
        memset(&p, 0, sizeof p);
        for (int i = 0; i < num_parts; ++i) {
            if (!parts[i] || !aligned(parts[i], 16))
                return fail(TP_ERR_INVALID_ARG, "%s: parts[%d] is null or not 16-byte aligned", fn, i);
            if (parts[i] == out && (i != 0 || out_dtype != TP_F32 || ld_out != ld_part))
                return fail(TP_ERR_INVALID_ARG,
                            "%s: only parts[0] may alias out, with fp32 output and ld_out == ld_part", fn);
            p.parts[i] = (const float *)parts[i];
        }
        p.num_parts = num_parts;
        p.ld_part = ld_part;
        p.out = out;
        p.ld_out = ld_out;
        p.bias = (const uint16_t *)bias;
        p.M = M;
        p.N = n_part;
        p.out_bf16 = out_dtype == TP_BF16;
        return hip_status(tpl::launch_combine_sum(p, stream), fn);
    }
    if (mode != TP_COMBINE_CONCAT)
        return fail(TP_ERR_INVALID_ARG, "%s: mode must be TP_COMBINE_SUM or TP_COMBINE_CONCAT", fn);
    const int es = elem_size(in_dtype);
    if (!es || in_dtype != out_dtype)
        return fail(TP_ERR_INVALID_ARG, "%s: CONCAT needs in_dtype == out_dtype in {TP_BF16, TP_F32}", fn);
    if (bias)
        return fail(TP_ERR_INVALID_ARG, "%s: CONCAT takes no bias", fn);
    const int64_t n_out = n_part * num_parts;
    if (ld_part < n_part || ld_out < n_out)
        return fail(TP_ERR_INVALID_ARG, "%s: ld_part must be >= n_part and ld_out >= num_parts*n_part", fn);
    int64_t one = 1;
    const int64_t *bl = blocks ? blocks : &one;
    const int nb = blocks ? num_blocks : 1;
    if (!blocks && num_blocks)
        return fail(TP_ERR_INVALID_ARG, "%s: num_blocks given without blocks", fn);
    int64_t unit = 0;
    tp_status s = check_blocks(fn, bl, nb, n_out, num_parts, &unit);
    if (s != TP_OK)
        return s;
    if (M == 0)
        return TP_OK;
    if (!out || !aligned(out, (uintptr_t)es))
        return fail(TP_ERR_INVALID_ARG, "%s: out is null or misaligned", fn);
    for (int i = 0; i < num_parts; ++i)
        if (!parts[i] || !aligned(parts[i], (uintptr_t)es))
            return fail(TP_ERR_INVALID_ARG, "%s: parts[%d] is null or misaligned", fn, i);
    tpl::CopySegment segs[tpl::kMaxParts * kMaxBlocks];
    int n = 0;
    for (int p = 0; p < num_parts; ++p) {
        int64_t loc = 0, off = 0;
        for (int i = 0; i < nb; ++i) {
            const int64_t size = bl[i] * unit;
            const int64_t piece = size / num_parts;
            segs[n++] = tpl::CopySegment{(const char *)parts[p] + loc * es,
                                         (char *)out + (off + p * piece) * es, ld_part * es, ld_out * es, M,
                                         piece * es};
            loc += piece;
            off += size;
        }
    }
    return hip_status(tpl::launch_copy_segments(segs, n, stream), fn);
}

tp_status tp_plan_shard_slice(const void *w_full, const void *b_full, void *w_shard, void *b_shard,
                              int64_t out_features, int64_t in_features, tp_dtype dtype, tp_style style,
                              const int64_t *blocks, int num_blocks, int tp_degree, int rank,
                              int64_t *shard_rows, int64_t *shard_cols, hipStream_t stream)
{
    const char *fn = "tp_plan_shard_slice";
    g_msg[0] = 0;
    const int es = elem_size(dtype);
    if (!es)
        return fail(TP_ERR_INVALID_ARG, "%s: dtype must be TP_BF16 or TP_F32", fn);
    if (style != TP_COLWISE && style != TP_ROWWISE && style != TP_ROWWISE_SPLIT_INPUT)
        return fail(TP_ERR_INVALID_ARG, "%s: style must be TP_COLWISE, TP_ROWWISE or TP_ROWWISE_SPLIT_INPUT", fn);
    if (tp_degree < 1)
        return fail(TP_ERR_INVALID_ARG, "%s: tp_degree=%d must be >= 1", fn, tp_degree);
    if (rank < 0 || rank >= tp_degree)
        return fail(TP_ERR_INVALID_ARG, "%s: rank=%d outside [0, %d)", fn, rank, tp_degree);
    if (out_features < 1 || in_features < 1 || out_features > kMaxDim || in_features > kMaxDim)
        return fail(TP_ERR_INVALID_ARG, "%s: out_features and in_features must be in [1, 2^30]", fn);
    if (!blocks && num_blocks)
        return fail(TP_ERR_INVALID_ARG, "%s: num_blocks given without blocks", fn);
    const int64_t dim = style == TP_COLWISE ? out_features : in_features;
    int64_t one = 1;
    const int64_t *bl = blocks ? blocks : &one;
    const int nb = blocks ? num_blocks : 1;
    int64_t unit = 0;
    tp_status s = check_blocks(fn, bl, nb, dim, tp_degree, &unit);
    if (s != TP_OK) {
        if (!blocks && s == TP_ERR_NOT_DIVISIBLE)
            return fail(TP_ERR_NOT_DIVISIBLE, "%s: tp_degree=%d does not divide the sharded dim %lld", fn,
                        tp_degree, (long long)dim);
        return s;
    }
    const int64_t rows = style == TP_COLWISE ? out_features / tp_degree : out_features;
    const int64_t cols = style == TP_COLWISE ? in_features : in_features / tp_degree;
    if (shard_rows)
        *shard_rows = rows;
    if (shard_cols)
        *shard_cols = cols;
    if (!w_shard)
        return TP_OK;  // shape query
    if (!w_full || !aligned(w_full, (uintptr_t)es) || !aligned(w_shard, (uintptr_t)es))
        return fail(TP_ERR_INVALID_ARG, "%s: weight pointers must be non-null and element aligned", fn);
    if (style != TP_COLWISE && (b_full || b_shard))
        return fail(TP_ERR_INVALID_ARG,
                    "%s: a rowwise shard owns no bias slice (the bias is added once after the sum)", fn);
    if ((b_full == nullptr) != (b_shard == nullptr))
        return fail(TP_ERR_INVALID_ARG, "%s: pass both bias pointers or neither", fn);
    if (b_full && (!aligned(b_full, (uintptr_t)es) || !aligned(b_shard, (uintptr_t)es)))
        return fail(TP_ERR_INVALID_ARG, "%s: bias pointers must be element aligned", fn);

    tpl::CopySegment segs[2 * kMaxBlocks];
    int n = 0;
    int64_t loc = 0, off = 0;
    for (int i = 0; i < nb; ++i) {
        const int64_t size = bl[i] * unit;
        const int64_t piece = size / tp_degree;
        const int64_t src = off + rank * piece;  // first row (colwise) / column (rowwise) taken
        if (style == TP_COLWISE) {
            segs[n++] = tpl::CopySegment{(const char *)w_full + src * in_features * es,
                                         (char *)w_shard + loc * in_features * es, in_features * es,
                                         in_features * es, piece, in_features * es};
            if (b_full)
                segs[n++] = tpl::CopySegment{(const char *)b_full + src * es, (char *)b_shard + loc * es, 0, 0,
                                             1, piece * es};
        } else {
            segs[n++] = tpl::CopySegment{(const char *)w_full + src * es, (char *)w_shard + loc * es,
                                         in_features * es, cols * es, out_features, piece * es};
        }
        loc += piece;
        off += size;
    }
    return hip_status(tpl::launch_copy_segments(segs, n, stream), fn);
}

}  // extern "C"
