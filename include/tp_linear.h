/*
 * tp_linear.h -- C ABI of libtp_linear.so: one rank's share of the
 * tensor-parallel linear layers of a diffusion transformer, on one AMD
 * Instinct MI355X (gfx950).
 *
 * Source pages (Hugging Face Diffusers documentation):
 *   [TP] "Tensor parallelism": the opening definition (weights split by
 *        column or row, partial results joined by AllReduce / AllGather at the
 *        layer boundary), "Load a sharded model", "Limitations", "Colwise and
 *        rowwise", "Fused projections", "What to leave out", "Constraints and
 *        verification".
 *   [DI] "Distributed inference": section "Tensor parallelism".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.   Weights are nn.Linear W[out_features, in_features], row-major,
 *           in_features contiguous.  Activations are row-major [tokens, features].
 *           A leading dimension ("ld") is the distance in ELEMENTS between
 *           consecutive rows.
 * Dtypes.   Weights, activations and biases are bf16 (16-bit brain float,
 *           passed as raw bits).  Rowwise partial sums are fp32.
 * Pointers. Every pointer argument except `parts` and `blocks` (host arrays),
 *           the shape / dtype outputs and tp_load_shard's `path` and `name`
 *           (host strings) is a DEVICE pointer on the current HIP device.  The caller owns
 *           all memory; the library allocates no device memory and keeps no
 *           state between calls apart from the thread-local error message.
 * Streams.  Work is enqueued on `stream` (0 = the legacy default stream) and
 *           TP_OK means "enqueued": synchronise the stream before reading the
 *           results on the host.  tp_load_shard alone returns after its
 *           copies have completed.
 * Errors.   Arguments are checked before any HIP call.  On a non-OK status
 *           nothing has been launched or written (tp_load_shard: a read error
 *           found part-way may leave the destination partly written), and
 *           tp_last_error() returns a message for the calling thread.  There is no fallback path: an
 *           unsupported request is an error.
 * Alignment. Device base pointers must be 16-byte aligned and every ld a
 *           multiple of 16 bytes (8 bf16 / 4 fp32 elements) unless stated
 *           otherwise.
 * Aliasing. Outputs must not overlap inputs, except that the SUM combine may
 *           write in place into parts[0] (same ld).
 * Empty.    M == 0 (no tokens) is a valid no-op for the compute entry points.
 */
#ifndef TP_LINEAR_H
#define TP_LINEAR_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TP_OK = 0,
    TP_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, bad ld, rank, dtype, mode ...  */
    TP_ERR_NOT_DIVISIBLE = -2, /* a divisibility rule of the plan is violated             */
    TP_ERR_UNSUPPORTED = -3,   /* valid request outside what the kernels implement        */
    TP_ERR_HIP = -4,           /* the HIP runtime reported an error at launch             */
    TP_ERR_IO = -5             /* a checkpoint file could not be read or is malformed     */
} tp_status;

typedef enum { TP_BF16 = 0, TP_F32 = 1 } tp_dtype;

/* GELU with the tanh approximation: g(v) = v/2 (1 + tanh(sqrt(2/pi)(v + 0.044715 v^3))).
 * SwiGLU of a packed [gate; up] projection ([TP] "Fused projections": blocks
 * {1, 1} for a SwiGLU gate and up projection of equal halves): the weight
 * holds 2 n rows, gate then up, and the n outputs are
 * silu(x . gate^T + b_gate) * (x . up^T + b_up), silu(v) = v / (1 + e^-v). */
typedef enum { TP_ACT_NONE = 0, TP_ACT_GELU_TANH = 1, TP_ACT_SWIGLU = 2 } tp_act;

/* [TP] "Colwise and rowwise": colwise shards output features (weight dim 0),
 * rowwise shards input features (weight dim 1).  rowwise_split_input also
 * shards input features, for a standalone layer whose input is replicated on
 * every rank: each rank cuts its own slice of that input.  Its weight shard is
 * cut exactly like a rowwise one. */
typedef enum { TP_COLWISE = 0, TP_ROWWISE = 1, TP_ROWWISE_SPLIT_INPUT = 2 } tp_style;

/* [TP] opening definition: AllReduce (sum of partials) or AllGather (concat of
 * output slices) at the layer boundary, done here on one device. */
typedef enum { TP_COMBINE_SUM = 0, TP_COMBINE_CONCAT = 1 } tp_combine;

/*
 * tp_linear_colwise -- [TP] "Colwise and rowwise": a colwise rank holds a row
 * block W_r of the weight (a slice of the output features) and computes its
 * slice of the output, Y_r = act(X . W_r^T + b_r).  A head-aligned fused-QKV
 * shard ([TP] attention paragraph) is used the same way.
 *
 *   x       [M, K]        bf16, row stride ldx (>= K)
 *   w_shard [n_shard, K]  bf16, row stride ldw (>= K)
 *   bias    [n_shard]     bf16, or NULL (no bias); 8-byte alignment suffices
 *   y       [M, n_shard]  y_dtype (TP_BF16 or TP_F32), row stride ldy (>= n_shard)
 *   act     TP_ACT_NONE or TP_ACT_GELU_TANH, applied after the bias; or
 *           TP_ACT_SWIGLU: w_shard then holds 2 n_shard rows, the rank's gate
 *           rows followed by its up rows (what tp_plan_shard_slice cuts from a
 *           [gate; up] weight with blocks {1, 1}), bias likewise 2 n_shard
 *           entries [b_gate; b_up] or NULL, and
 *           y = silu(x . gate^T + b_gate) * (x . up^T + b_up)
 *
 * Arithmetic: bf16 products, fp32 accumulation (MFMA), bias and activation in
 * fp32, one rounding to y_dtype (round to nearest even for bf16).
 * Kernels, all under the same contract: up to 5 rows without SwiGLU (2 for
 * K > 6144; K <= 8192) a weight-streaming kernel (the skinny adaLN
 * modulation shape); other problems with up to 128 rows a split-K MFMA kernel
 * (all rows and a run of at most 48 output columns per workgroup); more rows
 * the tiled MFMA kernel.
 * Requires K % 64 == 0 and n_shard % 16 == 0, each operand view (rows x
 * leading dimension) below 2 GiB, row strides of at most 2^31 elements and
 * at most 2^22 output tiles of 192 x 256 (TP_ERR_UNSUPPORTED otherwise).
 */
tp_status tp_linear_colwise(const void *x, int64_t ldx, const void *w_shard, int64_t ldw,
                            const void *bias, void *y, int64_t ldy, tp_dtype y_dtype,
                            tp_act act, int64_t M, int64_t n_shard, int64_t K,
                            hipStream_t stream);

/*
 * tp_linear_rowwise -- [TP] "Colwise and rowwise": a rowwise rank holds a
 * column block W_r of the weight (a slice of the input features) and computes
 * a partial sum P_r = X_r . W_r^T from the matching slice X_r of its input (in
 * a colwise->rowwise pair, the colwise output shard).  No bias: it is added
 * once, after the partial sums are combined (tp_partial_combine, SUM).
 *
 *   x_shard [M, k_shard]  bf16, row stride ldx (a column slice of a wider
 *                         activation is a pointer offset plus ldx = full width)
 *   w_shard [N, k_shard]  bf16, row stride ldw (a column slice of the full
 *                         weight works the same way)
 *   partial [M, N]        fp32, row stride ldp (>= N, multiple of 4)
 *
 * Arithmetic: bf16 products, fp32 accumulation, fp32 store.  Kernels as for
 * tp_linear_colwise.
 * Requires k_shard % 64 == 0 and N % 16 == 0, each operand view (rows x
 * leading dimension) below 2 GiB, row strides of at most 2^31 elements and
 * at most 2^22 output tiles of 192 x 256 (TP_ERR_UNSUPPORTED otherwise).
 */
tp_status tp_linear_rowwise(const void *x_shard, int64_t ldx, const void *w_shard, int64_t ldw,
                            float *partial, int64_t ldp, int64_t M, int64_t N, int64_t k_shard,
                            hipStream_t stream);

/*
 * tp_linear_tile_shape -- host-only query of how tp_linear_colwise and
 * tp_linear_rowwise would run a problem of this shape (M rows, N output
 * features, K input features, activation act; for TP_ACT_SWIGLU, N counts the
 * outputs, not the 2 N weight rows) on the current device: *tile_rows and
 * *tile_cols receive the tiled kernel's output tile (rows 256, 224, 192, 128 or 64;
 * columns 256 or 192, or 128 outputs with SwiGLU); for the split-K kernel
 * (up to 128 rows) the rows its instance holds (16, 32, 48, 64, 96 or 128,
 * the smallest that covers M) and the run of 4 to 48 output columns (at most
 * 16 with SwiGLU) that each workgroup owns; or both 0 when the
 * weight-streaming kernel would run.  The choice depends on the shape and on
 * the device's compute-unit count.  It lets a caller check results at the
 * tiles' real edges.  No device work, no allocation.
 * Errors: TP_ERR_INVALID_ARG for a null output pointer, an unknown act, or
 * sizes outside 0 <= M, 0 < N, 0 < K, all at most 2^30.
 */
tp_status tp_linear_tile_shape(int64_t M, int64_t N, int64_t K, tp_act act, int64_t *tile_rows,
                               int64_t *tile_cols);

/*
 * tp_linear_rowwise_split_input -- [TP] "Colwise and rowwise" (the
 * rowwise_split_input style) and "What to leave out" (a large AdaLN
 * modulation projection is sharded this way).  The input x_full [M, k_full]
 * is the same on every rank.  Rank r of P takes its slice of the input
 * features, x_r = x_full[:, r*k_full/P : (r+1)*k_full/P], and computes the
 * partial sum P_r = x_r . W_r^T with its column block W_r [N, k_full/P] of the
 * weight (tp_plan_shard_slice, TP_ROWWISE_SPLIT_INPUT).  Summing the P
 * partials with the bias added once (tp_partial_combine, SUM) gives every
 * output feature on every rank.
 *
 *   x_full  [M, k_full]    bf16, row stride ldx >= k_full
 *   w_shard [N, k_full/P]  bf16, row stride ldw
 *   partial [M, N]         fp32, row stride ldp (>= N, multiple of 4)
 *
 * Arithmetic and kernels as tp_linear_rowwise on the slice (a few rows: the
 * weight-streaming kernel, up to 128 rows the split-K kernel).
 * Errors (before any device work): TP_ERR_INVALID_ARG for tp_degree < 1 or
 * rank outside [0, tp_degree); TP_ERR_NOT_DIVISIBLE if tp_degree does not
 * divide k_full; then every check of tp_linear_rowwise on the slice.
 */
tp_status tp_linear_rowwise_split_input(const void *x_full, int64_t ldx, int64_t k_full,
                                        const void *w_shard, int64_t ldw, float *partial,
                                        int64_t ldp, int64_t M, int64_t N, int tp_degree,
                                        int rank, hipStream_t stream);

/*
 * tp_fused_qkv_split -- [TP] "Colwise and rowwise" (attention: colwise Q, K, V
 * give each rank a subset of heads, so tp_degree must divide the head count)
 * and "Fused projections" (a packed weight is sharded block by block).
 *
 * The fused weight w_qkv [3*H*hd, K] stacks Q, K and V on dim 0, each head-major
 * (row h*hd + d).  Rank r of P = tp_degree receives whole heads
 * [r*H/P, (r+1)*H/P) of each: w_shard [3*(H/P)*hd, K] = [Q_r; K_r; V_r], rows
 * contiguous (ld = K for both).  b_qkv [3*H*hd] -> b_shard [3*(H/P)*hd] the same
 * way; pass both NULL for no bias (one NULL and not the other is an error).
 * dtype: TP_BF16 or TP_F32 element size; the copy is bit-exact.
 *
 * Errors: TP_ERR_NOT_DIVISIBLE if P does not divide H; TP_ERR_INVALID_ARG for
 * P < 1, rank outside [0, P), non-positive sizes, or null/misaligned pointers;
 * TP_ERR_UNSUPPORTED for a fused weight of more than 2^30 rows (3*H*hd).
 * Only 4-byte alignment is required here.
 */
tp_status tp_fused_qkv_split(const void *w_qkv, const void *b_qkv, void *w_shard, void *b_shard,
                             int64_t num_heads, int64_t head_dim, int64_t K, tp_dtype dtype,
                             int tp_degree, int rank, hipStream_t stream);

/*
 * tp_partial_combine -- [TP] opening definition and pairing rule: the layer
 * boundary joins the ranks' results, an AllReduce for rowwise partial sums or
 * an AllGather for colwise output slices.  Here all ranks' buffers live on
 * one device and the join is a device-side kernel.
 *
 *   parts      HOST array of num_parts (1..16) device pointers, each [M, n_part]
 *              with row stride ld_part
 *   out        [M, n_out] with row stride ld_out (device)
 *
 * TP_COMBINE_SUM:  in_dtype must be TP_F32; out_dtype TP_F32 or TP_BF16;
 *   out = ((parts[0] + parts[1]) + ... + parts[num_parts-1]) + bias, fp32 adds
 *   in ascending part order, bias (bf16 [n_part], 8-byte aligned, or NULL) added once, then one
 *   rounding to out_dtype (nearest even).  n_out = n_part.  blocks must be
 *   NULL.  May run in place: out == parts[0] with ld_out == ld_part.
 * TP_COMBINE_CONCAT:  in_dtype == out_dtype (TP_BF16 or TP_F32); bias NULL;
 *   n_out = num_parts * n_part.  Part p's columns go to their global columns:
 *   blocks == NULL: column j -> p*n_part + j (plain colwise).  Otherwise blocks
 *   (host, num_blocks <= 16 proportional positive integers, [TP] "Fused
 *   projections") describe the packed output: block i spans
 *   s_i = blocks[i]*n_out/sum(blocks) columns at offset o_i, and part p's local
 *   piece i (s_i/num_parts columns, in block order) goes to o_i + p*s_i/num_parts.
 *   This inverts tp_fused_qkv_split (blocks {1,1,1}) and packed colwise slicing.
 *   Bit-exact copy; pointers and ld only need element alignment here.
 *
 * Errors: TP_ERR_NOT_DIVISIBLE when the blocks do not tile n_out per the
 * constraints of [TP] "Constraints and verification"; TP_ERR_INVALID_ARG for
 * bad counts, dtypes, pointers or leading dimensions; TP_ERR_UNSUPPORTED for
 * leading dimensions above 2^31 elements.
 */
tp_status tp_partial_combine(const void *const *parts, int num_parts, int64_t ld_part, void *out,
                             int64_t ld_out, tp_dtype in_dtype, tp_dtype out_dtype,
                             tp_combine mode, const void *bias, const int64_t *blocks,
                             int num_blocks, int64_t M, int64_t n_part, hipStream_t stream);

/*
 * tp_plan_shard_slice -- [TP] "Colwise and rowwise" and "Fused projections";
 * [TP] "Load a sharded model" (each rank keeps only its slice of every planned
 * weight).  Cuts rank `rank`'s shard out of a full nn.Linear weight
 * w_full [out_features, in_features] (+ bias b_full [out_features]).
 *
 *   TP_COLWISE: rows [r*O/P, (r+1)*O/P) -> w_shard [O/P, I]; the bias is cut
 *     the same way into b_shard [O/P].
 *   TP_ROWWISE, TP_ROWWISE_SPLIT_INPUT: columns [r*I/P, (r+1)*I/P) ->
 *     w_shard [O, I/P]; such a shard owns no bias slice (the bias is added
 *     once after the sum), so b_full and b_shard must be NULL.
 *   blocks != NULL (host, num_blocks <= 16 proportional positive integers):
 *     packed sharding of the sharded dim, each block cut independently and the
 *     rank's pieces kept in block order.
 *   w_shard == NULL: shape query only -- fills *shard_rows, *shard_cols and
 *     returns without touching the device (w_full may then be NULL too).
 *
 * Shards are written contiguously (ld = shard_cols).  dtype: TP_BF16 or TP_F32
 * element size; the copy is bit-exact.  Only 4-byte alignment is required.
 * Errors (checked before any device work, [TP] "Constraints and verification"):
 *   TP_ERR_NOT_DIVISIBLE if P does not divide the sharded dim, sum(blocks) does
 *   not divide it, or any single packed block is not divisible by P;
 *   TP_ERR_INVALID_ARG for P < 1, rank outside [0, P), bad style/dtype, a
 *   bias with a rowwise style, or null pointers.
 */
tp_status tp_plan_shard_slice(const void *w_full, const void *b_full, void *w_shard,
                              void *b_shard, int64_t out_features, int64_t in_features,
                              tp_dtype dtype, tp_style style, const int64_t *blocks,
                              int num_blocks, int tp_degree, int rank, int64_t *shard_rows,
                              int64_t *shard_cols, hipStream_t stream);

/*
 * tp_load_shard -- [TP] "Load a sharded model" (the checkpoint is sharded as it
 * is read: each rank reads only its own slice of each weight and places it on
 * its GPU, so no rank holds a full-size weight) and "Limitations" (the sharded
 * load works with safetensors weights only).  Reads rank `rank`'s shard of
 * the tensor `name` of the safetensors file `path` into device memory.
 *
 *   path, name host strings, read during the call.
 *   A 2-D tensor [out, in] is cut like tp_plan_shard_slice cuts it (style,
 *   blocks, tp_degree, rank; same rules and errors).  A 1-D tensor (a bias) is
 *   cut like the rows of a colwise weight, blocks included, and only with
 *   TP_COLWISE (a rowwise bias is not sharded: load it whole with tp_degree 1).
 *   dst        device buffer of dst_bytes >= the shard's bytes, owned by the
 *              caller; the shard is written row-major and contiguous
 *              (ld = shard_cols).  NULL: query only -- reads the header, fills
 *              the outputs, makes no HIP call.
 *   shard_rows, shard_cols, dtype   host outputs (each may be NULL); a 1-D
 *              shard reports shard_rows = 1.
 *
 * Only the byte ranges of the rank's slice are read (one range per packed
 * block for a colwise cut, one range per row and block for a rowwise cut),
 * through two pinned host staging buffers of at most 32 MiB each, allocated
 * and freed inside the call, with the host-to-device copy of one buffer on
 * `stream` overlapping the read into the other: the host memory used is the
 * header plus those buffers, whatever the tensor's size.  The call returns
 * when the shard is on the device.  Tensor dtypes BF16 and F32 are supported.
 * Errors: TP_ERR_IO (file missing or unreadable, malformed header, tensor
 * absent, data range outside the file, a failed read), TP_ERR_UNSUPPORTED
 * (other dtypes, other than one or two dimensions, a dimension of 0 or above
 * 2^30), TP_ERR_INVALID_ARG / TP_ERR_NOT_DIVISIBLE as for tp_plan_shard_slice,
 * TP_ERR_INVALID_ARG for a rowwise cut of a 1-D tensor or a dst_bytes below
 * the shard's size, TP_ERR_HIP for runtime failures.
 */
tp_status tp_load_shard(const char *path, const char *name, tp_style style, const int64_t *blocks,
                        int num_blocks, int tp_degree, int rank, void *dst, int64_t dst_bytes,
                        int64_t *shard_rows, int64_t *shard_cols, tp_dtype *dtype, hipStream_t stream);

/* Message describing the last non-OK status returned on the calling thread
 * (empty string if none).  The pointer stays valid until the next call on
 * the same thread. */
const char *tp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TP_LINEAR_H */
