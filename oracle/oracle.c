/*
 * oracle.c -- plain CPU oracle for one rank's share of tensor-parallel linear
 * layers (colwise / rowwise projections, head-aligned fused-QKV split, packed
 * slicing, and the layer-boundary combine).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no source, header, table or helper with the HIP library, and it includes no
 * GPU header.  Build: gcc -O2 -ffp-contract=off (never -ffast-math).
 *
 * Source pages (Hugging Face Diffusers documentation):
 *   [TP]  "Tensor parallelism" (optimization/tensor_parallelism), sections
 *         "Colwise and rowwise", "Fused projections", "Constraints and
 *         verification", and the opening definition of the method.
 *   [DI]  "Distributed inference", section "Tensor parallelism".
 *
 * Arithmetic conventions (readings where the pages are silent):
 *   - bf16 values are widened exactly; products of two bf16 numbers are exact
 *     in double; dot products accumulate in double, ascending k, multiply then
 *     add (no fused multiply-add: built with -ffp-contract=off).  This is the
 *     plain definition y = x.W^T + b evaluated to ~1e-16 relative.
 *   - Every rounding to bf16 is round-to-nearest, ties-to-even, done once from
 *     the double value (no double rounding through fp32).
 *   - The SUM combine adds fp32 partial buffers in fp32, in ascending rank
 *     order, then adds the bias once: the reading that an AllReduce over fp32
 *     partials sums them in their own precision in a fixed order.
 *
 * Weights use nn.Linear layout W[out_features, in_features], row-major, so
 * "dim 0" of the pages is a row index and "dim 1" a column index.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* bf16 <-> double                                                            */
/* ------------------------------------------------------------------------- */

/* Exact widening of a bf16 bit pattern: it is the top half of an fp32. */
double orc_bf16_to_double(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Correctly rounded double -> bf16 (nearest, ties to even).
 * bf16 keeps 8 significant bits and fp32's exponent range.  Write |v| = q*2^s
 * with the quantum 2^s of the bf16 binade that holds |v| (2^-133 below the
 * smallest normal), round q to an integer with ties to even, scale back.
 */
uint16_t orc_bf16_from_double(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    int e;
    (void)frexp(a, &e);                      /* a = m * 2^e, m in [0.5, 1) */
    int s = (e - 1 >= -126) ? (e - 8) : -133; /* quantum exponent          */
    double q = ldexp(a, -s);                  /* exact power-of-two scaling */
    double r = nearbyint(q);                  /* default mode: ties-to-even */
    double val = ldexp(r, s);
    if (val >= 0x1p128)
        return (uint16_t)(sign | 0x7F80u);     /* rounds past the max: inf   */
    float f = (float)val;                     /* exact: <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFFu));
}

void orc_round_bf16(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_from_double(in[i]);
}

void orc_widen_bf16(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_to_double(in[i]);
}

/* ------------------------------------------------------------------------- */
/* GELU, tanh form                                                            */
/* ------------------------------------------------------------------------- */

/*
 * GELU with the tanh approximation (Hendrycks & Gimpel, 2016):
 *   g(v) = v/2 * (1 + tanh( sqrt(2/pi) * (v + 0.044715 v^3) )).
 * The pages do not define the activation; the MLP workloads name GELU-tanh.
 */
double orc_gelu_tanh(double v)
{
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * v * (1.0 + tanh(c * (v + 0.044715 * v * v * v)));
}

/* ------------------------------------------------------------------------- */
/* Linear layer: y = act(x . W^T + b)                                         */
/* ------------------------------------------------------------------------- */

enum { ORC_ACT_NONE = 0, ORC_ACT_GELU_TANH = 1 };

typedef struct {
    const uint16_t *x;
    int64_t ldx;
    const uint16_t *w;
    int64_t ldw;
    const uint16_t *bias;
    int act;
    const int64_t *rows;
    int64_t n_rows;
    int64_t N, K;
    double *out; /* [n_rows, N] */
    int64_t r_begin, r_end;
} linear_job;

static void *linear_worker(void *arg)
{
    linear_job *j = (linear_job *)arg;
    double *xrow = (double *)malloc(sizeof(double) * (size_t)(j->K > 0 ? j->K : 1));
    for (int64_t t = j->r_begin; t < j->r_end; ++t) {
        const uint16_t *xs = j->x + j->rows[t] * j->ldx;
        for (int64_t k = 0; k < j->K; ++k)
            xrow[k] = orc_bf16_to_double(xs[k]);
        for (int64_t n = 0; n < j->N; ++n) {
            const uint16_t *ws = j->w + n * j->ldw;
            double acc = 0.0;
            for (int64_t k = 0; k < j->K; ++k) {
                double p = xrow[k] * orc_bf16_to_double(ws[k]);
                acc = acc + p;
            }
            if (j->bias)
                acc = acc + orc_bf16_to_double(j->bias[n]);
            if (j->act == ORC_ACT_GELU_TANH)
                acc = orc_gelu_tanh(acc);
            j->out[t * j->N + n] = acc;
        }
    }
    free(xrow);
    return NULL;
}

/*
 * For each listed row i: out[t, n] = act( sum_k x[rows[t], k] * W[n, k] + b[n] ).
 * x is [*, K] with row stride ldx (a strided column slice is a pointer offset
 * plus ldx), W is [N, K] with row stride ldw, bias is [N] or NULL.
 * Threads split the row list only, so every output element sees the same
 * operation sequence whatever the thread count.
 *
 * [TP] "Colwise and rowwise": the layer a shard stands for is an nn.Linear;
 * a colwise shard is this function on a row block of W, a rowwise shard on a
 * column block of W and of x (no bias: it is added once after the sum).
 */
void orc_linear_rows(const uint16_t *x, int64_t ldx, const uint16_t *w, int64_t ldw,
                     const uint16_t *bias, int act, const int64_t *rows, int64_t n_rows,
                     int64_t N, int64_t K, double *out, int n_threads)
{
    if (n_rows <= 0 || N <= 0)
        return;
    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > n_rows)
        n_threads = (int)n_rows;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    linear_job *jobs = (linear_job *)malloc(sizeof(linear_job) * (size_t)n_threads);
    for (int t = 0; t < n_threads; ++t) {
        linear_job j = {x, ldx, w, ldw, bias, act, rows, n_rows, N, K, out,
                        n_rows * t / n_threads, n_rows * (t + 1) / n_threads};
        jobs[t] = j;
    }
    for (int t = 1; t < n_threads; ++t)
        pthread_create(&tid[t], NULL, linear_worker, &jobs[t]);
    linear_worker(&jobs[0]);
    for (int t = 1; t < n_threads; ++t)
        pthread_join(tid[t], NULL);
    free(jobs);
    free(tid);
}

/* ------------------------------------------------------------------------- */
/* Shard slicing (weights)                                                    */
/* ------------------------------------------------------------------------- */

/*
 * [TP] "Colwise and rowwise": colwise shards the output features (weight
 * dim 0).  Rank r of P keeps rows [r*N/P, (r+1)*N/P) and the same bias range.
 * Caller guarantees P | N.
 */
void orc_shard_colwise(const uint16_t *w, const uint16_t *b, int64_t N, int64_t K, int P,
                       int r, uint16_t *w_shard, uint16_t *b_shard)
{
    int64_t n_loc = N / P;
    for (int64_t i = 0; i < n_loc; ++i)
        for (int64_t k = 0; k < K; ++k)
            w_shard[i * K + k] = w[(r * n_loc + i) * K + k];
    if (b && b_shard)
        for (int64_t i = 0; i < n_loc; ++i)
            b_shard[i] = b[r * n_loc + i];
}

/*
 * [TP] "Colwise and rowwise": rowwise shards the input features (weight
 * dim 1).  Rank r keeps columns [r*K/P, (r+1)*K/P) of every row.  The bias is
 * not sliced (it belongs to the summed output).  Caller guarantees P | K.
 */
void orc_shard_rowwise(const uint16_t *w, int64_t N, int64_t K, int P, int r, uint16_t *w_shard)
{
    int64_t k_loc = K / P;
    for (int64_t i = 0; i < N; ++i)
        for (int64_t k = 0; k < k_loc; ++k)
            w_shard[i * k_loc + k] = w[i * K + r * k_loc + k];
}

/*
 * [TP] "Fused projections": a packed weight holds several logical tensors
 * stacked along the sharded dim; each block is sharded on its own.  blocks[]
 * are proportional integers whose sum divides D = N: block i has
 * s_i = blocks[i] * (N / sum) rows starting at off_i = s_0 + .. + s_{i-1}.
 * Rank r keeps rows [off_i + r*s_i/P, off_i + (r+1)*s_i/P) of every block,
 * blocks kept in their original order.  The bias is cut the same way.
 * Caller guarantees sum | N and P | s_i.
 */
void orc_shard_packed_colwise(const uint16_t *w, const uint16_t *b, int64_t N, int64_t K,
                              const int64_t *blocks, int nb, int P, int r,
                              uint16_t *w_shard, uint16_t *b_shard)
{
    int64_t sum = 0;
    for (int i = 0; i < nb; ++i)
        sum += blocks[i];
    int64_t unit = N / sum;
    int64_t off = 0, dst = 0;
    for (int i = 0; i < nb; ++i) {
        int64_t s = blocks[i] * unit;
        int64_t part = s / P;
        for (int64_t t = 0; t < part; ++t) {
            int64_t src = off + r * part + t;
            for (int64_t k = 0; k < K; ++k)
                w_shard[dst * K + k] = w[src * K + k];
            if (b && b_shard)
                b_shard[dst] = b[src];
            ++dst;
        }
        off += s;
    }
}

/*
 * [TP] "Colwise and rowwise" (attention) and "Fused projections": a fused QKV
 * weight is [Q; K; V] stacked on dim 0, each H*hd rows, head-major inside
 * (row h*hd + d).  Colwise Q, K and V give each rank a subset of whole heads,
 * so P must divide H.  Rank r owns heads [r*H/P, (r+1)*H/P) of each of Q, K
 * and V; the shard is [Q_r; K_r; V_r].  Returns -1 when P does not divide H.
 */
int orc_qkv_split(const uint16_t *w, const uint16_t *b, int64_t H, int64_t hd, int64_t K,
                  int P, int r, uint16_t *w_shard, uint16_t *b_shard)
{
    if (P < 1 || r < 0 || r >= P || H % P != 0)
        return -1;
    int64_t h_loc = H / P;
    int64_t dst = 0;
    for (int which = 0; which < 3; ++which) {       /* Q, K, V */
        for (int64_t h = r * h_loc; h < (r + 1) * h_loc; ++h) {
            for (int64_t d = 0; d < hd; ++d) {
                int64_t src = which * H * hd + h * hd + d;
                for (int64_t k = 0; k < K; ++k)
                    w_shard[dst * K + k] = w[src * K + k];
                if (b && b_shard)
                    b_shard[dst] = b[src];
                ++dst;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Combine at the layer boundary                                              */
/* ------------------------------------------------------------------------- */

/*
 * [TP] opening definition and "Colwise and rowwise" (pairing): the rowwise
 * partial sums are added by an AllReduce at the block boundary.  On one GPU
 * that is out = ((p_0 + p_1) + ... + p_{P-1}) + b, in fp32, ascending rank,
 * bias (bf16, may be NULL) added once after the sum.
 */
void orc_combine_sum_f32(const float *const *parts, int P, int64_t ld_part, int64_t M,
                         int64_t N, const uint16_t *bias, float *out, int64_t ld_out)
{
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t n = 0; n < N; ++n) {
            float acc = parts[0][i * ld_part + n];
            for (int p = 1; p < P; ++p)
                acc = acc + parts[p][i * ld_part + n];
            if (bias)
                acc = acc + (float)orc_bf16_to_double(bias[n]);
            out[i * ld_out + n] = acc;
        }
    }
}

/*
 * [TP] opening definition (AllGather) and "Fused projections": the colwise
 * output slices are put back in global column order.  Shard r's output
 * columns are, block by block, its 1/P piece of each packed block (the
 * inverse of orc_shard_packed_colwise); blocks == NULL means one block
 * (plain colwise: shard r's column j goes to column r*n_part + j).
 * Elements are elem_size bytes (2 for bf16, 4 for fp32) copied verbatim.
 */
void orc_combine_concat(const void *const *parts, int P, int64_t ld_part, int64_t M,
                        int64_t n_part, const int64_t *blocks, int nb, int elem_size,
                        void *out, int64_t ld_out)
{
    int64_t one = 1;
    if (!blocks || nb <= 0) {
        blocks = &one;
        nb = 1;
    }
    int64_t sum = 0;
    for (int i = 0; i < nb; ++i)
        sum += blocks[i];
    int64_t n_full = n_part * P;
    int64_t unit = n_full / sum;
    for (int p = 0; p < P; ++p) {
        const char *src = (const char *)parts[p];
        int64_t loc = 0, off = 0;
        for (int i = 0; i < nb; ++i) {
            int64_t s = blocks[i] * unit;
            int64_t piece = s / P;
            for (int64_t t = 0; t < piece; ++t) {
                int64_t col_src = loc + t;
                int64_t col_dst = off + p * piece + t;
                for (int64_t row = 0; row < M; ++row)
                    memcpy((char *)out + (row * ld_out + col_dst) * elem_size,
                           src + (row * ld_part + col_src) * elem_size, (size_t)elem_size);
            }
            loc += piece;
            off += s;
        }
    }
}
