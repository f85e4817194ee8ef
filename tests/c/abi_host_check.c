/* A plain C11 consumer of the C ABI (include/tp_linear.h), linked against
 * libtp_linear.so.  It makes only calls that need no GPU: the tile-shape and
 * shard-shape queries, the validation that every entry point runs before any
 * device work, and the loader's error path for a missing file.  Prints one
 * line per check and "abi host check: N checks ok" when all pass; exits 1 on
 * the first failure. */
#include <stdalign.h>
#include <stdio.h>
#include <string.h>

#include "tp_linear.h"

static int checks = 0;
static _Alignas(16) unsigned short wdummy[8]; /* a valid, aligned weight address (never read) */

#define CHECK(cond, what)                                                        \
    do {                                                                         \
        ++checks;                                                                \
        if (!(cond)) {                                                           \
            printf("FAIL %s (last error: \"%s\")\n", what, tp_last_error());     \
            return 1;                                                            \
        }                                                                        \
        printf("ok   %s\n", what);                                               \
    } while (0)

int main(void)
{
    int64_t r = 0, c = 0;

    /* tile shapes on 256 compute units: the tiled kernel's choice, or (0, 0) for the
       weight-streaming kernel */
    CHECK(tp_linear_tile_shape(4608, 2304, 6144, TP_ACT_NONE, &r, &c) == TP_OK && r == 224 && c == 192,
          "tile shape 4608x2304x6144 is 224x192");
    CHECK(tp_linear_tile_shape(4608, 6144, 768, TP_ACT_NONE, &r, &c) == TP_OK && r == 224 && c == 256,
          "tile shape 4608x6144x768 is 224x256");
    CHECK(tp_linear_tile_shape(4, 9216, 6144, TP_ACT_NONE, &r, &c) == TP_OK && r == 0 && c == 0,
          "4 rows x 9216 x 6144 takes the weight-streaming kernel");
    CHECK(tp_linear_tile_shape(4, 9216, 6144, (tp_act)7, &r, &c) == TP_ERR_INVALID_ARG,
          "tile shape: unknown activation rejected");

    /* shard shapes (w_shard == NULL: query only) */
    CHECK(tp_plan_shard_slice(NULL, NULL, NULL, NULL, 18432, 6144, TP_BF16, TP_COLWISE, NULL, 0, 4, 1, &r, &c,
                              NULL) == TP_OK && r == 4608 && c == 6144,
          "colwise shard of [18432, 6144] at tp 4 is [4608, 6144]");
    CHECK(tp_plan_shard_slice(NULL, NULL, NULL, NULL, 6144, 18432, TP_BF16, TP_ROWWISE, NULL, 0, 8, 7, &r, &c,
                              NULL) == TP_OK && r == 6144 && c == 2304,
          "rowwise shard of [6144, 18432] at tp 8 is [6144, 2304]");
    {
        const int64_t blocks[3] = {1, 1, 1};
        CHECK(tp_plan_shard_slice(NULL, NULL, NULL, NULL, 18432, 6144, TP_BF16, TP_COLWISE, blocks, 3, 2, 0, &r,
                                  &c, NULL) == TP_OK && r == 9216 && c == 6144,
              "packed [1,1,1] colwise shard at tp 2 is [9216, 6144]");
    }
    CHECK(tp_plan_shard_slice(NULL, NULL, NULL, NULL, 6144, 6144, TP_BF16, TP_COLWISE, NULL, 0, 5, 0, &r, &c,
                              NULL) == TP_ERR_NOT_DIVISIBLE,
          "tp 5 does not divide 6144: rejected before device work");
    CHECK(strlen(tp_last_error()) > 0, "the failed call left a message");

    /* validation before any device work */
    CHECK(tp_fused_qkv_split(NULL, NULL, NULL, NULL, 48, 128, 6144, TP_BF16, 5, 0, NULL) == TP_ERR_NOT_DIVISIBLE,
          "QKV split: tp 5 does not divide 48 heads");
    CHECK(tp_fused_qkv_split(NULL, NULL, NULL, NULL, 48, 128, 6144, TP_BF16, 4, 4, NULL) == TP_ERR_INVALID_ARG,
          "QKV split: rank outside [0, tp)");
    CHECK(tp_linear_colwise(NULL, 6144, NULL, 6144, NULL, NULL, 2304, TP_BF16, TP_ACT_NONE, 4608, 2304, 6144,
                            NULL) == TP_ERR_INVALID_ARG,
          "colwise: null operands rejected");
    CHECK(tp_linear_colwise(NULL, 6144, wdummy, 6144, NULL, NULL, 2304, TP_BF16, TP_ACT_NONE, 0, 2304, 6144,
                            NULL) == TP_OK && tp_last_error()[0] == 0,
          "colwise: zero rows is a no-op");
    CHECK(tp_linear_rowwise(NULL, 768, NULL, 768, NULL, 6144, 4608, 6144, 100, NULL) == TP_ERR_UNSUPPORTED,
          "rowwise: K not a multiple of 64 rejected");
    CHECK(tp_partial_combine(NULL, 0, 6144, NULL, 6144, TP_F32, TP_F32, TP_COMBINE_SUM, NULL, NULL, 0, 4608,
                             6144, NULL) == TP_ERR_INVALID_ARG,
          "combine: no parts rejected");

    /* the loader's error path */
    CHECK(tp_load_shard("/nonexistent/ckpt.safetensors", "w", TP_COLWISE, NULL, 0, 2, 0, NULL, 0, &r, &c, NULL,
                        NULL) == TP_ERR_IO,
          "load: a missing file is an I/O error");

    printf("abi host check: %d checks ok\n", checks);
    return 0;
}
