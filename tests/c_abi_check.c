/* A plain C99 user of libsinkroute: the header must compile as C, and the
 * host-side calls (sizing, introspection, argument checks that return before
 * anything is enqueued) must work through it.  Nothing here touches a GPU.
 * Prints "ok" and exits 0, or names the first failed check and exits 1. */
#include <stdio.h>
#include <string.h>

#include "sinkroute.h"

static int failed = 0;

#define CHECK(cond)                                                  \
    do {                                                             \
        if (!(cond)) {                                               \
            printf("failed: %s (line %d)\n", #cond, __LINE__);      \
            failed = 1;                                              \
        }                                                            \
    } while (0)

static sr_shape shape_8b(int64_t T) {
    sr_shape s;
    memset(&s, 0, sizeof s);
    s.batch = 1;
    s.num_q_heads = 32;
    s.num_kv_heads = 8;
    s.head_dim = 128;
    s.seq_len = T;
    s.stride_t = 128;
    s.stride_h = T * 128;
    s.stride_b = 8 * T * 128;
    s.kv_dtype = SR_KV_BF16;
    return s;
}

int main(void) {
    sr_shape s = shape_8b(131072);
    sr_shape bad = s;
    sr_launch lau;
    sr_part parts[2];
    size_t ws;
    int32_t grid, lanes, cap, r;

    memset(&lau, 0, sizeof lau);
    CHECK(sizeof(sr_shape) == 56);
    CHECK(sizeof(sr_launch) == 16);
    CHECK(sizeof(sr_part) == 40);
    CHECK(sr_version() > 0);
    CHECK(strlen(sr_status_string(SR_ERR_UNSUPPORTED)) > 0);

    /* sizing: the ticket region (32768 + 1 tickets, padded) comes first */
    ws = sr_workspace_bytes(&s, NULL);
    CHECK(ws > 131328);
    CHECK(sr_workspace_bytes(&s, &lau) == ws); /* a zeroed policy is the default */
    bad.num_q_heads = 17 * 8; /* G = 17: outside the envelope */
    CHECK(sr_workspace_bytes(&bad, NULL) == 0);
    bad = s;
    bad.reserved = 1;
    CHECK(sr_workspace_bytes(&bad, NULL) == 0);

    /* introspection of the adaptive policy */
    grid = sr_grid_size(&s, NULL);
    lanes = sr_splits_for(&s, NULL, 4);
    cap = sr_split_cap(&s, NULL);
    CHECK(grid >= 8);
    CHECK(lanes >= 1 && lanes <= cap && (int64_t)lanes * 4 <= grid);
    r = sr_plan_parts(&s, NULL, 4, 0, parts, 2);
    CHECK(r >= 1 && r <= 2);
    CHECK(parts[0].item == 0 && parts[0].part == 0 && parts[0].first == 0);
    CHECK(parts[0].end > parts[0].first && parts[0].chunk >= 16);
    CHECK(sr_plan_parts(&s, NULL, 9, 0, parts, 2) == -1);    /* n_active > B*Hkv */
    CHECK(sr_plan_parts(&s, NULL, 4, grid, parts, 2) == -1); /* wg past the grid */
    CHECK(sr_plan_parts(&s, NULL, 4, 0, parts, 1) == -1);    /* room for < 2 parts */

    /* argument checks return before anything is enqueued */
    CHECK(sr_route(&s, NULL, NULL, 0.5f, NULL, NULL, NULL, NULL, NULL) == SR_ERR_INVALID_ARG);
    CHECK(sr_decode_attn(&s, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0.f, NULL, 0, NULL,
                         NULL) == SR_ERR_INVALID_ARG);
    CHECK(sr_route_decode(&bad, NULL, NULL, NULL, NULL, NULL, NULL, 0.5f, 0.f, NULL, NULL, NULL,
                          NULL, NULL, 0, NULL, NULL) == SR_ERR_INVALID_ARG);
    bad = s;
    bad.head_dim = 96;
    CHECK(sr_dense_decode(&bad, NULL, NULL, NULL, NULL, 0.f, NULL, 0, NULL, NULL) ==
          SR_ERR_UNSUPPORTED);

    if (!failed) printf("ok\n");
    return failed;
}
