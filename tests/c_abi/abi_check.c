/* A C99 caller of libep_route_topk: checks that the header is plain C and
 * that the host-side entry points behave as documented.  No GPU work is
 * launched: every compute call here is rejected by argument validation, and
 * ep_lpt_partition runs on the host. */
#include <stdio.h>
#include <string.h>

#include "ep_route_topk.h"

#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "%s:%d: %s failed (%s)\n", __FILE__, __LINE__, \
                    #cond, ep_last_error());                               \
            return 1;                                                      \
        }                                                                  \
    } while (0)

int main(void)
{
    CHECK(ep_abi_version() == EP_ABI_VERSION);
    CHECK(strcmp(ep_status_string(EP_OK), "") != 0);
    CHECK(ep_status_string(EP_ERR_TIMEOUT) != NULL);

    /* validation happens before anything is enqueued */
    CHECK(ep_dispatch(NULL, 4, 16, 2, NULL, NULL, NULL) == EP_ERR_INVALID_ARG);
    CHECK(ep_combine(NULL, NULL, NULL, 0, 16, 2, NULL, NULL) == EP_ERR_INVALID_ARG);
    CHECK(ep_route_topk(NULL, 4, 8, 9, 1, NULL, NULL, NULL) == EP_ERR_INVALID_ARG);
    CHECK(ep_fused_dispatch_combine_sync(NULL, NULL, NULL, 4, 16, 2, 8, 2, NULL, NULL, NULL,
                                         NULL, NULL, NULL, NULL, NULL, 0, NULL, 0, 9,
                                         NULL) == EP_ERR_INVALID_ARG);
    CHECK(ep_dispatch_layout_workspace_bytes(4096, 8, 256, 32) > 0);
    CHECK(ep_fused_row_stride_bytes(7168) % 128 == 0);

    /* the host scheduler: 3 peers, windows of 5, 0 and 9 rows, units of 4 rows */
    {
        const int32_t ro[4] = {0, 5, 5, 14};
        const double alpha[1] = {1.0}, beta[1] = {1.0};
        const int32_t cap[1] = {2};
        ep_task tasks[8];
        int64_t core_begin[3];
        double load[2];
        int64_t n = ep_lpt_task_count(ro, 3, 4);
        int64_t i, rows = 0;
        CHECK(n == 5);                                   /* 2 + 0 + 3 units */
        CHECK(ep_lpt_partition(ro, 3, 16, 4, NULL, alpha, beta, cap, 1, 2, tasks, 8,
                               core_begin, load) == EP_OK);
        CHECK(core_begin[0] == 0 && core_begin[2] == n);
        for (i = 0; i < n; ++i) rows += tasks[i].rows;
        CHECK(rows == 14);
        CHECK(load[0] + load[1] == 5 * 1.0 + 14 * 16.0);
        CHECK(ep_lpt_partition(ro, 3, 16, 4, NULL, alpha, beta, cap, 1, 2, tasks, 4,
                               core_begin, load) == EP_ERR_INVALID_ARG);
    }
    {
        int32_t peer[3 * 4];
        int32_t w, q;
        CHECK(ep_exchange_waves(4, peer) == EP_OK);
        for (w = 1; w < 4; ++w)
            for (q = 0; q < 4; ++q) CHECK(peer[(w - 1) * 4 + q] == (q + w) % 4);
        CHECK(ep_rank_coalesce_workspace_bytes(4096, 8, 256, 32) > 0);
        CHECK(ep_rank_coalesce(NULL, 4, 2, 8, 2, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                               NULL) == EP_ERR_INVALID_ARG);
    }
    printf("c abi ok\n");
    return 0;
}
