/* A C99 caller of libep_route_topk: checks that the header is plain C, that
 * the boundary's calls have exactly the prototypes written below (each is
 * assigned to a pointer of that type, so a differing signature does not
 * compile under -Werror), and that the host-side entry points behave as
 * documented.  No GPU work is launched: every compute call here is rejected
 * by argument validation, and ep_lpt_partition runs on the host. */
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

/* The boundary, written out independently of the header. */
typedef int (*abi_version_fn)(void);
typedef const char* (*status_string_fn)(ep_status);
typedef ep_status (*route_topk_fn)(const float*, int32_t, int32_t, int32_t, int32_t, int32_t*,
                                   float*, void*);
typedef size_t (*layout_ws_fn)(int32_t, int32_t, int32_t, int32_t);
typedef ep_status (*layout_fn)(const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t*,
                               int32_t*, int32_t*, int32_t*, int32_t*, int32_t*, void*, size_t,
                               void*);
typedef ep_status (*dispatch_fn)(const uint16_t*, int32_t, int32_t, int32_t, const int32_t*,
                                 uint16_t*, void*);
typedef ep_status (*combine_fn)(const uint16_t*, const int32_t*, const float*, int32_t, int32_t,
                                int32_t, uint16_t*, void*);
typedef size_t (*stride_fn)(int32_t);
typedef size_t (*fused_ws_fn)(int32_t, int32_t, int32_t, int32_t);
typedef ep_status (*fused_init_fn)(void*, size_t, void*);
typedef ep_status (*fused_fn)(const uint16_t*, const int32_t*, const float*, int32_t, int32_t,
                              int32_t, int32_t, int32_t, int32_t*, int32_t*, int32_t*, int32_t*,
                              int32_t*, uint8_t*, uint16_t*, void*, size_t, void*);
typedef ep_status (*device_error_fn)(const void*, void*);

int main(void)
{
    abi_version_fn f_version = ep_abi_version;
    status_string_fn f_status = ep_status_string;
    route_topk_fn f_route = ep_route_topk;
    layout_ws_fn f_layout_ws = ep_dispatch_layout_workspace_bytes;
    layout_fn f_layout = ep_dispatch_layout;
    dispatch_fn f_dispatch = ep_dispatch;
    combine_fn f_combine = ep_combine;
    stride_fn f_stride = ep_fused_row_stride_bytes;
    fused_ws_fn f_fused_ws = ep_fused_workspace_bytes;
    fused_init_fn f_fused_init = ep_fused_workspace_init;
    fused_fn f_fused = ep_fused_dispatch_combine;
    device_error_fn f_device_error = ep_get_device_error;

    /* each boundary call, through its pointer: validation rejects every one
     * before anything is enqueued */
    CHECK(f_version() == EP_ABI_VERSION);
    CHECK(strcmp(f_status(EP_ERR_WORKSPACE), "EP_ERR_WORKSPACE") == 0);
    CHECK(f_route(NULL, 4, 8, 2, 1, NULL, NULL, NULL) == EP_ERR_INVALID_ARG);
    CHECK(f_layout_ws(4096, 8, 256, 32) > 0);
    CHECK(f_layout(NULL, 4, 2, 8, 2, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
          EP_ERR_INVALID_ARG);
    CHECK(f_dispatch(NULL, 4, 16, 2, NULL, NULL, NULL) == EP_ERR_INVALID_ARG);
    CHECK(f_combine(NULL, NULL, NULL, 4, 16, 2, NULL, NULL) == EP_ERR_INVALID_ARG);
    CHECK(f_stride(7168) == 15360);
    CHECK(f_fused_ws(4096, 8, 256, 32) > f_layout_ws(4096, 8, 256, 32));
    CHECK(f_fused_init(NULL, 0, NULL) == EP_ERR_INVALID_ARG);
    CHECK(f_fused(NULL, NULL, NULL, 4, 16, 2, 8, 2, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                  NULL, 0, NULL) == EP_ERR_INVALID_ARG);
    CHECK(f_device_error(NULL, NULL) == EP_ERR_INVALID_ARG);

    CHECK(ep_abi_version() == EP_ABI_VERSION);
    CHECK(strcmp(ep_status_string(EP_OK), "") != 0);
    CHECK(ep_status_string(EP_ERR_TIMEOUT) != NULL);

    /* validation happens before anything is enqueued */
    CHECK(ep_dispatch(NULL, 4, 16, 2, NULL, NULL, NULL) == EP_ERR_INVALID_ARG);
    CHECK(ep_combine(NULL, NULL, NULL, 0, 16, 2, NULL, NULL) == EP_ERR_INVALID_ARG);
    CHECK(ep_route_topk(NULL, 4, 8, 9, 1, NULL, NULL, NULL) == EP_ERR_INVALID_ARG);
    CHECK(ep_fused_dispatch_combine_sync(NULL, NULL, NULL, 4, 16, 2, 8, 2, NULL, NULL, NULL,
                                         NULL, NULL, NULL, NULL, NULL, 0, 0, 9,
                                         NULL) == EP_ERR_INVALID_ARG);
    {
        uint64_t epoch = 0;
        CHECK(ep_fused_last_epoch(NULL, &epoch, NULL) == EP_ERR_INVALID_ARG);
    }
    CHECK(ep_dispatch_layout_workspace_bytes(4096, 8, 256, 32) > 0);
    CHECK(ep_fused_row_stride_bytes(7168) % 1024 == 0);

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
