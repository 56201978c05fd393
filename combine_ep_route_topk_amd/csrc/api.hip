// api.hip -- the extern "C" entry points of libep_route_topk (declared and
// documented in include/ep_route_topk.h): synchronous argument validation,
// workspace sizing, then kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstddef>
#include <cstring>
#include <random>

#include "../../include/ep_route_topk.h"
#include "ep_internal.h"

namespace ep {
LaunchTiming& launch_timing() {
    static thread_local LaunchTiming t;
    return t;
}
}  // namespace ep

namespace {

thread_local char g_err[512] = "";

// Clears the one-shot timing hook when a compute entry point returns.
struct TimingScope {
    ~TimingScope() { ep::launch_timing() = ep::LaunchTiming{}; }
};

ep_status fail(ep_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

ep_status ok() {
    g_err[0] = '\0';
    return EP_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

ep_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess)
        return fail(EP_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

// Sizes shared by route / layout / fused.
ep_status check_routing_sizes(const char* fn, int32_t T, int32_t k, int32_t E) {
    if (T < 1) return fail(EP_ERR_INVALID_ARG, "%s: T=%d must be >= 1", fn, T);
    if (E < 1) return fail(EP_ERR_INVALID_ARG, "%s: E=%d must be >= 1", fn, E);
    if (E > ep::kMaxE) return fail(EP_ERR_UNSUPPORTED, "%s: E=%d exceeds %d", fn, E, ep::kMaxE);
    if (k < 1 || k > E) return fail(EP_ERR_INVALID_ARG, "%s: k=%d must be in [1, E=%d]", fn, k, E);
    if (k > ep::kMaxK) return fail(EP_ERR_UNSUPPORTED, "%s: k=%d exceeds %d", fn, k, ep::kMaxK);
    if (int64_t(T) * k >= (int64_t(1) << 30))
        return fail(EP_ERR_UNSUPPORTED, "%s: T*k=%lld must be < 2^30", fn, (long long)T * k);
    return EP_OK;
}

ep_status check_rows(const char* fn, int32_t T, int32_t H, int32_t k) {
    if (T < 1) return fail(EP_ERR_INVALID_ARG, "%s: T=%d must be >= 1", fn, T);
    if (k < 1) return fail(EP_ERR_INVALID_ARG, "%s: k=%d must be >= 1", fn, k);
    if (k > ep::kMaxK) return fail(EP_ERR_UNSUPPORTED, "%s: k=%d exceeds %d", fn, k, ep::kMaxK);
    if (H < 8 || H % 8 != 0) return fail(EP_ERR_INVALID_ARG, "%s: H=%d must be a positive multiple of 8", fn, H);
    if (H > (1 << 20)) return fail(EP_ERR_UNSUPPORTED, "%s: H=%d exceeds 2^20", fn, H);
    if (int64_t(T) * k >= (int64_t(1) << 30))
        return fail(EP_ERR_UNSUPPORTED, "%s: T*k=%lld must be < 2^30", fn, (long long)T * k);
    if (int64_t(T) * H >= (int64_t(1) << 40))
        return fail(EP_ERR_UNSUPPORTED, "%s: T*H=%lld must be < 2^40", fn, (long long)T * H);
    return EP_OK;
}

#define EP_REQUIRE_PTR(fn, p, a)                                                     \
    do {                                                                             \
        if (!(p)) return fail(EP_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);         \
        if (!aligned((p), (a)))                                                      \
            return fail(EP_ERR_INVALID_ARG, "%s: %s is not %d-byte aligned", fn, #p, \
                        int(a));                                                     \
    } while (0)

#define EP_TRY(expr)                  \
    do {                              \
        ep_status st_ = (expr);       \
        if (st_ != EP_OK) return st_; \
    } while (0)

}  // namespace

extern "C" {

int ep_abi_version(void) { return EP_ABI_VERSION; }

const char* ep_status_string(ep_status status) {
    switch (status) {
        case EP_OK: return "EP_OK";
        case EP_ERR_INVALID_ARG: return "EP_ERR_INVALID_ARG";
        case EP_ERR_UNSUPPORTED: return "EP_ERR_UNSUPPORTED";
        case EP_ERR_WORKSPACE: return "EP_ERR_WORKSPACE";
        case EP_ERR_LAUNCH: return "EP_ERR_LAUNCH";
        case EP_ERR_DEVICE: return "EP_ERR_DEVICE";
        case EP_ERR_TIMEOUT: return "EP_ERR_TIMEOUT";
        default: return "EP_ERR_UNKNOWN";
    }
}

const char* ep_last_error(void) { return g_err; }

ep_status ep_set_timing_events(void* start_event, void* stop_event)
{
    ep::launch_timing() = ep::LaunchTiming{static_cast<hipEvent_t>(start_event),
                                           static_cast<hipEvent_t>(stop_event)};
    return ok();
}

ep_status ep_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                        int32_t normalize, int32_t* topk_idx, float* topk_w, void* stream)
{
    const char* fn = "ep_route_topk";
    TimingScope timing_scope;
    EP_TRY(check_routing_sizes(fn, T, k, E));
    EP_REQUIRE_PTR(fn, logits, 4);
    EP_REQUIRE_PTR(fn, topk_idx, 4);
    EP_REQUIRE_PTR(fn, topk_w, 4);
    return launched(ep::launch_route_topk(logits, T, E, k, normalize ? 1 : 0, topk_idx,
                                          topk_w, static_cast<hipStream_t>(stream)),
                    fn);
}

size_t ep_dispatch_layout_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t R)
{
    if (T < 1 || k < 1 || E < 1 || R < 1) return 0;
    return ep::layout_plan(T, k, E).bytes;
}

ep_status ep_dispatch_layout(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                             int32_t R, int32_t* expert_counts, int32_t* expert_offsets,
                             int32_t* rank_counts, int32_t* rank_offsets, int32_t* pos,
                             int32_t* slot_src, void* workspace, size_t workspace_bytes,
                             void* stream)
{
    const char* fn = "ep_dispatch_layout";
    TimingScope timing_scope;
    EP_TRY(check_routing_sizes(fn, T, k, E));
    if (R < 1 || E % R != 0)
        return fail(EP_ERR_INVALID_ARG, "%s: R=%d must be >= 1 and divide E=%d", fn, R, E);
    EP_REQUIRE_PTR(fn, topk_idx, 4);
    EP_REQUIRE_PTR(fn, expert_counts, 4);
    EP_REQUIRE_PTR(fn, expert_offsets, 4);
    EP_REQUIRE_PTR(fn, rank_counts, 4);
    EP_REQUIRE_PTR(fn, rank_offsets, 4);
    EP_REQUIRE_PTR(fn, pos, 4);
    if (slot_src && !aligned(slot_src, 4))
        return fail(EP_ERR_INVALID_ARG, "%s: slot_src is not 4-byte aligned", fn);
    EP_REQUIRE_PTR(fn, workspace, 256);
    const size_t need = ep::layout_plan(T, k, E).bytes;
    if (workspace_bytes < need)
        return fail(EP_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn,
                    workspace_bytes, need);
    return launched(ep::launch_dispatch_layout(topk_idx, T, k, E, R, expert_counts,
                                               expert_offsets, rank_counts, rank_offsets,
                                               pos, slot_src, workspace,
                                               static_cast<hipStream_t>(stream)),
                    fn);
}

ep_status ep_dispatch_layout_noalloc(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                                     int32_t R, int32_t* expert_counts, int32_t* expert_offsets,
                                     int32_t* rank_counts, int32_t* rank_offsets, int32_t* pos,
                                     int32_t* slot_src, void* stream)
{
    const char* fn = "ep_dispatch_layout_noalloc";
    TimingScope timing_scope;
    EP_TRY(check_routing_sizes(fn, T, k, E));
    if (R < 1 || E % R != 0)
        return fail(EP_ERR_INVALID_ARG, "%s: R=%d must be >= 1 and divide E=%d", fn, R, E);
    EP_REQUIRE_PTR(fn, topk_idx, 4);
    EP_REQUIRE_PTR(fn, expert_counts, 4);
    EP_REQUIRE_PTR(fn, expert_offsets, 4);
    EP_REQUIRE_PTR(fn, rank_counts, 4);
    EP_REQUIRE_PTR(fn, rank_offsets, 4);
    EP_REQUIRE_PTR(fn, pos, 4);
    if (slot_src && !aligned(slot_src, 4))
        return fail(EP_ERR_INVALID_ARG, "%s: slot_src is not 4-byte aligned", fn);
    const size_t need = ep::layout_plan(T, k, E).bytes;
    if (need > ep::kLayoutScratchBytes)
        return fail(EP_ERR_UNSUPPORTED,
                    "%s: T=%d k=%d E=%d needs %zu bytes of layout scratch; the library's static "
                    "buffer holds %zu (use ep_dispatch_layout with a workspace)",
                    fn, T, k, E, need, ep::kLayoutScratchBytes);
    void* ws = nullptr;
    const hipError_t e = ep::layout_scratch(&ws);
    if (e != hipSuccess)
        return fail(EP_ERR_DEVICE, "%s: the static scratch has no address on this device: %s",
                    fn, hipGetErrorString(e));
    return launched(ep::launch_dispatch_layout(topk_idx, T, k, E, R, expert_counts,
                                               expert_offsets, rank_counts, rank_offsets,
                                               pos, slot_src, ws,
                                               static_cast<hipStream_t>(stream)),
                    fn);
}

ep_status ep_dispatch(const uint16_t* x, int32_t T, int32_t H, int32_t k,
                      const int32_t* pos, uint16_t* send, void* stream)
{
    const char* fn = "ep_dispatch";
    TimingScope timing_scope;
    EP_TRY(check_rows(fn, T, H, k));
    EP_REQUIRE_PTR(fn, x, 16);
    EP_REQUIRE_PTR(fn, pos, 4);
    EP_REQUIRE_PTR(fn, send, 16);
    return launched(ep::launch_dispatch(x, T, H, k, pos, send,
                                        static_cast<hipStream_t>(stream)),
                    fn);
}

ep_status ep_combine(const uint16_t* y, const int32_t* pos, const float* topk_w,
                     int32_t T, int32_t H, int32_t k, uint16_t* out, void* stream)
{
    const char* fn = "ep_combine";
    TimingScope timing_scope;
    EP_TRY(check_rows(fn, T, H, k));
    EP_REQUIRE_PTR(fn, y, 16);
    EP_REQUIRE_PTR(fn, pos, 4);
    EP_REQUIRE_PTR(fn, topk_w, 4);
    EP_REQUIRE_PTR(fn, out, 16);
    return launched(ep::launch_combine(y, pos, topk_w, T, H, k, out,
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

ep_status ep_combine_grad(const uint16_t* grad_out, const uint16_t* y, const int32_t* pos,
                          const float* topk_w, int32_t T, int32_t H, int32_t k,
                          uint16_t* grad_y, float* grad_w, void* stream)
{
    const char* fn = "ep_combine_grad";
    TimingScope timing_scope;
    EP_TRY(check_rows(fn, T, H, k));
    EP_REQUIRE_PTR(fn, grad_out, 16);
    EP_REQUIRE_PTR(fn, y, 16);
    EP_REQUIRE_PTR(fn, pos, 4);
    EP_REQUIRE_PTR(fn, topk_w, 4);
    EP_REQUIRE_PTR(fn, grad_y, 16);
    EP_REQUIRE_PTR(fn, grad_w, 4);
    return launched(ep::launch_combine_grad(grad_out, y, pos, topk_w, T, H, k, grad_y, grad_w,
                                            static_cast<hipStream_t>(stream)),
                    fn);
}

ep_status ep_dispatch_grad(const uint16_t* grad_send, const int32_t* pos, int32_t T,
                           int32_t H, int32_t k, uint16_t* grad_x, void* stream)
{
    const char* fn = "ep_dispatch_grad";
    TimingScope timing_scope;
    EP_TRY(check_rows(fn, T, H, k));
    EP_REQUIRE_PTR(fn, grad_send, 16);
    EP_REQUIRE_PTR(fn, pos, 4);
    EP_REQUIRE_PTR(fn, grad_x, 16);
    return launched(ep::launch_dispatch_grad(grad_send, pos, T, H, k, grad_x,
                                             static_cast<hipStream_t>(stream)),
                    fn);
}

size_t ep_fused_row_stride_bytes(int32_t H)
{
    if (H < 8 || H % 8 != 0) return 0;
    return ep::fused_row_stride(H);
}

size_t ep_fused_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t R)
{
    if (T < 1 || k < 1 || E < 1 || R < 1) return 0;
    return ep::fused_plan(T, k, E).bytes;
}

ep_status ep_fused_workspace_init(void* workspace, size_t workspace_bytes, void* stream)
{
    const char* fn = "ep_fused_workspace_init";
    EP_REQUIRE_PTR(fn, workspace, 256);
    if (workspace_bytes < sizeof(ep::WsHeader))
        return fail(EP_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs at least %zu", fn,
                    workspace_bytes, sizeof(ep::WsHeader));
    // The first epoch is unpredictable across workspaces and processes, so a
    // trailer left in a reused send buffer by another workspace's call can
    // never be mistaken for one of this workspace's.
    static std::atomic<uint64_t> counter{0};
    std::random_device rd;
    uint64_t e = (uint64_t(rd()) << 32) ^ uint64_t(rd()) ^
                 uint64_t(std::chrono::steady_clock::now().time_since_epoch().count()) ^
                 (counter.fetch_add(1) * 0x9E3779B97F4A7C15ull);
    if (e == 0) e = 1;
    return launched(ep::launch_fused_init(workspace, e, static_cast<hipStream_t>(stream)), fn);
}

ep_status ep_fused_dispatch_combine_sync(const uint16_t* x, const int32_t* topk_idx,
                                         const float* topk_w, int32_t T, int32_t H, int32_t k,
                                         int32_t E, int32_t R, int32_t* expert_counts,
                                         int32_t* expert_offsets, int32_t* rank_counts,
                                         int32_t* rank_offsets, int32_t* pos,
                                         uint8_t* send_rows, uint16_t* out, void* workspace,
                                         size_t workspace_bytes, uint32_t spin_limit,
                                         int32_t sync, void* stream)
{
    const char* fn = "ep_fused_dispatch_combine";
    TimingScope timing_scope;
    if (sync < 0 || sync >= ep::kNumFusedSync)
        return fail(EP_ERR_INVALID_ARG, "%s: sync=%d is not one of the EP_FUSED_SYNC_* modes", fn,
                    sync);
    EP_TRY(check_routing_sizes(fn, T, k, E));
    EP_TRY(check_rows(fn, T, H, k));
    if (R < 1 || E % R != 0)
        return fail(EP_ERR_INVALID_ARG, "%s: R=%d must be >= 1 and divide E=%d", fn, R, E);
    EP_REQUIRE_PTR(fn, x, 16);
    EP_REQUIRE_PTR(fn, topk_idx, 4);
    EP_REQUIRE_PTR(fn, topk_w, 4);
    EP_REQUIRE_PTR(fn, expert_counts, 4);
    EP_REQUIRE_PTR(fn, expert_offsets, 4);
    EP_REQUIRE_PTR(fn, rank_counts, 4);
    EP_REQUIRE_PTR(fn, rank_offsets, 4);
    EP_REQUIRE_PTR(fn, pos, 4);
    EP_REQUIRE_PTR(fn, send_rows, 128);
    EP_REQUIRE_PTR(fn, out, 16);
    EP_REQUIRE_PTR(fn, workspace, 256);
    const size_t need = ep::fused_plan(T, k, E).bytes;
    if (workspace_bytes < need)
        return fail(EP_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn,
                    workspace_bytes, need);
    return launched(ep::launch_fused(x, topk_idx, topk_w, T, H, k, E, R, expert_counts,
                                     expert_offsets, rank_counts, rank_offsets, pos, send_rows,
                                     out, workspace, spin_limit, 0, sync,
                                     static_cast<hipStream_t>(stream)),
                    fn);
}

ep_status ep_fused_dispatch_combine(const uint16_t* x, const int32_t* topk_idx,
                                    const float* topk_w, int32_t T, int32_t H, int32_t k,
                                    int32_t E, int32_t R, int32_t* expert_counts,
                                    int32_t* expert_offsets, int32_t* rank_counts,
                                    int32_t* rank_offsets, int32_t* pos, uint8_t* send_rows,
                                    uint16_t* out, void* workspace, size_t workspace_bytes,
                                    void* stream)
{
    return ep_fused_dispatch_combine_sync(x, topk_idx, topk_w, T, H, k, E, R, expert_counts,
                                          expert_offsets, rank_counts, rank_offsets, pos,
                                          send_rows, out, workspace, workspace_bytes, 0,
                                          ep::kSyncItemEvents, stream);
}

ep_status ep_fused_last_epoch(const void* workspace, uint64_t* epoch, void* stream)
{
    const char* fn = "ep_fused_last_epoch";
    EP_REQUIRE_PTR(fn, workspace, 256);
    if (!epoch) return fail(EP_ERR_INVALID_ARG, "%s: epoch is NULL", fn);
    hipStream_t s = static_cast<hipStream_t>(stream);
    ep::WsHeader h{};
    hipError_t e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipMemcpy(&h, workspace, sizeof(h), hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return fail(EP_ERR_LAUNCH, "%s: reading the workspace failed: %s", fn,
                    hipGetErrorString(e));
    if (h.magic != ep::kFusedMagic)
        return fail(EP_ERR_WORKSPACE, "%s: not a fused workspace (ep_fused_workspace_init)", fn);
    *epoch = h.last_epoch;
    return ok();
}

ep_status ep_expert_slices(const int32_t* expert_offsets, int32_t E, int32_t P, int64_t* start,
                           int32_t* expert, int64_t* offset, void* stream)
{
    const char* fn = "ep_expert_slices";
    TimingScope timing_scope;
    if (E < 1 || E > (1 << 20)) return fail(EP_ERR_INVALID_ARG, "%s: E=%d must be in [1, 2^20]", fn, E);
    if (P < 1 || P >= (1 << 24)) return fail(EP_ERR_INVALID_ARG, "%s: P=%d must be in [1, 2^24)", fn, P);
    EP_REQUIRE_PTR(fn, expert_offsets, 4);
    EP_REQUIRE_PTR(fn, start, 8);
    EP_REQUIRE_PTR(fn, expert, 4);
    EP_REQUIRE_PTR(fn, offset, 8);
    return launched(ep::launch_slices(expert_offsets, E, P, start, expert, offset,
                                      static_cast<hipStream_t>(stream)),
                    fn);
}

int64_t ep_lpt_task_count(const int32_t* rank_offsets, int32_t R, int64_t unit_rows)
{
    if (!rank_offsets || R < 1 || unit_rows < 1) return -1;
    return ep::lpt_unit_count(rank_offsets, R, unit_rows);
}

ep_status ep_lpt_partition(const int32_t* rank_offsets, int32_t R, int64_t row_bytes,
                           int64_t unit_rows, const int32_t* tier_of_peer, const double* alpha,
                           const double* beta, const int32_t* cap, int32_t ntier, int32_t C,
                           ep_task* tasks, int64_t max_tasks, int64_t* core_begin,
                           double* core_load)
{
    const char* fn = "ep_lpt_partition";
    if (!rank_offsets || !alpha || !beta || !cap || !core_begin || (!tasks && max_tasks > 0))
        return fail(EP_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    if (R < 1 || ntier < 1 || C < 1 || unit_rows < 1 || row_bytes < 1)
        return fail(EP_ERR_INVALID_ARG, "%s: R=%d ntier=%d C=%d unit_rows=%lld row_bytes=%lld "
                    "must all be >= 1", fn, R, ntier, C, (long long)unit_rows, (long long)row_bytes);
    for (int32_t p = 0; p < R; ++p) {
        if (rank_offsets[p + 1] < rank_offsets[p] || rank_offsets[p] < 0)
            return fail(EP_ERR_INVALID_ARG, "%s: rank_offsets must be non-decreasing and >= 0", fn);
        if (tier_of_peer && (tier_of_peer[p] < 0 || tier_of_peer[p] >= ntier))
            return fail(EP_ERR_INVALID_ARG, "%s: tier_of_peer[%d]=%d outside [0, %d)", fn, p,
                        tier_of_peer[p], ntier);
    }
    for (int32_t t = 0; t < ntier; ++t)
        if (!(beta[t] > 0.0) || cap[t] < 1)
            return fail(EP_ERR_INVALID_ARG, "%s: tier %d needs beta > 0 and cap >= 1", fn, t);
    const int64_t need = ep::lpt_unit_count(rank_offsets, R, unit_rows);
    if (max_tasks < need)
        return fail(EP_ERR_INVALID_ARG, "%s: max_tasks=%lld, %lld units are needed", fn,
                    (long long)max_tasks, (long long)need);
    ep::lpt_partition(rank_offsets, R, row_bytes, unit_rows, tier_of_peer, alpha, beta, cap, C,
                      tasks, max_tasks, core_begin, core_load);
    return ok();
}

ep_status ep_window_copy(const void* src, void* dst, int64_t row_bytes, int64_t S,
                         const ep_task* tasks, const int64_t* core_begin,
                         const int64_t* slice_start, int32_t C, uint64_t* core_clock,
                         uint32_t* bad, void* stream)
{
    const char* fn = "ep_window_copy";
    TimingScope timing_scope;
    if (row_bytes < 16 || row_bytes % 16 != 0)
        return fail(EP_ERR_INVALID_ARG, "%s: row_bytes=%lld must be a positive multiple of 16", fn,
                    (long long)row_bytes);
    if (S < 0 || C < 1 || uint32_t(C) > ep::kMaxGrid)
        return fail(EP_ERR_INVALID_ARG, "%s: S=%lld must be >= 0 and C=%d in [1, 2^20]", fn,
                    (long long)S, C);
    if (!tasks == !slice_start)
        return fail(EP_ERR_INVALID_ARG, "%s: give either tasks (with core_begin) or slice_start", fn);
    if (tasks) {
        EP_REQUIRE_PTR(fn, tasks, 8);
        EP_REQUIRE_PTR(fn, core_begin, 8);
    } else {
        EP_REQUIRE_PTR(fn, slice_start, 8);
    }
    EP_REQUIRE_PTR(fn, src, 16);
    EP_REQUIRE_PTR(fn, dst, 16);
    if (core_clock && !aligned(core_clock, 8))
        return fail(EP_ERR_INVALID_ARG, "%s: core_clock is not 8-byte aligned", fn);
    if (bad && !aligned(bad, 4)) return fail(EP_ERR_INVALID_ARG, "%s: bad is not 4-byte aligned", fn);
    return launched(ep::launch_window_copy(src, dst, row_bytes, S, tasks, core_begin, slice_start,
                                           C, core_clock, bad, static_cast<hipStream_t>(stream)),
                    fn);
}

size_t ep_rank_coalesce_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t R)
{
    if (T < 1 || k < 1 || E < 1 || R < 1) return 0;
    return ep::coalesce_plan(T, k, R).bytes;
}

ep_status ep_rank_coalesce(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E, int32_t R,
                           int32_t* rank_counts, int32_t* rank_offsets, int32_t* row_of_pick,
                           int32_t* send_pos, int32_t* row_src, uint64_t* row_experts,
                           void* workspace, size_t workspace_bytes, void* stream)
{
    const char* fn = "ep_rank_coalesce";
    TimingScope timing_scope;
    EP_TRY(check_routing_sizes(fn, T, k, E));
    if (R < 1 || E % R != 0)
        return fail(EP_ERR_INVALID_ARG, "%s: R=%d must be >= 1 and divide E=%d", fn, R, E);
    if (E / R > 64)
        return fail(EP_ERR_UNSUPPORTED, "%s: E/R=%d local experts per rank exceed 64", fn, E / R);
    EP_REQUIRE_PTR(fn, topk_idx, 4);
    EP_REQUIRE_PTR(fn, rank_counts, 4);
    EP_REQUIRE_PTR(fn, rank_offsets, 4);
    EP_REQUIRE_PTR(fn, row_of_pick, 4);
    EP_REQUIRE_PTR(fn, send_pos, 4);
    EP_REQUIRE_PTR(fn, row_src, 4);
    EP_REQUIRE_PTR(fn, row_experts, 8);
    EP_REQUIRE_PTR(fn, workspace, 256);
    const size_t need = ep::coalesce_plan(T, k, R).bytes;
    if (workspace_bytes < need)
        return fail(EP_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn,
                    workspace_bytes, need);
    return launched(ep::launch_rank_coalesce(topk_idx, T, k, E, R, rank_counts, rank_offsets,
                                             row_of_pick, send_pos, row_src, row_experts,
                                             workspace, static_cast<hipStream_t>(stream)),
                    fn);
}

size_t ep_expand_records_workspace_bytes(int32_t C, int32_t L)
{
    if (C < 1 || L < 1 || L > 64) return 0;
    return ep::coalesce_plan(C, L, L).bytes;
}

ep_status ep_expand_records(const uint16_t* rows, const uint64_t* masks, int32_t C, int32_t H,
                            int32_t L, int32_t* expert_counts, int32_t* expert_offsets,
                            int32_t* pos, uint16_t* recv, int64_t recv_rows, void* workspace,
                            size_t workspace_bytes, void* stream)
{
    const char* fn = "ep_expand_records";
    TimingScope timing_scope;
    if (C < 1) return fail(EP_ERR_INVALID_ARG, "%s: C=%d must be >= 1", fn, C);
    if (L < 1 || L > 64) return fail(EP_ERR_INVALID_ARG, "%s: L=%d must be in [1, 64]", fn, L);
    if (int64_t(C) * L >= (int64_t(1) << 30))
        return fail(EP_ERR_UNSUPPORTED, "%s: C*L=%lld must be < 2^30", fn, (long long)C * L);
    if (H < 8 || H % 8 != 0)
        return fail(EP_ERR_INVALID_ARG, "%s: H=%d must be a positive multiple of 8", fn, H);
    if (H > (1 << 20)) return fail(EP_ERR_UNSUPPORTED, "%s: H=%d exceeds 2^20", fn, H);
    if (recv_rows < 0)
        return fail(EP_ERR_INVALID_ARG, "%s: recv_rows=%lld must be >= 0", fn, (long long)recv_rows);
    EP_REQUIRE_PTR(fn, rows, 16);
    EP_REQUIRE_PTR(fn, masks, 8);
    EP_REQUIRE_PTR(fn, expert_counts, 4);
    EP_REQUIRE_PTR(fn, expert_offsets, 4);
    EP_REQUIRE_PTR(fn, pos, 4);
    EP_REQUIRE_PTR(fn, recv, 16);
    EP_REQUIRE_PTR(fn, workspace, 256);
    const size_t need = ep::coalesce_plan(C, L, L).bytes;
    if (workspace_bytes < need)
        return fail(EP_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn,
                    workspace_bytes, need);
    return launched(ep::launch_expand_records(rows, masks, C, H, L, expert_counts, expert_offsets,
                                              pos, recv, recv_rows, workspace,
                                              static_cast<hipStream_t>(stream)),
                    fn);
}

ep_status ep_exchange_waves(int32_t N, int32_t* peer)
{
    const char* fn = "ep_exchange_waves";
    if (N < 1 || N > 32768) return fail(EP_ERR_INVALID_ARG, "%s: N=%d must be in [1, 32768]", fn, N);
    if (N > 1 && !peer) return fail(EP_ERR_INVALID_ARG, "%s: peer is NULL", fn);
    ep::exchange_waves(N, peer);
    return ok();
}

ep_status ep_get_device_error(const void* workspace, void* stream)
{
    const char* fn = "ep_get_device_error";
    EP_REQUIRE_PTR(fn, workspace, 256);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t head[2] = {0, 0};
    hipError_t e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipMemcpy(head, workspace, sizeof(head), hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return fail(EP_ERR_LAUNCH, "%s: reading the workspace failed: %s", fn,
                    hipGetErrorString(e));
    if (head[0] != ep::kLayoutMagic && head[0] != ep::kFusedMagic)
        return fail(EP_ERR_WORKSPACE, "%s: workspace was never written by this library", fn);
    if (head[1] == ep::kDevOk) return ok();
    if (head[1] == ep::kDevTimeout)
        return fail(EP_ERR_TIMEOUT, "%s: a bounded device-side wait expired", fn);
    if (head[1] == ep::kDevOverflow)
        return fail(EP_ERR_DEVICE, "%s: the slots outnumber the receive buffer's rows", fn);
    if (head[1] == ep::kDevSentinel)
        return fail(EP_ERR_DEVICE, "%s: a payload row began with the sentinel mode's reserved "
                    "pattern", fn);
    return fail(EP_ERR_DEVICE, "%s: an expert id outside [0, E) was seen", fn);
}

}  // extern "C"
