// Fiber-based SIMT emulation runtime (see fake/hip/hip_runtime.h).
#include <hip/hip_runtime.h>
#include <mutex>
#include <condition_variable>

namespace emu {
thread_local Group* g_group = nullptr;
thread_local int g_lane_tid = 0;
thread_local U3 g_block = {0, 0, 0};
U3 g_grid = {1, 1, 1};
std::atomic<int> g_errors{0};
long g_op_limit = 2000000000L;
int g_pool = 8;

void yield_op(int kind, uint64_t v, int a) {
    Group* g = g_group;
    int t = g_lane_tid;
    g->op[t] = kind;
    g->val[t] = v;
    g->arg[t] = a;
    swapcontext(&g->ctx[t], &g->sched);
}
uint64_t result() { return g_group->res[g_lane_tid]; }

static void fiber_main() {
    Group* g = g_group;
    int t = g_lane_tid;
    g->body();
    g->op[t] = OP_EXIT;
    swapcontext(&g->ctx[t], &g->sched);
}

static void fail(Group* g, const char* why) {
    fprintf(stderr, "[emu] block (%u,%u): %s\n", g_block.x, g_block.y, why);
    for (int t = 0; t < g->nthreads; t += 64) {
        fprintf(stderr, "  wave %d ops:", t / 64);
        for (int l = 0; l < 64 && t + l < g->nthreads; ++l) fprintf(stderr, " %d", g->op[t + l]);
        fprintf(stderr, "\n");
    }
    g_errors++;
    std::abort();
}

static void run_group(const std::function<void()>& body, int nthreads) {
    Group g;
    g.nthreads = nthreads;
    g.ctx.resize(nthreads);
    g.stacks.resize(nthreads);
    g.op.assign(nthreads, -1);          // -1 = not started / runnable
    g.val.assign(nthreads, 0);
    g.arg.assign(nthreads, 0);
    g.res.assign(nthreads, 0);
    g.body = body;
    g_group = &g;
    for (int t = 0; t < nthreads; ++t) {
        g.stacks[t].resize(256 * 1024);
        getcontext(&g.ctx[t]);
        g.ctx[t].uc_stack.ss_sp = g.stacks[t].data();
        g.ctx[t].uc_stack.ss_size = g.stacks[t].size();
        g.ctx[t].uc_link = nullptr;
        makecontext(&g.ctx[t], fiber_main, 0);
    }
    const int nw = (nthreads + 63) / 64;
    long idle_passes = 0;
    while (true) {
        bool ran_real = false, any_runnable = false;
        for (int t = 0; t < nthreads; ++t) {
            if (g.op[t] == -1 || g.op[t] == OP_NONE) {
                any_runnable = true;
                g_lane_tid = t;
                swapcontext(&g.sched, &g.ctx[t]);
                if (g.op[t] != OP_NONE) ran_real = true;
            }
        }
        // resolve wave ops: every lane of the wave that has not exited must be
        // at the same op; exited lanes are inactive (contribute 0, as lanes
        // outside EXEC do on the hardware)
        for (int w = 0; w < nw; ++w) {
            int lo = w * 64, hi = std::min(nthreads, lo + 64);
            int kind = -2;
            bool waiting = false, ready = true;
            for (int t = lo; t < hi; ++t) {
                int o = g.op[t];
                if (o == OP_EXIT) continue;
                if (o == OP_BALLOT || o == OP_SHFL) {
                    if (kind == -2) kind = o;
                    else if (kind != o) fail(&g, "lanes of one wave at different wave ops");
                    waiting = true;
                } else if (o == OP_SYNC) {
                    ready = false;
                    if (waiting) fail(&g, "part of a wave at a barrier, part at a wave op");
                } else {
                    ready = false;   // still running towards the op
                }
            }
            if (!waiting || !ready) {
                if (waiting) {
                    for (int t = lo; t < hi; ++t)
                        if (g.op[t] == OP_SYNC) fail(&g, "part of a wave at a barrier, part at a wave op");
                }
                continue;
            }
            if (kind == OP_BALLOT) {
                uint64_t m = 0;
                for (int t = lo; t < hi; ++t)
                    if (g.op[t] != OP_EXIT && g.val[t]) m |= uint64_t(1) << (t - lo);
                for (int t = lo; t < hi; ++t) g.res[t] = m;
            } else {
                for (int t = lo; t < hi; ++t) {
                    if (g.op[t] == OP_EXIT) continue;
                    int src = lo + g.arg[t];
                    if (src < lo || src >= hi) fail(&g, "shuffle source out of the wave");
                    if (g.op[src] == OP_EXIT) fail(&g, "shuffle reads an inactive lane");
                    g.res[t] = g.val[src];
                }
            }
            for (int t = lo; t < hi; ++t)
                if (g.op[t] != OP_EXIT) g.op[t] = OP_NONE;
            ran_real = true;
        }
        // resolve barrier
        int at_sync = 0, exited = 0;
        for (int t = 0; t < nthreads; ++t) {
            if (g.op[t] == OP_SYNC) at_sync++;
            if (g.op[t] == OP_EXIT) exited++;
        }
        if (exited == nthreads) break;
        if (at_sync > 0 && at_sync + exited == nthreads) {
            if (exited) fail(&g, "__syncthreads with some threads exited");
            for (int t = 0; t < nthreads; ++t) g.op[t] = OP_NONE;
            ran_real = true;
        }
        if (!any_runnable && !ran_real) fail(&g, "no fiber can make progress (deadlock inside the workgroup)");
        if (!ran_real) {
            if (++idle_passes > 50000000L) fail(&g, "spinning for too long");
            std::this_thread::yield();
        } else idle_passes = 0;
    }
    g_group = nullptr;
}

void launch(dim3 grid, dim3 block, std::function<void()> body) {
    g_grid = {grid.x, grid.y, grid.z};
    const long nblocks = long(grid.x) * grid.y;
    std::atomic<long> next{0};
    int pool = int(std::min<long>(nblocks, g_pool));
    std::vector<std::thread> th;
    for (int i = 0; i < pool; ++i)
        th.emplace_back([&]() {
            while (true) {
                long b = next.fetch_add(1);
                if (b >= nblocks) break;
                g_block = {unsigned(b % grid.x), unsigned(b / grid.x), 0};
                run_group(body, int(block.x));
            }
        });
    for (auto& t : th) t.join();
}
}  // namespace emu

extern "C" void emu_set_pool(int n) { emu::g_pool = n; }

// The batched combine on a chosen grid, so that small inputs take several
// full and partial batches (the library picks it only for large batches).
#include "../../combine_ep_route_topk_amd/csrc/ep_internal.h"
extern "C" int emu_combine_batched(const uint16_t* y, const int32_t* pos, const float* w, int T,
                                   int H, int k, uint16_t* out, int grid)
{
    const hipError_t e = ep::launch_combine_batched(y, pos, w, T, H, k, out, uint32_t(grid), nullptr);
    return e == hipSuccess ? 0 : int(e);
}
extern "C" int emu_errors() { return emu::g_errors.load(); }
