// Fiber-based SIMT emulation runtime (see fake/hip/hip_runtime.h).
#include <hip/hip_runtime.h>
#include <mutex>
#include <condition_variable>
#include <random>
#include <unordered_map>

namespace emu {
thread_local Group* g_group = nullptr;
thread_local int g_lane_tid = 0;
thread_local U3 g_block = {0, 0, 0};
U3 g_grid = {1, 1, 1};
std::atomic<int> g_errors{0};
long g_op_limit = 2000000000L;
int g_pool = 8;

// ------------------------------------------------------------ weak memory
constexpr int kXcds = 8;
bool g_weak = false;
uint64_t g_weak_seed = 0;
thread_local int g_xcd = 0;
thread_local std::mt19937_64 g_rng;

// A 16-byte granule of one XCD's cache: its bytes and which of them are
// dirty (written here, not yet written back to memory).
struct Granule {
    uint8_t b[16];
    uint16_t dirty;
};
struct XcdCache {
    std::mutex mu;
    std::unordered_map<uintptr_t, Granule> lines;
};
XcdCache g_xcds[kXcds];

bool weak_active() { return g_weak && g_group != nullptr; }

static uint16_t byte_mask(int off, int n) { return uint16_t(((1u << n) - 1u) << off); }

static Granule& granule(XcdCache& x, uintptr_t base) {
    auto it = x.lines.find(base);
    if (it == x.lines.end()) {
        Granule g;
        std::memcpy(g.b, reinterpret_cast<const void*>(base), 16);
        g.dirty = 0;
        it = x.lines.emplace(base, g).first;
    }
    return it->second;
}

// A queued store completes: coherent ones write through to memory (and
// update this XCD's copy), plain ones land dirty in this XCD's cache.
static void complete(const Pending& s) {
    XcdCache& x = g_xcds[g_xcd];
    const uintptr_t base = s.addr & ~uintptr_t(15);
    const int off = int(s.addr & 15);
    std::lock_guard<std::mutex> hold(x.mu);
    if (s.coherent) {
        std::memcpy(reinterpret_cast<void*>(s.addr), s.bytes, size_t(s.n));
        auto it = x.lines.find(base);
        if (it != x.lines.end()) std::memcpy(it->second.b + off, s.bytes, size_t(s.n));
    } else {
        Granule& g = granule(x, base);
        std::memcpy(g.b + off, s.bytes, size_t(s.n));
        g.dirty |= byte_mask(off, s.n);
    }
}

static void complete_one(std::vector<Pending>& q, size_t i) {
    const Pending s = q[i];
    q.erase(q.begin() + long(i));
    complete(s);
}

void complete_all() {
    if (!weak_active()) return;
    std::vector<Pending>& q = g_group->pending[size_t(g_lane_tid)];
    while (!q.empty()) complete_one(q, size_t(g_rng() % q.size()));   // any order
}

// While a lane runs, each of its memory operations may first complete one of
// its queued stores, chosen at random.
static void maybe_complete() {
    std::vector<Pending>& q = g_group->pending[size_t(g_lane_tid)];
    if (!q.empty() && (g_rng() & 3) == 0) complete_one(q, size_t(g_rng() % q.size()));
}

static void write_back(XcdCache& x) {
    for (auto& kv : x.lines) {
        Granule& g = kv.second;
        if (!g.dirty) continue;
        uint8_t* m = reinterpret_cast<uint8_t*>(kv.first);
        for (int i = 0; i < 16; ++i)
            if (g.dirty & (1u << i)) m[i] = g.b[i];
        g.dirty = 0;
    }
}

void mem_store(void* p, const void* src, int n, bool coherent) {
    if (!weak_active()) {
        std::memcpy(p, src, size_t(n));
        return;
    }
    maybe_complete();
    Pending s;
    s.addr = reinterpret_cast<uintptr_t>(p);
    s.n = n;
    s.coherent = coherent;
    if ((s.addr & 15) + uintptr_t(n) > 16) {
        std::fprintf(stderr, "[emu] a %d-byte store crosses a 16-byte granule\n", n);
        std::abort();
    }
    std::memcpy(s.bytes, src, size_t(n));
    g_group->pending[size_t(g_lane_tid)].push_back(s);
}

void mem_load(void* dst, const void* p, int n, bool coherent) {
    if (!weak_active()) {
        std::memcpy(dst, p, size_t(n));
        return;
    }
    maybe_complete();
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uintptr_t base = a & ~uintptr_t(15);
    const int off = int(a & 15);
    if (off + n > 16) {
        std::fprintf(stderr, "[emu] a %d-byte load crosses a 16-byte granule\n", n);
        std::abort();
    }
    // A load from a lane to bytes that the lane itself still has stores
    // queued for is served after them (one wave's accesses to one address stay
    // in order), so by the time it returns they have reached the cache level
    // every wave on this XCD reads: they complete first, in issue order.
    {
        std::vector<Pending>& q = g_group->pending[size_t(g_lane_tid)];
        for (size_t i = 0; i < q.size();) {
            if ((q[i].addr & ~uintptr_t(15)) == base) complete_one(q, i);
            else ++i;
        }
    }
    uint8_t buf[16];
    {
        XcdCache& x = g_xcds[g_xcd];
        std::lock_guard<std::mutex> hold(x.mu);
        auto it = x.lines.find(base);
        if (coherent) {
            // memory, but this XCD's own dirty bytes are what its cache holds
            std::memcpy(buf, reinterpret_cast<const void*>(base), 16);
            if (it != x.lines.end())
                for (int i = 0; i < 16; ++i)
                    if (it->second.dirty & (1u << i)) buf[i] = it->second.b[i];
        } else {
            std::memcpy(buf, granule(x, base).b, 16);
        }
    }
    std::memcpy(dst, buf + off, size_t(n));
}

void waitcnt(int bits) {
#ifndef EMU_MUTATE_NO_STORE_WAIT
    // s_waitcnt vmcnt(0): vmcnt is bits [3:0] and [15:14].  The counter is
    // the wave's, not the lane's: the hardware issues every store of the
    // wave, for all its active lanes, before it reaches the wait, and the
    // wait covers them all.  Each lane completes its own queue, then the
    // lanes of the wave meet (a wave op), so no lane goes past the wait
    // while another lane of its wave still has a store outstanding.
    if (weak_active() && (bits & 0xF) == 0 && ((bits >> 14) & 3) == 0) {
        complete_all();
        yield_op(OP_WAITCNT, 0, 0);
    }
#else
    (void)bits;
#endif
}

void fence(int order, const char* scope) {
    if (!weak_active()) {
        std::atomic_thread_fence(std::memory_order_seq_cst);
        return;
    }
    const bool agent = scope == nullptr || std::strcmp(scope, "agent") == 0 ||
                       std::strcmp(scope, "") == 0;
    const bool rel = order == __ATOMIC_RELEASE || order == __ATOMIC_ACQ_REL ||
                     order == __ATOMIC_SEQ_CST;
    const bool acq = order == __ATOMIC_ACQUIRE || order == __ATOMIC_ACQ_REL ||
                     order == __ATOMIC_SEQ_CST;
    if (rel) {
        // the lane's stores complete, then (agent scope) the XCD's cache is
        // written back
        complete_all();
        if (agent) {
            XcdCache& x = g_xcds[g_xcd];
            std::lock_guard<std::mutex> hold(x.mu);
            write_back(x);
        }
    }
    if (acq && agent) {
        // invalidate: clean granules go; dirty ones keep their dirty bytes
        // and refresh the rest from memory
        XcdCache& x = g_xcds[g_xcd];
        std::lock_guard<std::mutex> hold(x.mu);
        for (auto it = x.lines.begin(); it != x.lines.end();) {
            Granule& g = it->second;
            if (!g.dirty) {
                it = x.lines.erase(it);
                continue;
            }
            const uint8_t* m = reinterpret_cast<const uint8_t*>(it->first);
            for (int i = 0; i < 16; ++i)
                if (!(g.dirty & (1u << i))) g.b[i] = m[i];
            ++it;
        }
    }
    std::atomic_thread_fence(std::memory_order_seq_cst);
}

// Kernel boundary: every cache written back and emptied.
static void flush_all_caches() {
    for (XcdCache& x : g_xcds) {
        std::lock_guard<std::mutex> hold(x.mu);
        write_back(x);
        x.lines.clear();
    }
}

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
    complete_all();              // a lane's stores complete before it ends
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
    g.pending.assign(size_t(nthreads), {});
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
        if (g_weak) {
            // background completion: on the hardware a store completes
            // whether or not its wave runs on
            for (int t = 0; t < nthreads; ++t) {
                std::vector<Pending>& q = g.pending[size_t(t)];
                if (!q.empty() && (g_rng() & 63) == 0) complete_one(q, size_t(g_rng() % q.size()));
            }
        }
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
                if (o == OP_BALLOT || o == OP_SHFL || o == OP_WAITCNT) {
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
            } else if (kind == OP_SHFL) {
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
                g_xcd = int(b % kXcds);
                g_rng.seed(g_weak_seed ^ (uint64_t(b) * 0x9E3779B97F4A7C15ull));
                run_group(body, int(block.x));
            }
        });
    for (auto& t : th) t.join();
    if (g_weak) flush_all_caches();
}
}  // namespace emu

extern "C" void emu_set_pool(int n) { emu::g_pool = n; }

// Weak memory mode on (seed for its random choices) or off.
extern "C" void emu_set_weak(int on, unsigned long long seed) {
    emu::flush_all_caches();
    emu::g_weak = on != 0;
    emu::g_weak_seed = seed;
}

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

// Message-passing litmus test of the weak memory mode: workgroup 0 (XCD 0)
// writes a 16-byte datum, then a flag; workgroup 1 (XCD 1) polls the flag and
// then reads the datum.  Returns how many of `trials` runs read a stale datum.
//   mode 0: plain datum store, coherent flag store, no release -- stale
//   mode 1: coherent datum store, wait for it, coherent flag; the reader
//           acquires, then loads plainly -- never stale
//   mode 2: plain datum store, agent-scope release (write-back), flag;
//           the reader acquires -- never stale
//   mode 3: as mode 1, but the reader loads the datum once before polling
//           and not again after an acquire -- stale (its cached copy)
//   mode 4: as mode 3 with an acquire after the flag -- never stale
// Mode 5 of the litmus: every lane of one wave stores its own word of the
// data (coherent stores), the wave waits for its stores, then lane 0 alone
// stores the flag.  The wait is the wave's, so the reader must never see a
// word of another lane stale.
static int litmus_wave_wait(int trials)
{
    int stale = 0;
    alignas(16) static uint32_t words[64];
    alignas(16) static uint64_t flag[2];
    for (int trial = 0; trial < trials; ++trial) {
        std::memset(words, 0, sizeof words);
        std::memset(flag, 0, sizeof flag);
        std::atomic<int> seen_stale{0};
        emu::launch(dim3(2), dim3(64), [&]() {
            const unsigned lane = threadIdx.x;
            if (blockIdx.x == 0) {
                const uint32_t v = uint32_t(trial) * 64u + lane + 1u;
                emu::mem_store(&words[lane], &v, 4, true);
                __builtin_amdgcn_s_waitcnt(0x0F70);
                if (lane == 0) __hip_atomic_store(&flag[0], uint64_t(1), __ATOMIC_RELAXED, 3);
            } else {
                if (lane != 0) return;
                long spins = 0;
                while (__hip_atomic_load(&flag[0], __ATOMIC_RELAXED, 3) != 1) {
                    if (++spins > 50000000L) { std::fprintf(stderr, "[emu] litmus hung\n"); std::abort(); }
                }
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                for (unsigned i = 0; i < 64; ++i) {
                    uint32_t r;
                    emu::mem_load(&r, &words[i], 4, false);
                    if (r != uint32_t(trial) * 64u + i + 1u) {
                        seen_stale.fetch_add(1);
                        break;
                    }
                }
            }
        });
        stale += seen_stale.load();
    }
    return stale;
}

extern "C" int emu_litmus_message_passing(int mode, int trials)
{
    if (mode == 5) return litmus_wave_wait(trials);
    int stale = 0;
    alignas(16) static uint32_t datum[4];
    alignas(16) static uint64_t flag[2];
    for (int trial = 0; trial < trials; ++trial) {
        std::memset(datum, 0, sizeof datum);
        std::memset(flag, 0, sizeof flag);
        std::atomic<int> seen_stale{0};
        emu::launch(dim3(2), dim3(64), [&]() {
            if (threadIdx.x != 0) return;
            const uint32_t v[4] = {uint32_t(trial) + 1u, 2u, 3u, 4u};
            if (blockIdx.x == 0) {
                emu::mem_store(datum, v, 16, mode == 1 || mode >= 3);
                if (mode == 1 || mode >= 3) __builtin_amdgcn_s_waitcnt(0x0F70);
                if (mode == 2) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                __hip_atomic_store(&flag[0], uint64_t(1), __ATOMIC_RELAXED, 3);
                for (int i = 0; i < 64; ++i) (void)__hip_atomic_load(&flag[1], __ATOMIC_RELAXED, 3);
            } else {
                uint32_t r[4];
                if (mode >= 3) emu::mem_load(r, datum, 16, false);   // primes this XCD's cache
                long spins = 0;
                while (__hip_atomic_load(&flag[0], __ATOMIC_RELAXED, 3) != 1) {
                    if (++spins > 50000000L) { std::fprintf(stderr, "[emu] litmus hung\n"); std::abort(); }
                }
                if (mode != 0 && mode != 3) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                emu::mem_load(r, datum, 16, false);
                if (std::memcmp(r, v, 16) != 0) seen_stale.fetch_add(1);
            }
        });
        stale += seen_stale.load();
    }
    return stale;
}
