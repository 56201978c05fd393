// partition.hip -- skew-balanced work partition for consumers of the send
// buffer, and a persistent consumer that follows a partition.
//
// UBEP sec. 3.3 ("Token-level Load Partition", Algorithm 1): the slots of the
// send buffer are cut into equal contiguous slices, one per worker, so no two
// workers differ by more than one slot however skewed the experts are; each
// worker finds the expert whose cumulative range covers its first slot, and
// the offset inside it, by a search over the cumulative counts.  Here a wave
// per worker searches expert_offsets with ballots over 64 pivots per step
// (two steps for E <= 4096) instead of UBEP's three-pivot vector count.
//
// StrataCL sec. 6.2 and App. B: the windows of the destination peers are cut
// into transfer units, each with an estimated cost alpha_t + bytes / beta_t
// for the peer's tier, and an LPT-style list scheduler assigns them, longest
// first, to the least-loaded core whose next issue stripe still has room for
// the unit's peer under a per-tier fan-out cap; each core then follows its
// task list in order.  That scheduler is host code (ep_lpt_partition).
//
// ep_window_copy is the consumer: C persistent workgroups, one per "core",
// each copying the rows of its tasks (or of its slice) from the send buffer
// to a receive buffer of the same layout -- the one-GPU stand-in for the
// per-peer transfers -- and recording when it started and finished, so the
// completion-time gap between the cores can be measured.
#include <algorithm>
#include <cstring>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/ep_route_topk.h"
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kWavesPerBlock = kBlock / kWave;

// ---------------------------------------------------------------- slices
// One wave per worker p: start = floor(p*S/P); the covering expert is the
// last e in [0, E) with expert_offsets[e] <= start (empty experts, whose
// range is empty, are never the last such e when start < S).  Each step puts
// 64 pivots over the window [lo, hi) and keeps the part after the last pivot
// at or below start.
__global__ __launch_bounds__(kBlock) void slices_kernel(const int32_t* __restrict__ eo, int E,
                                                        int P, int64_t* __restrict__ start,
                                                        int32_t* __restrict__ expert,
                                                        int64_t* __restrict__ offset)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = lane_id();
    const int p = int(blockIdx.x) * kWavesPerBlock + wave;
    if (p > P) return;
    const int64_t S = eo[E];
    const int64_t st = int64_t(p) * S / P;
    if (p == P) {
        if (lane == 0) start[P] = S;
        return;
    }
    int e = E;
    if (st < S) {
        int lo = 0, hi = E;
        while (hi - lo > 1) {
            const int stride = (hi - lo + kWave - 1) / kWave;
            const int pv = lo + lane * stride;
            const bool le = pv < hi && int64_t(eo[pv]) <= st;
            const uint64_t m = ballot(le);          // lane 0 (pivot lo) always holds
            const int last = 63 - __clzll((long long)m);
            const int nlo = lo + last * stride;
            hi = nlo + stride < hi ? nlo + stride : hi;
            lo = nlo;
        }
        e = lo;
    }
    if (lane == 0) {
        start[p] = st;
        expert[p] = e;
        offset[p] = e < E ? st - eo[e] : 0;
    }
}

// ---------------------------------------------------------------- consumer
// Copies rows [r0, r0 + n) of a buffer of row_bytes-byte rows with the whole
// workgroup, 16 bytes per thread and round: streaming loads, streaming
// stores.  row_bytes is a multiple of 16.
__device__ __forceinline__ void copy_rows(const char* __restrict__ src, char* __restrict__ dst,
                                          int64_t row_bytes, int64_t r0, int64_t n)
{
    const int64_t b0 = r0 * row_bytes;
    const int64_t nv = n * row_bytes / 16;
    constexpr int U = 4;
    int64_t v = threadIdx.x;
    for (; v + (U - 1) * kBlock < nv; v += U * kBlock) {
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = load16_nt(src + b0 + (v + u * kBlock) * 16);
#pragma unroll
        for (int u = 0; u < U; ++u) store16_nt(dst + b0 + (v + u * kBlock) * 16, x[u]);
    }
    for (; v < nv; v += kBlock) store16_nt(dst + b0 + v * 16, load16_nt(src + b0 + v * 16));
}

// Workgroup c follows tasks[core_begin[c] .. core_begin[c+1]) in order, or,
// with no task list, copies slice [slice_start[c], slice_start[c+1]).  A task
// outside [0, S) rows is skipped and counted in *bad.  core_clock[2c] and
// [2c+1]: the constant-rate wall clock (wall_clock64) when the workgroup
// started and ended.
__global__ __launch_bounds__(kBlock) void window_copy_kernel(
    const char* __restrict__ src, char* __restrict__ dst, int64_t row_bytes, int64_t S,
    const ep_task* __restrict__ tasks, const int64_t* __restrict__ core_begin,
    const int64_t* __restrict__ slice_start, uint64_t* __restrict__ core_clock,
    uint32_t* __restrict__ bad)
{
    const int c = blockIdx.x;
    const uint64_t t0 = uint64_t(wall_clock64());
    if (tasks) {
        for (int64_t i = core_begin[c]; i < core_begin[c + 1]; ++i) {
            const int64_t r0 = tasks[i].first_row, n = tasks[i].rows;
            if (r0 < 0 || n < 0 || r0 > S || n > S - r0) {
                if (bad && threadIdx.x == 0) atomicAdd(bad, 1u);
                continue;
            }
            copy_rows(src, dst, row_bytes, r0, n);
        }
    } else {
        const int64_t r0 = slice_start[c], r1 = slice_start[c + 1];
        if (r0 >= 0 && r0 <= r1 && r1 <= S)
            copy_rows(src, dst, row_bytes, r0, r1 - r0);
        else if (bad && threadIdx.x == 0)
            atomicAdd(bad, 1u);
    }
    __syncthreads();
    if (core_clock && threadIdx.x == 0) {
        core_clock[2 * c] = t0;
        core_clock[2 * c + 1] = uint64_t(wall_clock64());
    }
}

}  // namespace

hipError_t launch_slices(const int32_t* eo, int E, int P, int64_t* start, int32_t* expert,
                         int64_t* offset, hipStream_t s)
{
    const uint32_t grid = uint32_t((P + 1 + kWavesPerBlock - 1) / kWavesPerBlock);
    EP_LAUNCH(slices_kernel, dim3(grid), dim3(kBlock), 0, s, eo, E, P, start, expert, offset);
    return hipGetLastError();
}

hipError_t launch_window_copy(const void* src, void* dst, int64_t row_bytes, int64_t S,
                              const ep_task* tasks, const int64_t* core_begin,
                              const int64_t* slice_start, int C, uint64_t* core_clock,
                              uint32_t* bad, hipStream_t s)
{
    EP_LAUNCH(window_copy_kernel, dim3(C), dim3(kBlock), 0, s, static_cast<const char*>(src),
              static_cast<char*>(dst), row_bytes, S, tasks, core_begin, slice_start, core_clock,
              bad);
    return hipGetLastError();
}

// ---------------------------------------------------------------- LPT (host)
int64_t lpt_unit_count(const int32_t* rank_offsets, int R, int64_t unit_rows)
{
    int64_t u = 0;
    for (int p = 0; p < R; ++p) {
        const int64_t rows = int64_t(rank_offsets[p + 1]) - rank_offsets[p];
        u += (rows + unit_rows - 1) / unit_rows;
    }
    return u;
}

// Returns the number of tasks, or -1 when max_tasks is too small.
int64_t lpt_partition(const int32_t* rank_offsets, int R, int64_t row_bytes, int64_t unit_rows,
                      const int32_t* tier_of_peer, const double* alpha, const double* beta,
                      const int32_t* cap, int C, ep_task* tasks, int64_t max_tasks,
                      int64_t* core_begin, double* core_load)
{
    struct Unit {
        double cost;
        int32_t peer;
        int64_t first_row, rows;
    };
    std::vector<Unit> units;
    for (int p = 0; p < R; ++p) {
        const int t = tier_of_peer ? tier_of_peer[p] : 0;
        for (int64_t r = rank_offsets[p]; r < rank_offsets[p + 1]; r += unit_rows) {
            const int64_t n = std::min<int64_t>(unit_rows, int64_t(rank_offsets[p + 1]) - r);
            units.push_back({alpha[t] + double(n * row_bytes) / beta[t], p, r, n});
        }
    }
    const int64_t U = int64_t(units.size());
    if (U > max_tasks) return -1;
    // longest first; equal costs keep their unit order
    std::vector<int64_t> order(U);
    for (int64_t j = 0; j < U; ++j) order[j] = j;
    std::stable_sort(order.begin(), order.end(),
                     [&](int64_t a, int64_t b) { return units[a].cost > units[b].cost; });
    // cores ordered by (load, index): the least-loaded core with room comes first
    std::set<std::pair<double, int>> by_load;
    std::vector<double> load(C, 0.0);
    std::vector<int64_t> next(C, 0);
    for (int c = 0; c < C; ++c) by_load.insert({0.0, c});
    std::unordered_map<int64_t, int32_t> fan;       // (stripe * R + peer) -> units
    auto room = [&](int64_t k, int p) {
        auto it = fan.find(k * R + p);
        const int t = tier_of_peer ? tier_of_peer[p] : 0;
        return it == fan.end() || it->second < cap[t];
    };
    std::vector<int> core_of(U);
    std::vector<int64_t> stripe_of(U);
    for (int64_t i = 0; i < U; ++i) {
        const int64_t j = order[i];
        const int p = units[j].peer;
        int best = -1;
        for (const auto& lc : by_load)
            if (room(next[lc.second], p)) {
                best = lc.second;
                break;
            }
        if (best < 0) {                              // nobody has room: skip stripes
            best = by_load.begin()->second;
            while (!room(next[best], p)) ++next[best];
        }
        core_of[j] = best;
        stripe_of[j] = next[best];
        fan[next[best] * R + p] += 1;
        next[best] += 1;
        by_load.erase({load[best], best});
        load[best] += units[j].cost;
        by_load.insert({load[best], best});
    }
    // per-core task lists in stripe order
    std::vector<int64_t> count(C + 1, 0);
    for (int64_t j = 0; j < U; ++j) count[core_of[j] + 1] += 1;
    for (int c = 0; c < C; ++c) count[c + 1] += count[c];
    std::vector<int64_t> fill(count.begin(), count.end() - 1);
    std::vector<int64_t> by_core(U);
    for (int64_t j = 0; j < U; ++j) by_core[fill[core_of[j]]++] = j;
    for (int c = 0; c < C; ++c)
        std::sort(by_core.begin() + count[c], by_core.begin() + count[c + 1],
                  [&](int64_t a, int64_t b) { return stripe_of[a] < stripe_of[b]; });
    for (int64_t i = 0; i < U; ++i) {
        const int64_t j = by_core[i];
        tasks[i].peer = units[j].peer;
        tasks[i].stripe = int32_t(stripe_of[j]);
        tasks[i].first_row = units[j].first_row;
        tasks[i].rows = units[j].rows;
        tasks[i].cost = units[j].cost;
    }
    for (int c = 0; c <= C; ++c) core_begin[c] = count[c];
    if (core_load)
        for (int c = 0; c < C; ++c) core_load[c] = load[c];
    return U;
}

}  // namespace ep
