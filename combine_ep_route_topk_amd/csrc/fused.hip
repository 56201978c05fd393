// fused.hip -- flag-in-payload persistent mode: dispatch layout + dispatch +
// combine (identity experts) in ONE launch, with no kernel-boundary barrier.
//
// UBEP sec. 3.2 (kernel decomposition): instead of global barriers, tasks
// poll the data they depend on as soon as it is published (the prefix-sum
// tasks write the per-expert offsets, reordering tasks poll for them).
// UBEP sec. 3.4 / Fig. 6 (Data-as-Flag): the readiness flag travels inside
// the data, so seeing the flag proves the data arrived.  UBEP sec. 6 /
// Table 5: hardware without large single-copy-atomic writes needs fences or
// acknowledgements, and GPU work maps to persistent kernels.  HyperParallel-MoE
// sec. 4.3-4.4: a single launch whose workers wait on event counters with
// static thresholds.
//
// Work items are handed out by an atomic ticket in dependency order, and an
// item only ever waits for items with smaller tickets -- which were claimed
// by workgroups that are already running -- so the launch cannot deadlock
// whatever the number of co-resident workgroups:
//   [hist]    one per tile: tile histogram + stable ranks (shared with the
//             three-launch layout), then hist_done += 1 (release).
//   [scan]    one per kScanItems counters: waits for hist_done == nTiles
//             (an event counter with a static threshold), block scan, then
//             decoupled look-back over 64-bit status words that carry the
//             call's epoch next to flag and value, then publishes every
//             base as a 64-bit word (epoch << 32 | base): the base value is
//             its own readiness flag.
//   [scatter] tokens [8i, 8i+8): polls the base words of its picks, computes
//             pos, copies each x row into its k send rows (streaming stores),
//             writes {slot_src, 0} into the rows' trailers, one release fence
//             per wave, then the 64-bit epoch into every trailer.
//   [combine] tokens [8i, 8i+8): recomputes pos, polls the k trailers of
//             each token until they hold this call's epoch, one acquire fence
//             per wave, then the same fp32 reduction as ep_combine.
// A row's trailer is its flag: on gfx950 a 64-bit aligned store is
// single-copy atomic but a 14 KiB row is not, hence payload -> release ->
// trailer, and trailer -> acquire -> payload on the reading side.  Fences
// are amortised over a wave's 2 tokens x k rows.
//
// Every wait is bounded by spin_limit polling rounds; an expired wait sets
// the workspace's timeout word and every later wait gives up at once, so the
// grid always drains.  The last workgroup to leave derives the per-expert /
// per-rank counts, records the error word and resets the counters and the
// epoch for the next call (the workspace is reused without a memset).
#include "ep_combine_dev.h"
#include "ep_device.h"
#include "ep_internal.h"
#include "ep_layout_dev.h"

namespace ep {
namespace {

constexpr int kTokPerWave = 2;                               // per scatter/combine item
constexpr int kTokPerItem = kTokPerWave * kWavesPerBlock;    // 8
constexpr uint64_t kStFlagAggregate = uint64_t(1) << 30;
constexpr uint64_t kStFlagInclusive = uint64_t(2) << 30;
constexpr uint64_t kStValueMask = (uint64_t(1) << 30) - 1;

struct FusedArgs {
    const uint16_t* x;
    const int32_t* idx;
    const float* w;
    int T, k, E, R, nvec;
    int64_t S;
    int nTiles, nCnt, nScan, nItems;      // nItems scatter items == combine items
    int64_t stride;                       // bytes per send row (payload + trailer + pad)
    int64_t trailer_off;                  // = 2H
    int32_t* expert_counts;
    int32_t* expert_offsets;
    int32_t* rank_counts;
    int32_t* rank_offsets;
    int32_t* pos;
    uint8_t* send_rows;
    uint16_t* out;
    WsHeader* hdr;
    int32_t* cnt;
    int32_t* local_rank;
    uint64_t* status;
    uint64_t* fbase;
    uint32_t spin_limit;
};

// Bounded wait helper state: returns false once this wait has used up its
// polling rounds (it then raises the call's timeout word) or once another
// wait has raised it.  The shared word is read only every 64th round: all
// waiting waves reading one line on every round would serialise behind it.
struct Waiter {
    uint32_t spins = 0;
    __device__ bool tick(WsHeader* hdr, uint32_t limit) {
        ++spins;
        if ((spins & 63) == 0 && ld_relaxed(&hdr->timeout.v) != 0) return false;
        if (spins > limit) {
            st_relaxed(&hdr->timeout.v, 1u);
            return false;
        }
        backoff();
        return true;
    }
};

__device__ __forceinline__ bool published(uint64_t word, uint32_t ep32) {
    return uint32_t(word >> 32) == ep32;
}

// ---------------------------------------------------------------- hist item
__device__ void do_hist(const FusedArgs& a, int tile, int32_t (*hist)[kMaxE]) {
    hist_tile(a.idx, a.S, a.E, a.nTiles, tile, a.cnt, a.local_rank, hist);
    fence_release();                       // this wave's cnt / local_rank writes
    __syncthreads();
    if (threadIdx.x == 0) fetch_add(&a.hdr->hist_done.v, 1u);
}

// ---------------------------------------------------------------- scan item
__device__ void do_scan(const FusedArgs& a, int blk, uint32_t ep32, int* sh_wave_total,
                        int* sh_word)
{
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = lane_id();
    if (tid == 0) {
        Waiter wt;
        bool ok = true;
        while (ld_relaxed(&a.hdr->hist_done.v) < uint32_t(a.nTiles))
            if (!(ok = wt.tick(a.hdr, a.spin_limit))) break;
        sh_word[0] = ok;
    }
    __syncthreads();
    fence_acquire();
    if (!__builtin_amdgcn_readfirstlane(sh_word[0])) return;

    const BlockScan bs = block_scan(a.cnt, a.nCnt, blk, sh_wave_total);
    const uint64_t tag = uint64_t(ep32) << 32;
    if (wave == 0) {
        int exclusive = 0;
        if (blk == 0) {
            if (lane == 0) st_relaxed64(&a.status[0], tag | kStFlagInclusive | uint64_t(bs.total));
        } else {
            if (lane == 0) st_relaxed64(&a.status[blk], tag | kStFlagAggregate | uint64_t(bs.total));
            int look = blk - 1;
            Waiter wt;
            while (true) {
                const int j = look - lane;
                const uint64_t st = j >= 0 ? ld_relaxed64(&a.status[j]) : (tag | kStFlagInclusive);
                const bool ready = published(st, ep32) && ((st >> 30) & 3) != 0;
                if (ballot(!ready) != 0) {
                    if (!wt.tick(a.hdr, a.spin_limit)) break;
                    continue;
                }
                const uint64_t inc = ballot(((st >> 30) & 3) == 2);
                const int val = int(st & kStValueMask);
                if (inc != 0) {
                    const int first = __ffsll((unsigned long long)inc) - 1;
                    exclusive += wave_sum(lane <= first ? val : 0);
                    break;
                }
                exclusive += wave_sum(val);
                look -= kWave;
            }
            if (lane == 0)
                st_relaxed64(&a.status[blk],
                             tag | kStFlagInclusive | uint64_t(exclusive + bs.total));
        }
        if (lane == 0) sh_word[1] = exclusive;
    }
    __syncthreads();

    int run = sh_word[1] + bs.thread_excl;
    fence_release();                       // local_rank (acquired above) before the bases
#pragma unroll
    for (int q = 0; q < kScanPerThread; ++q) {
        const int i = bs.i0 + q;
        if (i < a.nCnt) {
            if (i % a.nTiles == 0) a.expert_offsets[i / a.nTiles] = run;
            st_relaxed64(&a.fbase[i], tag | uint32_t(run));
            run += bs.v[q];
            if (i == a.nCnt - 1) a.expert_offsets[a.E] = run;
        }
    }
}

// Positions of the picks of this wave's tokens: lane j < k of token slot i
// gets p[i] (or -1).  Polls the published bases; false on timeout.
__device__ __forceinline__ bool wave_positions(const FusedArgs& a, int t_first, uint32_t ep32,
                                               int (&p)[kTokPerWave], int64_t (&s)[kTokPerWave])
{
    const int lane = lane_id();
    uint64_t word[kTokPerWave];
    int e[kTokPerWave];
#pragma unroll
    for (int i = 0; i < kTokPerWave; ++i) {
        const int t = t_first + i;
        s[i] = int64_t(t) * a.k + lane;
        e[i] = (lane < a.k && t < a.T) ? a.idx[s[i]] : -1;
        word[i] = 0;
    }
    Waiter wt;
    while (true) {
        bool ready = true;
#pragma unroll
        for (int i = 0; i < kTokPerWave; ++i) {
            if (unsigned(e[i]) < unsigned(a.E) && !published(word[i], ep32)) {
                word[i] = ld_relaxed64(&a.fbase[int64_t(e[i]) * a.nTiles + s[i] / kTileSlots]);
                ready = ready && published(word[i], ep32);
            }
        }
        if (ballot(!ready) == 0) break;
        if (!wt.tick(a.hdr, a.spin_limit)) return false;
    }
    fence_acquire();                       // the ranks written by the hist items
#pragma unroll
    for (int i = 0; i < kTokPerWave; ++i) {
        p[i] = unsigned(e[i]) < unsigned(a.E) ? int(uint32_t(word[i])) + a.local_rank[s[i]] : -1;
        if (uint64_t(uint32_t(p[i])) >= uint64_t(a.S)) p[i] = -1;   // never address outside the rows
    }
    return true;
}

// ---------------------------------------------------------------- scatter item
__device__ void do_scatter(const FusedArgs& a, int item, uint64_t epoch) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = lane_id();
    const int t_first = item * kTokPerItem + wave * kTokPerWave;
    if (t_first >= a.T) return;
    int p[kTokPerWave];
    int64_t s[kTokPerWave];
    if (!wave_positions(a, t_first, uint32_t(epoch), p, s)) return;

    for (int i = 0; i < kTokPerWave; ++i) {
        const int t = t_first + i;
        if (t >= a.T) break;
        if (lane < a.k) a.pos[s[i]] = p[i];
        const char* src = reinterpret_cast<const char*>(a.x) + int64_t(t) * a.nvec * 16;
        // payload: 8 vectors per lane per round, then k streaming stores each
        for (int c0 = 0; c0 < a.nvec; c0 += kWave * 8) {
            u32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int vi = c0 + u * kWave + lane;
                if (vi < a.nvec) v[u] = load16(src + int64_t(vi) * 16);
            }
            for (int j = 0; j < a.k; ++j) {
                const int pj = __builtin_amdgcn_readlane(p[i], j);
                if (pj < 0) continue;
                char* row = reinterpret_cast<char*>(a.send_rows) + int64_t(pj) * a.stride;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int vi = c0 + u * kWave + lane;
                    if (vi < a.nvec) store16_nt(row + int64_t(vi) * 16, v[u]);
                }
            }
        }
        // trailer bytes 8..15: the slot's source index, then zero
        if (lane < a.k && p[i] >= 0) {
            uint64_t* tr = reinterpret_cast<uint64_t*>(a.send_rows + int64_t(p[i]) * a.stride +
                                                       a.trailer_off);
            tr[1] = uint64_t(uint32_t(s[i]));
        }
    }
    fence_release();                       // payloads + trailer tails before the flags
    for (int i = 0; i < kTokPerWave; ++i) {
        if (lane < a.k && p[i] >= 0 && t_first + i < a.T) {
            uint64_t* tr = reinterpret_cast<uint64_t*>(a.send_rows + int64_t(p[i]) * a.stride +
                                                       a.trailer_off);
            st_relaxed64(tr, epoch);
        }
    }
}

// ---------------------------------------------------------------- combine item
template <int KC>
__device__ void do_combine(const FusedArgs& a, int item, uint64_t epoch) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = lane_id();
    const int k = KC > 0 ? KC : a.k;
    const int t_first = item * kTokPerItem + wave * kTokPerWave;
    if (t_first >= a.T) return;
    int p[kTokPerWave];
    int64_t s[kTokPerWave];
    if (!wave_positions(a, t_first, uint32_t(epoch), p, s)) return;

    // wait for the k trailers of each token to carry this call's epoch
    Waiter wt;
    while (true) {
        bool ready = true;
#pragma unroll
        for (int i = 0; i < kTokPerWave; ++i) {
            if (lane < k && p[i] >= 0) {
                const uint64_t* tr = reinterpret_cast<const uint64_t*>(
                    a.send_rows + int64_t(p[i]) * a.stride + a.trailer_off);
                ready = ready && ld_relaxed64(tr) == epoch;
            }
        }
        if (ballot(!ready) == 0) break;
        if (!wt.tick(a.hdr, a.spin_limit)) return;
    }
    fence_acquire();                       // the rows' payloads

    const uint32_t S = uint32_t(a.S);
    const char* rows = reinterpret_cast<const char*>(a.send_rows);
    for (int i = 0; i < kTokPerWave; ++i) {
        const int t = t_first + i;
        if (t >= a.T) break;
        const float wl = lane < k ? a.w[int64_t(t) * k + lane] : 0.0f;
        char* dst = reinterpret_cast<char*>(a.out) + int64_t(t) * a.nvec * 16;
        constexpr int U = 2;
        for (int c0 = 0; c0 < a.nvec; c0 += kWave * U) {
            const int v0 = c0 + lane;
            if (c0 + kWave * U <= a.nvec) {
                const uint32_t off = uint32_t(v0) * 16u;
                float acc[U][8];
                if constexpr (KC > 0) {
                    u32x4 r[KC][U];
#pragma unroll
                    for (int j = 0; j < KC; ++j) {
                        const int pj = __builtin_amdgcn_readlane(p[i], j);
                        const char* src = rows + int64_t(pj < 0 ? 0 : pj) * a.stride + off;
#pragma unroll
                        for (int u = 0; u < U; ++u)
                            r[j][u] = uint32_t(pj) < S ? load16_nt(src + u * kWave * 16)
                                                       : u32x4{0, 0, 0, 0};
                    }
#pragma unroll
                    for (int j = 0; j < KC; ++j)
                        accumulate<U>(acc, r[j], __shfl(wl, j, kWave), j == 0);
                } else {
                    for (int j = 0; j < k; ++j) {
                        const int pj = __builtin_amdgcn_readlane(p[i], j);
                        const char* src = rows + int64_t(pj < 0 ? 0 : pj) * a.stride + off;
                        u32x4 r[U];
#pragma unroll
                        for (int u = 0; u < U; ++u)
                            r[u] = uint32_t(pj) < S ? load16_nt(src + u * kWave * 16)
                                                    : u32x4{0, 0, 0, 0};
                        accumulate<U>(acc, r, __shfl(wl, j, kWave), j == 0);
                    }
                }
                store_acc<U>(dst + off, acc);
            } else {
                for (int u = 0; u < U; ++u) {
                    const int vi = v0 + u * kWave;
                    const uint32_t off = uint32_t(vi < a.nvec ? vi : 0) * 16u;
                    float acc[1][8];
                    for (int j = 0; j < k; ++j) {
                        const int pj = __builtin_amdgcn_readlane(p[i], j);
                        const char* src = rows + int64_t(pj < 0 ? 0 : pj) * a.stride + off;
                        u32x4 r[1];
                        r[0] = (uint32_t(pj) < S && vi < a.nvec) ? load16_nt(src)
                                                                 : u32x4{0, 0, 0, 0};
                        accumulate<1>(acc, r, __shfl(wl, j, kWave), j == 0);
                    }
                    if (vi < a.nvec) store_acc<1>(dst + off, acc);
                }
            }
        }
    }
}

// ---------------------------------------------------------------- the launch
template <int KC>
__global__ __launch_bounds__(kBlock) void fused_kernel(FusedArgs a) {
    __shared__ int32_t hist[kWavesPerBlock][kMaxE];
    __shared__ int sh_wave_total[kWavesPerBlock];
    __shared__ int sh_word[2];
    __shared__ int sh_ticket;
    const int tid = threadIdx.x;
    const uint64_t epoch = a.hdr->epoch;          // constant during the call
    const int first_scan = a.nTiles;
    const int first_scatter = first_scan + a.nScan;
    const int first_combine = first_scatter + a.nItems;
    const int total = first_combine + a.nItems;

    // The barrier opens each round, BEFORE thread 0 claims the ticket: a
    // divergent thread-0 block must never follow another one (the end of a
    // hist item) with no barrier in between, or the compiler may merge the
    // two and build an inner loop that only lane 0 leaves -- the other 255
    // threads would then cycle on a stale ticket forever.  The ticket is made
    // wave-uniform so every branch on it is a scalar branch.
    while (true) {
        __syncthreads();                  // everyone has read the last ticket
        if (tid == 0) sh_ticket = int(fetch_add(&a.hdr->work_ticket.v, 1u));
        __syncthreads();
        const int ticket = __builtin_amdgcn_readfirstlane(sh_ticket);
        if (ticket >= total) break;
        if (ticket < first_scan) do_hist(a, ticket, hist);
        else if (ticket < first_scatter) do_scan(a, ticket - first_scan, uint32_t(epoch), sh_wave_total, sh_word);
        else if (ticket < first_combine) do_scatter(a, ticket - first_scatter, epoch);
        else do_combine<KC>(a, ticket - first_combine, epoch);
    }

    // Leave: the last workgroup out finishes the outputs and resets the state.
    fence_release();
    __syncthreads();
    if (tid == 0) sh_word[0] = fetch_add_acq_rel(&a.hdr->exit_count.v, 1u) == gridDim.x - 1;
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(sh_word[0])) return;
    fence_acquire();
    const int L = a.E / a.R;
    for (int e = tid; e < a.E; e += kBlock)
        a.expert_counts[e] = a.expert_offsets[e + 1] - a.expert_offsets[e];
    for (int r = tid; r <= a.R; r += kBlock) {
        a.rank_offsets[r] = a.expert_offsets[r * L];
        if (r < a.R) a.rank_counts[r] = a.expert_offsets[(r + 1) * L] - a.expert_offsets[r * L];
    }
    if (tid == 0) {
        WsHeader* h = a.hdr;
        uint32_t err = kDevOk;
        if (h->timeout.v) err = kDevTimeout;
        else if (a.expert_offsets[a.E] != a.S) err = kDevBadExpert;
        h->error = err;
        h->timeout.v = 0;
        h->work_ticket.v = 0;
        h->hist_done.v = 0;
        h->exit_count.v = 0;
        h->last_epoch = epoch;
        uint64_t next = epoch + 1;
        if (uint32_t(next) == 0) next += 1;       // the 32-bit tag is never 0
        h->epoch = next;
    }
}

__global__ void fused_init_kernel(WsHeader* hdr, uint64_t first_epoch) {
    if (threadIdx.x == 0) {
        hdr->magic = kFusedMagic;
        hdr->error = kDevOk;
        hdr->scan_ticket.v = 0;
        hdr->timeout.v = 0;
        hdr->work_ticket.v = 0;
        hdr->hist_done.v = 0;
        hdr->exit_count.v = 0;
        hdr->epoch = first_epoch;
        hdr->last_epoch = 0;
    }
}

int resident_grid(const void* kernel) {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    const int slot = dev < 64 ? dev : 63;
    if (cached[slot] > 0) return cached[slot];
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBlock, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    cached[slot] = per_cu * cus;
    return cached[slot];
}

}  // namespace

hipError_t launch_fused_init(void* ws, uint64_t first_epoch, hipStream_t s) {
    if (uint32_t(first_epoch) == 0) first_epoch += 1;
    EP_LAUNCH(fused_init_kernel, dim3(1), dim3(64), 0, s,
                       static_cast<WsHeader*>(ws), first_epoch);
    return hipGetLastError();
}

hipError_t launch_fused(const uint16_t* x, const int32_t* topk_idx, const float* topk_w,
                        int T, int H, int k, int E, int R, int32_t* expert_counts,
                        int32_t* expert_offsets, int32_t* rank_counts,
                        int32_t* rank_offsets, int32_t* pos, uint8_t* send_rows,
                        uint16_t* out, void* ws, uint32_t spin_limit, int grid,
                        hipStream_t s)
{
    const FusedPlan f = fused_plan(T, k, E);
    char* w = static_cast<char*>(ws);
    FusedArgs a{};
    a.x = x;
    a.idx = topk_idx;
    a.w = topk_w;
    a.T = T;
    a.k = k;
    a.E = E;
    a.R = R;
    a.nvec = H / 8;
    a.S = f.lay.S;
    a.nTiles = f.lay.nTiles;
    a.nCnt = f.lay.nCnt;
    a.nScan = f.lay.nScan;
    a.nItems = (T + kTokPerItem - 1) / kTokPerItem;
    a.stride = int64_t(fused_row_stride(H));
    a.trailer_off = int64_t(2) * H;
    a.expert_counts = expert_counts;
    a.expert_offsets = expert_offsets;
    a.rank_counts = rank_counts;
    a.rank_offsets = rank_offsets;
    a.pos = pos;
    a.send_rows = send_rows;
    a.out = out;
    a.hdr = reinterpret_cast<WsHeader*>(w);
    a.cnt = reinterpret_cast<int32_t*>(w + f.lay.off_cnt);
    a.local_rank = reinterpret_cast<int32_t*>(w + f.lay.off_rank);
    a.status = reinterpret_cast<uint64_t*>(w + f.off_status64);
    a.fbase = reinterpret_cast<uint64_t*>(w + f.off_fbase);
    a.spin_limit = spin_limit ? spin_limit : kDefaultSpinLimit;

    const void* kern = k == 8 ? reinterpret_cast<const void*>(&fused_kernel<8>)
                              : reinterpret_cast<const void*>(&fused_kernel<0>);
    const int items = a.nTiles + a.nScan + 2 * a.nItems;
    int g = grid > 0 ? grid : resident_grid(kern);
    if (g > items) g = items;
    if (k == 8)
        EP_LAUNCH((fused_kernel<8>), dim3(g), dim3(kBlock), 0, s, a);
    else
        EP_LAUNCH((fused_kernel<0>), dim3(g), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace ep
