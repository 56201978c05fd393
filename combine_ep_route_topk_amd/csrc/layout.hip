// layout.hip -- dispatch layout on gfx950: per-expert counts, prefix-sum
// offsets and a stable position for every (token, pick) slot.
//
// UBEP sec. 2.3 / Fig. 2: per-expert token counts, then offset calculation,
// then a contiguous per-expert reordering; UBEP sec. 3.2: prefix sums of the
// counts give each expert's offset; StrataCL appendix "Hierarchical Workload
// Partitioning for MoE Dispatch/Combine": the placement metadata is the
// destination expert, per-expert counts, prefix-sum offsets and token-local
// offsets.  The slots s = t*k + j are ordered expert-major and, inside one
// expert, by ascending s, i.e. a stable counting sort.
//
// Three launches on one stream (the kernel boundaries are the barriers):
//   1. hist  -- one workgroup per tile of kTileSlots slots.  Each wave walks
//      its 64-slot chunks in order; lanes with the same expert find each other
//      with ceil(log2 E) ballots (wave multisplit), the group's lowest lane
//      adds the group size to the wave's private LDS counter with an LDS
//      atomic and broadcasts the old value: that is the slots' rank.  Ranks
//      are therefore deterministic and stable; no atomic order is observed.
//      Per-wave counts are then turned into per-wave offsets, giving
//      cnt[e][tile] (expert-major) and each slot's rank inside (tile, e).
//   2. scan  -- exclusive prefix sum of cnt flattened expert-major, single
//      pass with decoupled look-back: blocks take ids from an atomic ticket,
//      publish their aggregate, then look back over predecessors 64 at a time.
//      Each 32-bit status word packs a 2-bit flag with a 30-bit value, so one
//      relaxed atomic load sees both and no fence is needed: the status word
//      IS the data.  The result base[e][tile] is the first send row of
//      expert e's slots from that tile; base[e][0] is expert e's offset.
//   3. pos   -- pos[s] = base[e][tile(s)] + rank(s); slot_src[pos[s]] = s;
//      block 0 derives the per-expert / per-rank counts and offsets.
// When the counters are few (nCnt <= kRedundantScanMax: 32 K, i.e. 128 KiB),
// steps 2 and 3 are one launch instead: every tile's workgroup reads all of
// cnt (from L2) and computes the bases of its own tile itself,
//   base[e][tile] = offset[e] + sum_{t < tile} cnt[e][t],
//   offset = exclusive scan over e of sum_t cnt[e][t],
// which costs each workgroup a 32 KiB read at T=4096, k=8, E=256 and saves a
// launch and the look-back (measured on MI355X: layout 14.3 -> ~10 us).
// A layout of a single tile runs all of it in one workgroup and one launch.
#include <atomic>
#include <mutex>

#include "ep_device.h"
#include "ep_internal.h"
#include "ep_layout_dev.h"

namespace ep {
namespace {

constexpr uint32_t kFlagAggregate = 1u << 30;
constexpr uint32_t kFlagInclusive = 2u << 30;
constexpr uint32_t kValueMask = (1u << 30) - 1;

__global__ __launch_bounds__(kBlock) void layout_hist_kernel(
    const int32_t* __restrict__ topk_idx, int64_t S, int E, int nTiles, int nScan,
    int32_t* __restrict__ cnt, int32_t* __restrict__ local_rank,
    uint32_t* __restrict__ status, WsHeader* __restrict__ hdr)
{
    __shared__ int32_t hist[kWavesPerBlock][kMaxE];
    // Reset the scan state for this call; the scan kernel runs after this
    // kernel completes (stream order).
    if (blockIdx.x == 0) {
        for (int i = threadIdx.x; i < nScan; i += kBlock) status[i] = 0;
        if (threadIdx.x == 0) {
            hdr->scan_ticket.v = 0;
            hdr->timeout.v = 0;
        }
    }
    hist_tile(topk_idx, S, E, nTiles, blockIdx.x, cnt, local_rank, hist);
}

__global__ __launch_bounds__(kBlock) void layout_scan_kernel(
    const int32_t* __restrict__ cnt, int nCnt, int nTiles, int E,
    int32_t* __restrict__ base, int32_t* __restrict__ expert_offsets,
    uint32_t* __restrict__ status, WsHeader* __restrict__ hdr, uint32_t spin_limit)
{
    __shared__ int sh_block;
    __shared__ int sh_wave_total[kWavesPerBlock];
    __shared__ int sh_exclusive;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = lane_id();

    // Ticket order = order in which blocks started, so every predecessor a
    // block waits for is already running (forward progress).
    if (tid == 0) sh_block = int(fetch_add(&hdr->scan_ticket.v, 1u));
    __syncthreads();
    const int blk = sh_block;
    const BlockScan<kScanItems> bs = block_scan<kScanItems>(cnt, nCnt, blk, sh_wave_total);

    if (wave == 0) {
        int exclusive = 0;
        if (blk == 0) {
            if (lane == 0) st_relaxed(&status[0], kFlagInclusive | uint32_t(bs.total));
        } else {
            if (lane == 0) st_relaxed(&status[blk], kFlagAggregate | uint32_t(bs.total));
            int look = blk - 1;
            uint32_t spins = 0;
            while (true) {
                const int j = look - lane;
                const uint32_t st = j >= 0 ? ld_relaxed(&status[j]) : kFlagInclusive;
                if (ballot((st >> 30) == 0) != 0) {       // a predecessor not published yet
                    if (++spins > spin_limit) {
                        if (lane == 0) st_relaxed(&hdr->timeout.v, 1u);
                        break;
                    }
                    backoff();
                    continue;
                }
                const uint64_t inc = ballot((st >> 30) == 2);
                const int val = int(st & kValueMask);
                if (inc != 0) {
                    const int first = __ffsll((unsigned long long)inc) - 1;
                    exclusive += wave_sum(lane <= first ? val : 0);
                    break;
                }
                exclusive += wave_sum(val);
                look -= kWave;
            }
            if (lane == 0)
                st_relaxed(&status[blk], kFlagInclusive | uint32_t(exclusive + bs.total));
        }
        if (lane == 0) sh_exclusive = exclusive;
    }
    __syncthreads();

    int run = sh_exclusive + bs.thread_excl;
    // counter i is (expert i / nTiles, tile i % nTiles): one division per
    // thread, then the tile steps along
    int e = bs.i0 / nTiles;
    int tile = bs.i0 - e * nTiles;
#pragma unroll
    for (int q = 0; q < BlockScan<kScanItems>::kPer; ++q) {
        const int i = bs.i0 + q;
        if (i < nCnt) {
            base[i] = run;
            if (tile == 0) expert_offsets[e] = run;
            run += bs.v[q];
            if (i == nCnt - 1) expert_offsets[E] = run;
        }
        if (++tile == nTiles) {
            tile = 0;
            ++e;
        }
    }
}

__global__ __launch_bounds__(kBlock) void layout_pos_kernel(
    const int32_t* __restrict__ topk_idx, int64_t S, int E, int R, int nTiles,
    const int32_t* __restrict__ base, const int32_t* __restrict__ local_rank,
    int32_t* __restrict__ expert_counts, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ rank_counts, int32_t* __restrict__ rank_offsets,
    int32_t* __restrict__ pos, int32_t* __restrict__ slot_src, WsHeader* __restrict__ hdr,
    int64_t expect)
{
    const int64_t s = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    if (s < S) {
        const int e = topk_idx[s];
        const int lr = local_rank[s];     // loaded with the id, not after it
        if (unsigned(e) < unsigned(E)) {
            const int p = base[int64_t(e) * nTiles + s / kTileSlots] + lr;
            pos[s] = p;
            if (slot_src) slot_src[p] = int(s);
        } else {
            pos[s] = -1;
        }
    }
    if (blockIdx.x == 0) {
        const int L = E / R;
        for (int e = threadIdx.x; e < E; e += kBlock)
            expert_counts[e] = expert_offsets[e + 1] - expert_offsets[e];
        for (int r = threadIdx.x; r <= R; r += kBlock) {
            rank_offsets[r] = expert_offsets[r * L];
            if (r < R) rank_counts[r] = expert_offsets[(r + 1) * L] - expert_offsets[r * L];
        }
        if (threadIdx.x == 0) {
            uint32_t err = kDevOk;
            if (hdr->timeout.v) err = kDevTimeout;
            else if (expect >= 0 && expert_offsets[E] != expect) err = kDevBadExpert;
            hdr->error = err;
            hdr->magic = kLayoutMagic;
        }
    }
}

// Scan + positions of one tile by one workgroup (see the header).  Experts
// are split contiguously, kExpPerThread per thread, so the scan over experts
// is a thread-local run plus one block-wide scan.
constexpr int kExpPerThread = kMaxE / kBlock;    // 4
// Counters per expert per load round.  32 (one round at T*k <= 32768) was
// slower on MI355X: scanpos 5.6 -> 5.9 us at T=4096, 11.9 -> 13.1 us at
// T=16384 (k=8, E=256).
constexpr int kTilesPerRound = 16;
static_assert(kExpPerThread * kBlock == kMaxE, "expert split");
__device__ __forceinline__ void scanpos_tile(
    int tile, const int32_t* __restrict__ topk_idx, int64_t S, int E, int R, int nTiles,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ local_rank,
    int32_t* __restrict__ expert_counts, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ rank_counts, int32_t* __restrict__ rank_offsets,
    int32_t* __restrict__ pos, int32_t* __restrict__ slot_src, WsHeader* __restrict__ hdr,
    int64_t expect)
{
    __shared__ int sh_off[kMaxE + 1];      // expert offsets (exclusive scan)
    __shared__ int sh_base[kMaxE];         // first row of (expert, this tile)
    __shared__ int sh_wave_total[kWavesPerBlock];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = lane_id();

    // this thread's slots of the tile: their ids and ranks are loaded first,
    // so those loads overlap the counter loads below.  Every load in this
    // kernel is unconditional, from a clamped in-bounds address whose value is
    // then dropped (slot 0 for a slot past S; a rank whose slot has no valid
    // expert is never used): a guarded load becomes a branch with a full
    // memory wait inside, which would put the loads one round trip apart.
    constexpr int kSlotsPerThread = kTileSlots / kBlock;
    int se[kSlotsPerThread], sr[kSlotsPerThread];
#pragma unroll
    for (int u = 0; u < kSlotsPerThread; ++u) {
        const int64_t s = int64_t(tile) * kTileSlots + u * kBlock + tid;
        const int64_t sc = s < S ? s : 0;
        se[u] = topk_idx[sc];
        sr[u] = local_rank[sc];
    }
#pragma unroll
    for (int u = 0; u < kSlotsPerThread; ++u) {
        const int64_t s = int64_t(tile) * kTileSlots + u * kBlock + tid;
        if (s >= S) se[u] = -1;
    }

    // per expert: its total over all tiles and its count before this tile.
    // Each round issues all its loads (kExpPerThread experts x kTilesPerRound
    // counters, as 16-byte vectors) before adding any: the counters come from
    // L2, and a loop of dependent load-add steps would pay one L2 latency per
    // step.
    int tot[kExpPerThread], pre[kExpPerThread];
#pragma unroll
    for (int q = 0; q < kExpPerThread; ++q) tot[q] = pre[q] = 0;
    const int e0 = tid * kExpPerThread;
    if (nTiles % 4 == 0) {                      // rows are 16-byte aligned
        for (int t0 = 0; t0 < nTiles; t0 += kTilesPerRound) {
            int4 c[kExpPerThread][kTilesPerRound / 4];
#pragma unroll
            for (int q = 0; q < kExpPerThread; ++q)
#pragma unroll
                for (int m = 0; m < kTilesPerRound / 4; ++m) {
                    const int t = t0 + 4 * m;
                    const bool in = e0 + q < E && t < nTiles;
                    const int4 x =
                        *reinterpret_cast<const int4*>(cnt + (in ? int64_t(e0 + q) * nTiles + t : 0));
                    const int mk = in ? -1 : 0;       // a mask, not a branch
                    c[q][m] = make_int4(x.x & mk, x.y & mk, x.z & mk, x.w & mk);
                }
#pragma unroll
            for (int q = 0; q < kExpPerThread; ++q)
#pragma unroll
                for (int m = 0; m < kTilesPerRound / 4; ++m) {
                    const int t = t0 + 4 * m;
                    tot[q] += c[q][m].x + c[q][m].y + c[q][m].z + c[q][m].w;
                    pre[q] += (t < tile ? c[q][m].x : 0) + (t + 1 < tile ? c[q][m].y : 0) +
                              (t + 2 < tile ? c[q][m].z : 0) + (t + 3 < tile ? c[q][m].w : 0);
                }
        }
    } else {
        for (int t0 = 0; t0 < nTiles; t0 += 4) {
            int c[kExpPerThread][4];
#pragma unroll
            for (int q = 0; q < kExpPerThread; ++q)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const bool in = e0 + q < E && t0 + m < nTiles;
                    c[q][m] = cnt[in ? int64_t(e0 + q) * nTiles + t0 + m : 0] & (in ? -1 : 0);
                }
#pragma unroll
            for (int q = 0; q < kExpPerThread; ++q)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    tot[q] += c[q][m];
                    pre[q] += t0 + m < tile ? c[q][m] : 0;
                }
        }
    }
    int tsum = 0;
#pragma unroll
    for (int q = 0; q < kExpPerThread; ++q) tsum += tot[q];
    // block-wide exclusive scan of the per-thread totals
    const int incl = wave_inclusive_sum(tsum);
    if (lane == kWave - 1) sh_wave_total[wave] = incl;
    __syncthreads();
    int run = incl - tsum;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w)
        if (w < wave) run += sh_wave_total[w];
#pragma unroll
    for (int q = 0; q < kExpPerThread; ++q) {
        const int e = tid * kExpPerThread + q;
        if (e < E) {
            sh_off[e] = run;
            sh_base[e] = run + pre[q];
            if (tile == 0) {
                expert_offsets[e] = run;
                expert_counts[e] = tot[q];
            }
            if (e == E - 1) {
                sh_off[E] = run + tot[q];
                if (tile == 0) expert_offsets[E] = run + tot[q];
            }
        }
        run += tot[q];
    }
    __syncthreads();

    if (tile == 0) {
        const int L = E / R;
        for (int r = tid; r <= R; r += kBlock) {
            rank_offsets[r] = sh_off[r * L];
            if (r < R) rank_counts[r] = sh_off[(r + 1) * L] - sh_off[r * L];
        }
        if (tid == 0) {
            hdr->error = expect >= 0 && sh_off[E] != expect ? kDevBadExpert : kDevOk;
            hdr->magic = kLayoutMagic;
        }
    }

    // positions of this tile's slots
#pragma unroll
    for (int u = 0; u < kSlotsPerThread; ++u) {
        const int64_t s = int64_t(tile) * kTileSlots + u * kBlock + tid;
        if (s >= S) break;
        const int e = se[u];
        if (unsigned(e) < unsigned(E)) {
            const int p = sh_base[e] + sr[u];
            pos[s] = p;
            if (slot_src) slot_src[p] = int(s);
        } else {
            pos[s] = -1;
        }
    }
}

__global__ __launch_bounds__(kBlock) void layout_scanpos_kernel(
    const int32_t* __restrict__ topk_idx, int64_t S, int E, int R, int nTiles,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ local_rank,
    int32_t* __restrict__ expert_counts, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ rank_counts, int32_t* __restrict__ rank_offsets,
    int32_t* __restrict__ pos, int32_t* __restrict__ slot_src, WsHeader* __restrict__ hdr,
    int64_t expect)
{
    scanpos_tile(blockIdx.x, topk_idx, S, E, R, nTiles, cnt, local_rank, expert_counts,
                 expert_offsets, rank_counts, rank_offsets, pos, slot_src, hdr, expect);
}

// A layout of one tile (T*k <= kTileSlots, e.g. a decode batch): histogram,
// scan and positions in ONE workgroup and one launch, with nothing in global
// memory between the steps -- the per-expert totals and each wave's offsets
// stay in LDS and every slot's expert and in-wave rank in registers, so the
// slot ids are read once and no counter or rank makes a round trip.
__global__ __launch_bounds__(kBlock) void layout_single_kernel(
    const int32_t* __restrict__ topk_idx, int64_t S, int E, int R,
    int32_t* __restrict__ expert_counts, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ rank_counts, int32_t* __restrict__ rank_offsets,
    int32_t* __restrict__ pos, int32_t* __restrict__ slot_src, WsHeader* __restrict__ hdr,
    int64_t expect)
{
    __shared__ int32_t hist[kWavesPerBlock][kMaxE];
    __shared__ int sh_tot[kMaxE];
    __shared__ int sh_off[kMaxE + 1];
    __shared__ int sh_wave_total[kWavesPerBlock];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = lane_id();
    int key[kChunksPerWave];
    int rank[kChunksPerWave];
    tile_ranks(topk_idx, S, E, 1, 0, nullptr, sh_tot, hist, key, rank);

    // exclusive scan of the totals over the experts, kExpPerThread per thread
    int tot[kExpPerThread];
    int tsum = 0;
#pragma unroll
    for (int q = 0; q < kExpPerThread; ++q) {
        const int e = tid * kExpPerThread + q;
        tot[q] = e < E ? sh_tot[e] : 0;
        tsum += tot[q];
    }
    const int incl = wave_inclusive_sum(tsum);
    if (lane == kWave - 1) sh_wave_total[wave] = incl;
    __syncthreads();
    int run = incl - tsum;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w)
        if (w < wave) run += sh_wave_total[w];
#pragma unroll
    for (int q = 0; q < kExpPerThread; ++q) {
        const int e = tid * kExpPerThread + q;
        if (e < E) {
            sh_off[e] = run;
            expert_offsets[e] = run;
            expert_counts[e] = tot[q];
            if (e == E - 1) {
                sh_off[E] = run + tot[q];
                expert_offsets[E] = run + tot[q];
            }
        }
        run += tot[q];
    }
    __syncthreads();
    const int L = E / R;
    for (int r = tid; r <= R; r += kBlock) {
        rank_offsets[r] = sh_off[r * L];
        if (r < R) rank_counts[r] = sh_off[(r + 1) * L] - sh_off[r * L];
    }
    if (tid == 0) {
        hdr->error = expect >= 0 && sh_off[E] != expect ? kDevBadExpert : kDevOk;
        hdr->magic = kLayoutMagic;
    }
    // positions: the expert's offset, the wave's offset inside the expert,
    // the slot's rank inside the wave
    const int64_t wave_first = int64_t(wave) * kChunksPerWave * kWave;
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) {
        const int64_t s = wave_first + c * kWave + lane;
        if (s >= S) continue;
        if (key[c] >= 0) {
            const int p = sh_off[key[c]] + hist[wave][key[c]] + rank[c];
            pos[s] = p;
            if (slot_src) slot_src[p] = int(s);
        } else {
            pos[s] = -1;
        }
    }
}

}  // namespace

// The workspace of ep_dispatch_layout_noalloc: a file-scope device array, so
// no call allocates.  Each GPU the library runs on holds its own copy at its
// own address; host code never passes this name to a kernel (on the host it
// is only a stand-in for the symbol), it passes the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kLayoutScratchBytes];

hipError_t layout_scratch(void** ptr)
{
    constexpr int kMaxDevices = 64;
    static std::atomic<void*> addr[kMaxDevices];
    static std::mutex lookup;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> hold(lookup);
        p = addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_dispatch_layout(const int32_t* topk_idx, int T, int k, int E, int R,
                                  int32_t* expert_counts, int32_t* expert_offsets,
                                  int32_t* rank_counts, int32_t* rank_offsets,
                                  int32_t* pos, int32_t* slot_src, void* ws, hipStream_t s)
{
    return launch_dispatch_layout_skips(topk_idx, T, k, E, R, expert_counts, expert_offsets,
                                        rank_counts, rank_offsets, pos, slot_src, ws,
                                        int64_t(T) * k, s);
}

hipError_t launch_dispatch_layout_skips(const int32_t* topk_idx, int T, int k, int E, int R,
                                        int32_t* expert_counts, int32_t* expert_offsets,
                                        int32_t* rank_counts, int32_t* rank_offsets,
                                        int32_t* pos, int32_t* slot_src, void* ws,
                                        int64_t expect, hipStream_t s)
{
    const LayoutPlan p = layout_plan(T, k, E);
    char* w = static_cast<char*>(ws);
    WsHeader* hdr = reinterpret_cast<WsHeader*>(w);
    uint32_t* status = reinterpret_cast<uint32_t*>(w + p.off_status);
    int32_t* cnt = reinterpret_cast<int32_t*>(w + p.off_cnt);
    int32_t* base = reinterpret_cast<int32_t*>(w + p.off_base);
    int32_t* rank = reinterpret_cast<int32_t*>(w + p.off_rank);

    if (p.nTiles == 1) {
        EP_LAUNCH(layout_single_kernel, dim3(1), dim3(kBlock), 0, s, topk_idx, p.S, E, R,
                  expert_counts, expert_offsets, rank_counts, rank_offsets, pos, slot_src, hdr,
                  expect);
        return hipGetLastError();
    }
    EP_LAUNCH(layout_hist_kernel, dim3(p.nTiles), dim3(kBlock), 0, s,
                       topk_idx, p.S, E, p.nTiles, p.nScan, cnt, rank, status, hdr);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (p.nCnt <= kRedundantScanMax) {
        EP_LAUNCH(layout_scanpos_kernel, dim3(p.nTiles), dim3(kBlock), 0, s,
                  topk_idx, p.S, E, R, p.nTiles, cnt, rank, expert_counts, expert_offsets,
                  rank_counts, rank_offsets, pos, slot_src, hdr, expect);
        return hipGetLastError();
    }
    EP_LAUNCH(layout_scan_kernel, dim3(p.nScan), dim3(kBlock), 0, s,
                       cnt, p.nCnt, p.nTiles, E, base, expert_offsets, status, hdr,
                       kDefaultSpinLimit);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int grid = int((p.S + kBlock - 1) / kBlock);
    EP_LAUNCH(layout_pos_kernel, dim3(grid), dim3(kBlock), 0, s,
                       topk_idx, p.S, E, R, p.nTiles, base, rank, expert_counts,
                       expert_offsets, rank_counts, rank_offsets, pos, slot_src, hdr, expect);
    return hipGetLastError();
}

}  // namespace ep
