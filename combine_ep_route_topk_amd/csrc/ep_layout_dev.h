// ep_layout_dev.h -- device building blocks of the dispatch layout shared by
// the three-launch layout (layout.hip) and the persistent fused mode
// (fused.hip): the per-tile histogram with stable ranks, and a block-wide
// exclusive scan of ITEMS counters.
#pragma once

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

constexpr int kWavesPerBlock = kBlock / kWave;                          // 4
constexpr int kChunksPerWave = kTileSlots / (kWavesPerBlock * kWave);   // 4
static_assert(kChunksPerWave * kWavesPerBlock * kWave == kTileSlots, "tile split");

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

// Histogram of one tile of kTileSlots slots (UBEP sec. 2.3: per-expert token
// counts) plus each slot's stable rank among the tile's slots of the same
// expert (StrataCL appendix: token-local offsets).  Each wave walks its
// 64-slot chunks in slot order; lanes holding the same expert find each other
// with ceil(log2 E) ballots; the group's lowest lane adds the group size to
// the wave's private LDS counter (LDS atomic, returns the old value) and
// broadcasts the old value, which is the base rank of the group.  Waves then
// turn their private counts into per-wave offsets.  Deterministic: no result
// depends on the order in which atomics land.
// Writes cnt[e * nTiles + tile] for every e < E and local_rank[s] for every
// valid slot of the tile, with agent-coherent stores: once the wave's stores
// have completed they are visible on every XCD, so a persistent caller can
// publish "tile done" after a wait for its own stores instead of an L2
// write-back.  `hist` is the block's LDS scratch.
// The LDS part of hist_tile: after it, hist[w][e] holds wave w's exclusive
// offset among the tile's slots of expert e (waves in order), key[c] / rank[c]
// the expert (-1 if none) and in-wave rank of this lane's slot in chunk c, and
// -- where given -- cnt[e * nTiles + tile] (agent-coherent store) and
// sh_tot[e] (LDS) the tile's count of expert e.
__device__ __forceinline__ void tile_ranks(const int32_t* __restrict__ topk_idx, int64_t S,
                                           int E, int nTiles, int tile,
                                           int32_t* __restrict__ cnt, int* sh_tot,
                                           int32_t (*hist)[kMaxE],
                                           int (&key)[kChunksPerWave],
                                           int (&rank)[kChunksPerWave])
{
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = lane_id();
    const int64_t wave_first =
        int64_t(tile) * kTileSlots + int64_t(wave) * kChunksPerWave * kWave;

    // All chunks' slot ids are loaded first (their latency overlaps the
    // counter reset), each from a clamped in-bounds address (slot 0 for a
    // slot past S, then dropped): a guarded load would become a branch with a
    // full memory wait inside, and the chunks' loads would go out one round
    // trip at a time.
    int ids[kChunksPerWave];
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) {
        const int64_t s = wave_first + c * kWave + lane;
        ids[c] = topk_idx[s < S ? s : 0];
    }

    for (int i = tid; i < kWavesPerBlock * E; i += kBlock) hist[i / E][i % E] = 0;
    __syncthreads();

    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) {
        const int64_t s = wave_first + c * kWave + lane;
        const int e = s < S ? ids[c] : -1;
        const bool valid = unsigned(e) < unsigned(E);
        uint64_t peers = ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t bal = ballot(bit);
            peers &= bit ? bal : ~bal;
        }
        const uint64_t below = peers & lanes_below();
        int old = 0;
        if (valid && below == 0) old = atomicAdd(&hist[wave][e], popc64(peers));
        const int leader = valid ? __ffsll((unsigned long long)peers) - 1 : lane;
        const int base = __shfl(old, leader, kWave);
        key[c] = valid ? e : -1;
        rank[c] = base + popc64(below);
    }
    __syncthreads();

    for (int e = tid; e < E; e += kBlock) {
        int run = 0;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) {
            const int c = hist[w][e];
            hist[w][e] = run;
            run += c;
        }
        if (cnt)
            st_relaxed(reinterpret_cast<uint32_t*>(&cnt[int64_t(e) * nTiles + tile]),
                       uint32_t(run));
        if (sh_tot) sh_tot[e] = run;
    }
    __syncthreads();
}

__device__ __forceinline__ void hist_tile(const int32_t* __restrict__ topk_idx, int64_t S,
                                          int E, int nTiles, int tile,
                                          int32_t* __restrict__ cnt,
                                          int32_t* __restrict__ local_rank,
                                          int32_t (*hist)[kMaxE])
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = lane_id();
    int key[kChunksPerWave];
    int rank[kChunksPerWave];
    tile_ranks(topk_idx, S, E, nTiles, tile, cnt, nullptr, hist, key, rank);
    const int64_t wave_first =
        int64_t(tile) * kTileSlots + int64_t(wave) * kChunksPerWave * kWave;
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) {
        const int64_t s = wave_first + c * kWave + lane;
        if (key[c] >= 0)
            st_relaxed(reinterpret_cast<uint32_t*>(&local_rank[s]),
                       uint32_t(hist[wave][key[c]] + rank[c]));
    }
}

// Block-wide scan of the ITEMS counters of scan block `blk`: loads
// v[q] = cnt[i0 + q] (0 past nCnt), as 16-byte vectors when nCnt % 4 == 0,
// and returns this thread's
// exclusive offset inside the block and the block total.  `sh_wave_total`
// is LDS scratch.
template <int ITEMS>
struct BlockScan {
    static constexpr int kPer = ITEMS / kBlock;      // counters per thread
    static_assert(kPer * kBlock == ITEMS && kPer % 4 == 0, "scan split");
    int v[kPer];
    int i0;
    int thread_excl;
    int total;
};

template <int ITEMS>
__device__ __forceinline__ BlockScan<ITEMS> block_scan(const int32_t* __restrict__ cnt, int nCnt,
                                                       int blk, int* sh_wave_total)
{
    constexpr int kScanPerThread = BlockScan<ITEMS>::kPer;
    BlockScan<ITEMS> r;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = lane_id();
    r.i0 = blk * ITEMS + tid * kScanPerThread;
    int tsum = 0;
    // Every load is unconditional, from a clamped in-bounds address (counter
    // 0) whose value is then dropped: a guarded load becomes a branch with a
    // full memory wait inside, and the thread's loads would go out one round
    // trip apart instead of together.
    if (nCnt % 4 == 0) {                   // a 4-group is wholly inside or outside
#pragma unroll
        for (int m = 0; m < kScanPerThread / 4; ++m) {
            const int i = r.i0 + 4 * m;
            const bool in = i < nCnt;
            const int4 x = *reinterpret_cast<const int4*>(cnt + (in ? i : 0));
            r.v[4 * m] = in ? x.x : 0;
            r.v[4 * m + 1] = in ? x.y : 0;
            r.v[4 * m + 2] = in ? x.z : 0;
            r.v[4 * m + 3] = in ? x.w : 0;
        }
    } else {
#pragma unroll
        for (int q = 0; q < kScanPerThread; ++q) {
            const int i = r.i0 + q;
            const int x = cnt[i < nCnt ? i : 0];
            r.v[q] = i < nCnt ? x : 0;
        }
    }
#pragma unroll
    for (int q = 0; q < kScanPerThread; ++q) tsum += r.v[q];
    const int incl = wave_inclusive_sum(tsum);
    if (lane == kWave - 1) sh_wave_total[wave] = incl;
    __syncthreads();
    int wave_off = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
        if (w < wave) wave_off += sh_wave_total[w];
        total += sh_wave_total[w];
    }
    r.thread_excl = wave_off + incl - tsum;
    r.total = total;
    return r;
}

}  // namespace ep
