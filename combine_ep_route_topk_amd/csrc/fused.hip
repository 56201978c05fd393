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
//             three-launch layout), then hist_done += 1 (release).  A layout
//             of one tile is a single item instead, which also scans the
//             counts and publishes the bases (no scan items).
//   [scan]    one per kFusedScanItems counters: waits for hist_done == nTiles
//             (an event counter with a static threshold), block scan, then
//             decoupled look-back over 64-bit status words that carry the
//             call's epoch next to flag and value, then publishes every
//             base as a 64-bit word (epoch << 32 | base): the base value is
//             its own readiness flag.
//   [scatter] ST tokens (2 or 4): wave 0 polls the base words of the item's
//             picks and puts the positions in LDS; the waves of a token
//             (4 / ST) copy one share of its row each into its k send rows with
//             agent-coherent streaming stores; every wave waits for its
//             stores to complete, and after a barrier wave 0 writes pos and
//             {slot_src, 0} into the rows' trailers, then the 64-bit epoch.
//   [combine] kCombTok tokens: wave 0 waits for the event words of the
//             scatter items of its tokens (one epoch-tagged word per item),
//             reads the positions those items wrote to pos, acquire-polls the
//             rows' trailers until they hold this call's epoch; after a
//             barrier each wave reduces one token's k rows with the same fp32
//             arithmetic as ep_combine, up to kCombBatch row segments before
//             it stores any of them.
//   A batch with fewer scatter items than workgroups splits the rows of each
//   scatter and combine item into parts (item-event mode; an event word per
//   part), so that its few tokens still spread over the GPU.
// A row's trailer is its flag: on gfx950 a 64-bit aligned store is
// single-copy atomic but a 14 KiB row is not, hence payload -> release ->
// trailer, and trailer -> acquire -> payload on the reading side.  An
// agent-scope release FENCE writes back the whole L2 of the XCD (a first
// version that fenced once per scatter item took 404 us a call at T=4096,
// H=7168, k=8), so the scatter side releases the way an agent-scope atomic
// store does instead: the
// payload is stored agent-coherent (sc1), each wave waits for its stores to
// complete, then the flags are stored.  The combine side keeps one acquire
// fence (an L2 invalidate, cheap) per item.
//
// Scatter items are small (2 or 4 tokens) and outnumber the resident workgroups
// at the shapes that matter, so the first ticket of almost every workgroup is
// layout or scatter work: no workgroup sits on a combine item waiting for
// rows that nobody is writing yet.
//
// Every wait is bounded by spin_limit polling rounds; an expired wait sets
// the workspace's timeout word and every later wait gives up soon after, so
// the grid always drains.  The workgroup whose final ticket claim is the last
// of all finishes the per-expert / per-rank counts, records the error word
// and resets the counters and the epoch for the next call (the workspace is
// reused without a memset).
#include <atomic>

#include "ep_combine_dev.h"
#include "ep_device.h"
#include "ep_internal.h"
#include "ep_layout_dev.h"

namespace ep {
namespace {

// Tokens per scatter item (ST, a template parameter of the kernel): 2, two
// waves per token, each half of the row; or 4, one wave per token and row.
// launch_fused picks 4 for rows of at most 8 KiB and for a small batch split
// into row parts, 2 otherwise.  Measured on MI355X, fused call, 4 tokens
// everywhere against 2: T=4096, H=4096 112.1-113.5 -> 109.8-110.0 us (item
// events); T=128, H=7168 26.5-26.7 -> 24.9 us (item events) but 27.0-27.2 ->
// 30.0-30.4 us (row flags); T=4096, H=7168 183.2-184.1 -> 186.2-188.0 us and
// T=16384, H=7168 720.8-722.8 -> 736.0-736.4 us.  With the rule, against 2
// everywhere: T=4096, H=4096 110.8-111.7 -> 108.2-110.7 us (item events),
// checksum 114.1 -> 108.8-109.3, sentinel 116.3-116.7 -> 111.0-111.4; T=128
// 26.1-26.2 -> 24.4-24.5 us (item events); the other shapes unchanged.
constexpr int kCombTok = kWavesPerBlock;       // tokens per combine item (1 wave each)
static_assert(kWavesPerBlock % kCombTok == 0, "whole waves per combine token");
constexpr int kScatU = 7;                      // 16-byte vectors per lane per row segment
constexpr int kMaxItemPicks = kCombTok * kMaxK;
constexpr int kPickRounds = kMaxItemPicks / kWave;   // lanes cover the picks in <= 4 rounds
constexpr uint64_t kStFlagAggregate = uint64_t(1) << 30;
constexpr uint64_t kStFlagInclusive = uint64_t(2) << 30;
constexpr uint64_t kStValueMask = (uint64_t(1) << 30) - 1;

struct FusedArgs {
    const uint16_t* x;
    const int32_t* idx;
    const float* w;
    int T, k, E, R, nvec;
    int64_t S;
    int nTiles, nCnt, nScan, nScat, nComb;
    int parts;                            // row parts per scatter / combine item (item events)
    int t_keep;                           // tokens from here on store their rows cached
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
    uint64_t* sdone;                      // per scatter item: (epoch tag << 32) | value
    uint32_t spin_limit;
    int sync;                             // FusedSync: how combine items wait for rows
};

// Bounded wait helper state: returns false once this wait has used up its
// polling rounds (it then raises the call's timeout word) or once another
// wait has raised it.  The shared word is read only every 64th round: all
// waiting waves reading one line on every round would serialise behind it.
// The pause between rounds grows (about 0.05, 0.4, then 1.7 us): a wait that
// lasts is for work still well ahead, and the polls of many waiting waves
// would otherwise take memory bandwidth from the work they wait for.
struct Waiter {
    uint32_t spins = 0;
    __device__ bool tick(WsHeader* hdr, uint32_t limit) {
        ++spins;
        if ((spins & 63) == 0 && ld_relaxed(&hdr->timeout.v) != 0) return false;
        if (spins > limit) {
            st_relaxed(&hdr->timeout.v, 1u);
            fence_release();
            return false;
        }
        if (spins < 16) __builtin_amdgcn_s_sleep(2);
        else if (spins < 256) __builtin_amdgcn_s_sleep(16);
        else __builtin_amdgcn_s_sleep(64);
        return true;
    }
};

__device__ __forceinline__ bool published(uint64_t word, uint32_t ep32) {
    return uint32_t(word >> 32) == ep32;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

// The leading 16 bytes of send row p, read as two agent-scope 8-byte loads
// (they see stores from any XCD once those have completed).
__device__ __forceinline__ void lead_words(const FusedArgs& a, int p, uint32_t (&w)[4]) {
    const uint64_t* d = reinterpret_cast<const uint64_t*>(a.send_rows + int64_t(p) * a.stride);
    const uint64_t lo = ld_relaxed64(d);
    const uint64_t hi = ld_relaxed64(d + 1);
    w[0] = uint32_t(lo);
    w[1] = uint32_t(lo >> 32);
    w[2] = uint32_t(hi);
    w[3] = uint32_t(hi >> 32);
}

// ---------------------------------------------------------------- hist item
__device__ void do_hist(const FusedArgs& a, int tile, int32_t (*hist)[kMaxE]) {
    hist_tile(a.idx, a.S, a.E, a.nTiles, tile, a.cnt, a.local_rank, hist);
    // cnt / local_rank are agent-coherent stores: once every wave has seen
    // its own complete, the tile is visible on every XCD and can be counted.
    wait_own_stores();
    __syncthreads();
    if (threadIdx.x == 0) fetch_add(&a.hdr->hist_done.v, 1u);
}

// ---------------------------------------------------------------- one-tile layout item
// A layout of a single tile (T*k <= kTileSlots, e.g. a decode batch) is one
// item: the histogram leaves the per-expert totals in LDS, the workgroup
// scans them itself and publishes the bases as soon as its ranks are stored.
// No scan item waits on hist_done, invalidates its cache and reads the
// counts back -- a chain that cost more than the histogram at this size.
__device__ void do_layout1(const FusedArgs& a, uint32_t ep32, int32_t (*hist)[kMaxE],
                           int* sh_tot, int* sh_wave_total)
{
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = lane_id();
    int key[kChunksPerWave];
    int rank[kChunksPerWave];
    tile_ranks(a.idx, a.S, a.E, 1, 0, nullptr, sh_tot, hist, key, rank);
    const int64_t wave_first = int64_t(wave) * kChunksPerWave * kWave;
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) {
        const int64_t s = wave_first + c * kWave + lane;
        if (key[c] >= 0)
            st_relaxed(reinterpret_cast<uint32_t*>(&a.local_rank[s]),
                       uint32_t(hist[wave][key[c]] + rank[c]));
    }
    // exclusive scan of the totals, kMaxE / kBlock experts per thread
    constexpr int kPer = kMaxE / kBlock;
    int tot[kPer];
    int tsum = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int e = tid * kPer + q;
        tot[q] = e < a.E ? sh_tot[e] : 0;
        tsum += tot[q];
    }
    const int incl = wave_inclusive_sum(tsum);
    if (lane == kWave - 1) sh_wave_total[wave] = incl;
    // the ranks are agent-coherent stores: once every wave has seen its own
    // complete, a reader that sees a base also sees them
    wait_own_stores();
    __syncthreads();
    int run = incl - tsum;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w)
        if (w < wave) run += sh_wave_total[w];
    const uint64_t tag = uint64_t(ep32) << 32;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int e = tid * kPer + q;
        if (e < a.E) {
            st_relaxed(reinterpret_cast<uint32_t*>(&a.expert_offsets[e]), uint32_t(run));
            st_relaxed64(&a.fbase[e], tag | uint32_t(run));
            if (e == a.E - 1)
                st_relaxed(reinterpret_cast<uint32_t*>(&a.expert_offsets[a.E]),
                           uint32_t(run + tot[q]));
        }
        run += tot[q];
    }
    // expert_offsets complete before this workgroup's next ticket claim (the
    // workgroup that makes the last claim of all reads them after an acquire)
    wait_own_stores();
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

    const BlockScan<kFusedScanItems> bs =
        block_scan<kFusedScanItems>(a.cnt, a.nCnt, blk, sh_wave_total);
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

    // The ranks a reader of these bases will use were stored agent-coherent
    // and completed before hist_done counted their tile, so publishing needs
    // no write-back first.
    int run = sh_word[1] + bs.thread_excl;
    // counter i is (expert i / nTiles, tile i % nTiles): one division per
    // thread, then the tile steps along (an integer division per counter
    // cost more VALU time than the stores at small layouts)
    int e = bs.i0 / a.nTiles;
    int tile = bs.i0 - e * a.nTiles;
#pragma unroll
    for (int q = 0; q < BlockScan<kFusedScanItems>::kPer; ++q) {
        const int i = bs.i0 + q;
        if (i < a.nCnt) {
            if (tile == 0)
                st_relaxed(reinterpret_cast<uint32_t*>(&a.expert_offsets[e]), uint32_t(run));
            st_relaxed64(&a.fbase[i], tag | uint32_t(run));
            run += bs.v[q];
            if (i == a.nCnt - 1)
                st_relaxed(reinterpret_cast<uint32_t*>(&a.expert_offsets[a.E]), uint32_t(run));
        }
        if (++tile == a.nTiles) {
            tile = 0;
            ++e;
        }
    }
    // expert_offsets (agent-coherent) complete before this workgroup's next
    // ticket claim: the workgroup that makes the last claim of all reads them
    // after an acquire.
    wait_own_stores();
}

// Positions of the picks of tokens [t0, t0 + ntok), run by ONE wave: pick
// q = i*k + j (slot s = t0*k + q) is handled by lane q % 64 in round q / 64.
// Polls the published base words, then p = base + local rank (or -1 for an id
// outside [0, E) or a token past T).  Writes sh_pos[q] and returns the
// positions in p[round]; false on timeout.
__device__ bool item_positions(const FusedArgs& a, int t0, int ntok, uint32_t ep32,
                               int* sh_pos, int (&p)[kPickRounds])
{
    const int lane = lane_id();
    const int npick = ntok * a.k;
    const int64_t s0 = int64_t(t0) * a.k;
    int e[kPickRounds];
    uint64_t word[kPickRounds];
#pragma unroll
    for (int r = 0; r < kPickRounds; ++r) {
        const int q = r * kWave + lane;
        const int64_t s = s0 + q;
        e[r] = (q < npick && s < a.S) ? a.idx[s] : -1;
        word[r] = 0;
    }
    // One full poll first (an item claimed after the layout is done finds
    // every base published at once).  If it fails, wait on ONE word -- every
    // lane reads the base word of pick 0, so a wave sends one request per
    // polling round instead of one per pick while the layout runs (thousands
    // of waves may wait here, and their polls would slow it) -- then poll
    // all words again; the scan publishes them within a short window.
    Waiter wt;
    for (int round = 0;; ++round) {
        if (round == 1) {
            const int e0 = __builtin_amdgcn_readfirstlane(e[0]);
            if (unsigned(e0) < unsigned(a.E)) {
                const uint64_t* w0 = &a.fbase[int64_t(e0) * a.nTiles + s0 / kTileSlots];
                Waiter wt0;
                while (!published(ld_relaxed64(w0), ep32))
                    if (!wt0.tick(a.hdr, a.spin_limit)) return false;
            }
        }
        bool ready = true;
#pragma unroll
        for (int r = 0; r < kPickRounds; ++r) {
            const int64_t s = s0 + r * kWave + lane;
            if (unsigned(e[r]) < unsigned(a.E) && !published(word[r], ep32)) {
                word[r] = ld_relaxed64(&a.fbase[int64_t(e[r]) * a.nTiles + s / kTileSlots]);
                ready = ready && published(word[r], ep32);
            }
        }
        if (ballot(!ready) == 0) break;
        if (!wt.tick(a.hdr, a.spin_limit)) return false;
    }
    fence_acquire();                       // the ranks written by the hist items
#pragma unroll
    for (int r = 0; r < kPickRounds; ++r) {
        const int q = r * kWave + lane;
        const int64_t s = s0 + q;
        int pr = -1;
        if (unsigned(e[r]) < unsigned(a.E)) {
            pr = int(uint32_t(word[r])) + a.local_rank[s];
            if (uint64_t(uint32_t(pr)) >= uint64_t(a.S)) pr = -1;   // never address outside the rows
        }
        p[r] = pr;
        if (q < npick) sh_pos[q] = pr;
    }
    return true;
}

__device__ __forceinline__ uint64_t* trailer(const FusedArgs& a, int p) {
    return reinterpret_cast<uint64_t*>(a.send_rows + int64_t(p) * a.stride + a.trailer_off);
}

// The flag of 1 KiB chunk c (kWave 16-byte vectors) of row p, after the
// trailer (sub-row flag mode).
__device__ __forceinline__ uint64_t* chunk_flag(const FusedArgs& a, int p, int c) {
    return trailer(a, p) + 2 + c;
}

// Sub-row flag mode, one wave: waits until chunk c of every row in prow[0..k)
// holds this call's flag.  No acquire fence: in this mode the chunk's data is
// read with agent-coherent loads (load16_coherent), issued only after the
// flags were seen -- an L2 invalidate per chunk and wave would cost more than
// the copy.  False on timeout.
__device__ bool chunk_ready(const FusedArgs& a, const int* prow, int k, int c, uint64_t epoch)
{
    const int lane = lane_id();
    Waiter wt;
    while (true) {
        bool ready = true;
        for (int j = lane; j < k; j += kWave) {
            const int p = prow[j];
            if (p >= 0) ready = ready && ld_relaxed64(chunk_flag(a, p, c)) == epoch;
        }
        if (ballot(!ready) == 0) break;
        if (!wt.tick(a.hdr, a.spin_limit)) return false;
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);   // no load moves above the flags
    return true;
}

// ---------------------------------------------------------------- scatter item
// U whole 64-vector chunks of a row, from the lane's byte offset lane_off:
// U loads per lane, then U streaming stores per valid pick.
template <int U>
__device__ __forceinline__ void scatter_whole(const char* __restrict__ src, const FusedArgs& a,
                                              const int* prow, uint32_t lane_off,
                                              uint32_t skip_off, bool keep)
{
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load16(src + lane_off + u * kWave * 16);
    char* rows = reinterpret_cast<char*>(a.send_rows);
    for (int j = 0; j < a.k; ++j) {
        const int p = __builtin_amdgcn_readfirstlane(prow[j]);
        if (p < 0) continue;
        const __amdgpu_buffer_rsrc_t row = buffer_rsrc(rows + int64_t(p) * a.stride, a.stride);
        if (keep) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (lane_off + u * kWave * 16 != skip_off)
                    store16_coherent_keep(row, int(lane_off) + u * kWave * 16, v[u]);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (lane_off + u * kWave * 16 != skip_off)
                    store16_coherent(row, int(lane_off) + u * kWave * 16, v[u]);
        }
    }
}

// The last, partial segment of a row: one vector at a time.  Plain scalar
// arguments: a call that took the argument struct by reference would force
// the whole struct into scratch memory.
__device__ __noinline__ void scatter_tail(const char* __restrict__ src, char* __restrict__ rows,
                                          int64_t stride, const int* prow, int k, int nvec,
                                          int v0, bool skip_first, bool keep)
{
    for (int u = 0; u < kScatU; ++u) {
        const int vi = v0 + u * kWave;
        if (vi >= nvec) break;
        if (skip_first && vi == 0) continue;
        const u32x4 v = load16(src + int64_t(vi) * 16);
        for (int j = 0; j < k; ++j) {
            const int p = prow[j];         // lanes may have left: no wave op here
            if (p < 0) continue;
            const __amdgpu_buffer_rsrc_t r = buffer_rsrc(rows + int64_t(p) * stride, stride);
            if (keep) store16_coherent_keep(r, vi * 16, v);
            else store16_coherent(r, vi * 16, v);
        }
    }
}

template <int ST>
__device__ void do_scatter(const FusedArgs& a, int item, int part, uint64_t epoch, int* sh_pos,
                           int* sh_word)
{
    constexpr int kSWpt = kWavesPerBlock / ST;      // waves per scatter token
    static_assert(ST * kSWpt == kWavesPerBlock, "whole waves per scatter token");
    static_assert(kCombTok % ST == 0 && kCombTok / ST <= 2,
                  "a combine item covers one or two whole scatter items");
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = lane_id();
    const int t0 = item * ST;
    if (wave == 0) {
        int p[kPickRounds];
        const bool ok = item_positions(a, t0, ST, uint32_t(epoch), sh_pos, p);
        if (lane == 0) sh_word[0] = ok;
    }
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(sh_word[0])) return;

    if (a.parts > 1) {
        // one part of each row: 64-vector chunks [c0, c0 + nc) of both
        // tokens, a chunk per wave at a time (one load, k stores per lane)
        const int nchunk = (a.nvec + kWave - 1) / kWave;
        const int c0 = part * nchunk / a.parts;
        const int nc = (part + 1) * nchunk / a.parts - c0;
        char* rows = reinterpret_cast<char*>(a.send_rows);
        for (int q = wave; q < ST * nc; q += kWavesPerBlock) {
            const int i = q / nc;
            const int t = t0 + i;
            if (t >= a.T) break;
            const int vi = (c0 + q % nc) * kWave + lane;
            const int* prow = sh_pos + i * a.k;
            if (vi < a.nvec) {
                const u32x4 v =
                    load16(reinterpret_cast<const char*>(a.x) + (int64_t(t) * a.nvec + vi) * 16);
                for (int j = 0; j < a.k; ++j) {
                    const int p = prow[j];         // lanes may have left: no wave op here
                    if (p < 0) continue;
                    const __amdgpu_buffer_rsrc_t r =
                        buffer_rsrc(rows + int64_t(p) * a.stride, a.stride);
                    if (t >= a.t_keep) store16_coherent_keep(r, vi * 16, v);
                    else store16_coherent(r, vi * 16, v);
                }
            }
        }
    }
    // payload: the kSWpt waves of token t0 + i copy one share each of the
    // row's 64-vector chunks, in runs of kScatU chunks, then of 4, then 1
    // (runs of kScatU alternating between two waves left one wave with 7/8
    // of an 8 KiB row)
    const int i = wave / kSWpt;
    const int wi = wave % kSWpt;
    const int t = t0 + i;
    if (a.parts == 1 && t < a.T) {
        const char* src = reinterpret_cast<const char*>(a.x) + int64_t(t) * a.nvec * 16;
        const int* prow = sh_pos + i * a.k;
        const int nchunk = (a.nvec + kWave - 1) / kWave;
        const int nwhole = a.nvec / kWave;
        const int ce = (wi + 1) * nchunk / kSWpt;
        const int we = ce < nwhole ? ce : nwhole;         // this wave's whole chunks end here
        // sentinel mode: the leading 16 bytes are written last, below
        const uint32_t skip = a.sync == kSyncSentinel ? 0u : ~0u;
        const bool keep = t >= a.t_keep;
        for (int c0 = wi * nchunk / kSWpt; c0 < ce;) {
            const int run = we - c0 >= kScatU ? kScatU : we - c0 >= 4 ? 4 : we - c0 >= 1 ? 1 : 0;
            const uint32_t off = uint32_t(c0 * kWave + lane) * 16u;
            if (run == kScatU) scatter_whole<kScatU>(src, a, prow, off, skip, keep);
            else if (run == 4) scatter_whole<4>(src, a, prow, off, skip, keep);
            else if (run == 1) scatter_whole<1>(src, a, prow, off, skip, keep);
            else                                          // the row's partial last chunk
                scatter_tail(src, reinterpret_cast<char*>(a.send_rows), a.stride, prow, a.k,
                             a.nvec, c0 * kWave + lane, skip == 0u, keep);
            const int nc = run > 0 ? run : 1;
            if (a.sync == kSyncChunkFlag) {
                // sub-row flags: this wave's chunks of the k rows, as soon as
                // its own stores of them have completed
                wait_own_stores();
                for (int q = lane; q < a.k * nc; q += kWave) {
                    const int p = prow[q / nc];
                    if (p >= 0) st_relaxed64(chunk_flag(a, p, c0 + q % nc), epoch);
                }
            }
            c0 += nc;
        }
    }
    // Release without an L2 write-back: every payload store is agent-coherent
    // (sc1), so once each wave has seen its own stores complete and the
    // workgroup has met at the barrier, the whole item's payload is visible
    // on every XCD.  This is the sequence an agent-scope release store
    // lowers to (wait for prior stores, then the sc1 flag store), minus the
    // L2 write-back that exists only for non-coherent stores -- and that
    // write-back, once per item, cost more than the copy itself.
    wait_own_stores();
    __syncthreads();

    if (wave != 0) return;
    const int npick = ST * a.k;
    const int64_t s0 = int64_t(t0) * a.k;
    const uint64_t tag = uint64_t(uint32_t(epoch)) << 32;
    if (a.sync == kSyncSentinel) {
        // Sentinel Polling: each row's leading 16 bytes, written only now,
        // are its readiness word; a payload that holds the reserved word
        // there could never be told apart from an unwritten row, so it is
        // reported, and every wait of the call gives up.
        bool clash = false;
        for (int q = lane; q < npick; q += kWave) {
            const int64_t s = s0 + q;
            if (s >= a.S) break;
            const int p = sh_pos[q];
            st_relaxed(reinterpret_cast<uint32_t*>(&a.pos[s]), uint32_t(p));
            if (p < 0) continue;
            const int t = t0 + q / a.k;
            const u32x4 lead = load16(reinterpret_cast<const char*>(a.x) + int64_t(t) * a.nvec * 16);
#pragma unroll
            for (int c = 0; c < 4; ++c) clash = clash || lead[c] == kSentinelWord;
            uint64_t* d = reinterpret_cast<uint64_t*>(a.send_rows + int64_t(p) * a.stride);
            st_relaxed64(d, uint64_t(lead[0]) | (uint64_t(lead[1]) << 32));
            st_relaxed64(d + 1, uint64_t(lead[2]) | (uint64_t(lead[3]) << 32));
        }
        if (ballot(clash) != 0 && lane == 0) {
            st_relaxed(&a.hdr->collision.v, 1u);
            st_relaxed(&a.hdr->timeout.v, 1u);
        }
        return;
    }
    if (a.sync == kSyncChunkFlag) {        // the flags are out already
        for (int q = lane; q < npick; q += kWave) {
            const int64_t s = s0 + q;
            if (s >= a.S) break;
            st_relaxed(reinterpret_cast<uint32_t*>(&a.pos[s]), uint32_t(sh_pos[q]));
        }
        return;
    }
    if (a.sync == kSyncChecksum) {
        // Data for Checksum: no per-row flag; the item's word carries the sum
        // of the 32-bit words of every row's leading 16 bytes (its marker).
        uint32_t sum = 0;
        for (int q = lane; q < npick; q += kWave) {
            const int64_t s = s0 + q;
            if (s >= a.S) break;
            const int p = sh_pos[q];
            st_relaxed(reinterpret_cast<uint32_t*>(&a.pos[s]), uint32_t(p));
            if (p < 0) continue;
            const int t = t0 + q / a.k;
            const u32x4 lead = load16(reinterpret_cast<const char*>(a.x) + int64_t(t) * a.nvec * 16);
            sum += lead[0] + lead[1] + lead[2] + lead[3];
        }
        sum = wave_sum_u32(sum);
        if (lane == 0) st_relaxed64(&a.sdone[item], tag | sum);
        return;
    }
    // item events / row flags: pos, trailer tails (agent-coherent), then the
    // epochs.  With row parts every part stores pos (the same values), and
    // part 0 the trailers.
    for (int q = lane; q < npick; q += kWave) {
        const int64_t s = s0 + q;
        if (s >= a.S) break;
        const int p = sh_pos[q];
        st_relaxed(reinterpret_cast<uint32_t*>(&a.pos[s]), uint32_t(p));
        if (part == 0 && p >= 0) st_relaxed64(trailer(a, p) + 1, uint64_t(uint32_t(s)));
    }
    wait_own_stores();                     // pos and trailer tails before the flags
    if (part == 0) {
        for (int q = lane; q < npick; q += kWave) {
            const int64_t s = s0 + q;
            if (s >= a.S) break;
            const int p = sh_pos[q];
            if (p >= 0) st_relaxed64(trailer(a, p), epoch);
        }
    }
    // the item's (part's) event word: its pos entries and its part of the
    // rows are final
    if (a.sync == kSyncItemEvents && lane == 0) st_relaxed64(&a.sdone[item * a.parts + part], tag);
}

// ---------------------------------------------------------------- combine item
// One 64-vector segment that lies inside the row: all picks' loads first (KC
// unrolled), then the fixed-order reduction.
// COH: the rows are read with agent-coherent loads (sub-row flag mode).
template <bool COH>
__device__ __forceinline__ u32x4 row_load(const FusedArgs& a, int p, uint32_t off) {
    char* row = reinterpret_cast<char*>(a.send_rows) + int64_t(p) * a.stride;
    if constexpr (COH) return load16_coherent(buffer_rsrc(row, a.stride), int(off));
    else return load16_nt(row + off);
}

template <int KC, bool COH>
__device__ __forceinline__ void combine_whole(const FusedArgs& a, const int (&pj)[KC > 0 ? KC : 1],
                                              const int* prow, const float* wrow,
                                              uint32_t off, char* dst)
{
    const uint32_t S = uint32_t(a.S);
    float acc[1][8];
    if constexpr (KC > 0) {
        u32x4 r[KC][1];
#pragma unroll
        for (int j = 0; j < KC; ++j)
            r[j][0] = uint32_t(pj[j]) < S ? row_load<COH>(a, pj[j], off) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < KC; ++j) accumulate<1>(acc, r[j], wrow[j], j == 0);
    } else {
        for (int j = 0; j < a.k; ++j) {
            const int p = __builtin_amdgcn_readfirstlane(prow[j]);
            u32x4 r[1];
            r[0] = uint32_t(p) < S ? row_load<COH>(a, p, off) : u32x4{0, 0, 0, 0};
            accumulate<1>(acc, r, wrow[j], j == 0);
        }
    }
    store_acc_coherent<1>(buffer_rsrc(dst, int64_t(a.nvec) * 16), off, acc);
}

// The last, partial segment of a row (scalar arguments, as scatter_tail).
__device__ __noinline__ void combine_tail(const char* __restrict__ rows, int64_t stride,
                                          uint32_t S, const int* prow, const float* wrow,
                                          int k, int nvec, int v0, char* dst, bool coherent)
{
    if (v0 >= nvec) return;
    const uint32_t off = uint32_t(v0) * 16u;
    float acc[1][8];
    for (int j = 0; j < k; ++j) {
        const int p = prow[j];             // lanes may have left: no wave op here
        u32x4 r[1] = {u32x4{0, 0, 0, 0}};
        if (uint32_t(p) < S) {
            const char* src = rows + int64_t(p) * stride + off;
            if (coherent) {                // two agent-scope 8-byte loads
                const uint64_t lo = ld_relaxed64(reinterpret_cast<const uint64_t*>(src));
                const uint64_t hi = ld_relaxed64(reinterpret_cast<const uint64_t*>(src) + 1);
                r[0] = u32x4{uint32_t(lo), uint32_t(lo >> 32), uint32_t(hi), uint32_t(hi >> 32)};
            } else {
                r[0] = load16_nt(src);
            }
        }
        accumulate<1>(acc, r, wrow[j], j == 0);
    }
    store_acc<1>(dst + off, acc);
}

// The batched reduction of one token whose picks all lie inside the rows.
// A wave reads and reduces up to kCombBatch 64-vector segments of its token,
// holding the packed results in registers, and only then stores them: its
// output writes come as one burst after its gathered reads, not alternating
// with them segment by segment (measured on MI355X at T=4096, H=7168, k=8,
// the whole fused call: 202.7 -> 190.3 us; at T=16384 with a skewed incast,
// 763 -> 721 us; batches of 7: 198 / 746 us).  The loads go through one
// descriptor per pick, so a lane's only address register is its offset in the
// row, and carry no per-pick condition.
constexpr int kCombBatch = 14;
constexpr int kCpolNt = 2;                      // streaming (nt) buffer access

template <int KC>
__device__ __forceinline__ u32x4 reduce_segment(const __amdgpu_buffer_rsrc_t (&rj)[KC],
                                                const float (&wj)[KC], uint32_t off)
{
    u32x4 r[KC][1];
#pragma unroll
    for (int j = 0; j < KC; ++j)
        r[j][0] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rj[j], int(off), 0, kCpolNt));
    float acc[1][8];
#pragma unroll
    for (int j = 0; j < KC; ++j) accumulate<1>(acc, r[j], wj[j], j == 0);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[0][2 * q], acc[0][2 * q + 1]);
    return o;
}

template <int KC>
__device__ __forceinline__ void combine_token_batched(const FusedArgs& a, const int (&pj)[KC],
                                                      const int* prow, const float* wrow,
                                                      char* dst)
{
    const int lane = lane_id();
    const int nwhole = a.nvec / kWave;
    const uint32_t lane_off = uint32_t(lane) * 16u;
    const __amdgpu_buffer_rsrc_t orow = buffer_rsrc(dst, int64_t(a.nvec) * 16);
    __amdgpu_buffer_rsrc_t rj[KC];
    float wj[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) {
        rj[j] = buffer_rsrc(reinterpret_cast<char*>(a.send_rows) + int64_t(pj[j]) * a.stride,
                            a.stride);
        wj[j] = wrow[j];
    }
    for (int s0 = 0; s0 < nwhole; s0 += kCombBatch) {
        u32x4 o[kCombBatch];
#pragma unroll
        for (int b = 0; b < kCombBatch; ++b) {
            // a short last batch skips its missing segments: a uniform
            // branch, and each segment's loads are waited for inside it
            if (s0 + b < nwhole) {
                o[b] = reduce_segment<KC>(rj, wj, uint32_t(s0 + b) * (kWave * 16u) + lane_off);
                // reduced here, not sunk down to its store: sinking would keep
                // every segment's loaded rows live at once
                asm volatile("" : "+v"(o[b]));
            }
        }
#pragma unroll
        for (int b = 0; b < kCombBatch; ++b)
            if (s0 + b < nwhole)
                store16_coherent(orow, int(uint32_t(s0 + b) * (kWave * 16u) + lane_off), o[b]);
    }
    if (nwhole * kWave < a.nvec)
        combine_tail(reinterpret_cast<const char*>(a.send_rows), a.stride, uint32_t(a.S), prow,
                     wrow, a.k, a.nvec, nwhole * kWave + lane, dst, false);
}

// Waits, in one wave, until the rows p[] of a combine item are complete by
// the Data-as-Flag check of a.sync (row flag, checksum or sentinel).  The
// positions came from the published bases, not from the scatter items.
template <int ST>
__device__ bool rows_ready(const FusedArgs& a, int t0, const int (&p)[kPickRounds],
                           uint64_t epoch)
{
    const int lane = lane_id();
    Waiter wt;
    if (a.sync == kSyncRowFlag) {
        while (true) {
            bool ready = true;
#pragma unroll
            for (int r = 0; r < kPickRounds; ++r)
                if (p[r] >= 0) ready = ready && ld_relaxed64(trailer(a, p[r])) == epoch;
            if (ballot(!ready) == 0) return true;
            if (!wt.tick(a.hdr, a.spin_limit)) return false;
        }
    }
    if (a.sync == kSyncSentinel) {
        while (true) {
            bool ready = true;
#pragma unroll
            for (int r = 0; r < kPickRounds; ++r) {
                if (p[r] < 0) continue;
                uint32_t w[4];
                lead_words(a, p[r], w);
#pragma unroll
                for (int c = 0; c < 4; ++c) ready = ready && w[c] != kSentinelWord;
            }
            if (ballot(!ready) == 0) return true;
            if (!wt.tick(a.hdr, a.spin_limit)) return false;
        }
    }
    // kSyncChecksum: the scatter items' words, then the rows' markers summed
    // per item must match them
    const uint32_t ep32 = uint32_t(epoch);
    const int sfirst = t0 / ST;
    const int nsc = a.nScat - sfirst < kCombTok / ST ? a.nScat - sfirst : kCombTok / ST;
    uint64_t word = 0;
    while (true) {
        if (lane < nsc) word = ld_relaxed64(&a.sdone[sfirst + lane]);
        const bool mine = lane < nsc ? published(word, ep32) : true;
        if (ballot(!mine) == 0) break;
        if (!wt.tick(a.hdr, a.spin_limit)) return false;
    }
    fence_acquire();
    static_assert(kCombTok / ST <= 2, "at most two scatter items per combine item");
    const uint32_t want0 = uint32_t(__shfl(word, 0, kWave));
    const uint32_t want1 = uint32_t(__shfl(word, 1, kWave));
    const int per_item = ST * a.k;
    while (true) {
        uint32_t sum0 = 0, sum1 = 0;
#pragma unroll
        for (int r = 0; r < kPickRounds; ++r) {
            if (p[r] < 0) continue;
            uint32_t w[4];
            lead_words(a, p[r], w);
            const uint32_t v = w[0] + w[1] + w[2] + w[3];
            if ((r * kWave + lane) / per_item == 0) sum0 += v;
            else sum1 += v;
        }
        sum0 = wave_sum_u32(sum0);
        sum1 = wave_sum_u32(sum1);
        if (sum0 == want0 && (nsc < 2 || sum1 == want1)) return true;
        if (!wt.tick(a.hdr, a.spin_limit)) return false;
    }
}

template <int KC, int ST>
__device__ void do_combine(const FusedArgs& a, int item, int part, uint64_t epoch, int* sh_pos,
                           int* sh_word)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = lane_id();
    const int t0 = item * kCombTok;
    if (wave == 0 && a.sync != kSyncItemEvents) {
        int p[kPickRounds];
        bool ok = item_positions(a, t0, kCombTok, uint32_t(epoch), sh_pos, p);
        // sub-row flags: each wave waits per chunk below
        if (ok && a.sync != kSyncChunkFlag) ok = rows_ready<ST>(a, t0, p, epoch);
        if (ok) fence_acquire();           // the rows' payloads
        if (lane == 0) sh_word[0] = ok;
    } else if (wave == 0) {
        // 1. the event words of the scatter items of these tokens: once they
        //    hold this call's epoch, those items' pos entries are final (one
        //    word per scatter item instead of recomputing every position from
        //    the published bases and ranks -- fewer dependent load rounds,
        //    which cost several microseconds each while HBM is saturated)
        bool ok = true;
        const int sfirst = t0 / ST;
        const int nsc = a.nScat - sfirst < kCombTok / ST ? a.nScat - sfirst : kCombTok / ST;
        Waiter wt0;
        while (true) {
            const uint64_t tag = uint64_t(uint32_t(epoch)) << 32;
            const bool mine =
                lane < nsc ? ld_relaxed64(&a.sdone[(sfirst + lane) * a.parts + part]) == tag : true;
            if (ballot(!mine) == 0) break;
            if (!wt0.tick(a.hdr, a.spin_limit)) {
                ok = false;
                break;
            }
        }
        int p[kPickRounds];
        if (ok) {
            fence_acquire();               // the pos entries of those items
            // 2. positions of the item's picks, from pos (every load from a
            //    clamped in-bounds slot, so the rounds' loads go out together)
            const int npick = kCombTok * a.k;
            const int64_t s0 = int64_t(t0) * a.k;
#pragma unroll
            for (int r = 0; r < kPickRounds; ++r) {
                const int q = r * kWave + lane;
                const int64_t s = s0 + q;
                const bool in = q < npick && s < a.S;
                int pr = a.pos[in ? s : 0];
                if (!in || uint64_t(uint32_t(pr)) >= uint64_t(a.S)) pr = -1;   // never address outside the rows
                p[r] = pr;
                if (q < npick) sh_pos[q] = pr;
            }
            // 3. acquire-poll every row's trailer (the Data-as-Flag check)
            Waiter wt;
            while (true) {
                bool ready = true;
#pragma unroll
                for (int r = 0; r < kPickRounds; ++r)
                    if (p[r] >= 0) ready = ready && ld_relaxed64(trailer(a, p[r])) == epoch;
                if (ballot(!ready) == 0) break;
                if (!wt.tick(a.hdr, a.spin_limit)) {
                    ok = false;
                    break;
                }
            }
            fence_acquire();               // the rows' payloads
        }
        if (lane == 0) sh_word[0] = ok;
    }
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(sh_word[0])) return;

    // kWavesPerBlock / kCombTok waves per token, alternating 64-vector segments
    constexpr int kWpt = kWavesPerBlock / kCombTok;
    const int i = wave / kWpt;
    const int t = t0 + i;
    if (t >= a.T) return;
    const int k = KC > 0 ? KC : a.k;
    const int* prow = sh_pos + i * k;
    const float* wrow = a.w + int64_t(t) * k;
    char* dst = reinterpret_cast<char*>(a.out) + int64_t(t) * a.nvec * 16;
    int pj[KC > 0 ? KC : 1];
#pragma unroll
    for (int j = 0; j < (KC > 0 ? KC : 1); ++j)
        pj[j] = KC > 0 ? __builtin_amdgcn_readfirstlane(prow[j]) : 0;
    if constexpr (KC > 0 && kWpt == 1) {
        // rows known complete (not the per-chunk mode), whole rows and every
        // pick inside
        bool inside = a.sync != kSyncChunkFlag && a.parts == 1;
#pragma unroll
        for (int j = 0; j < KC; ++j) inside = inside && uint32_t(pj[j]) < uint32_t(a.S);
        if (inside) {
            combine_token_batched<KC>(a, pj, prow, wrow, dst);
            return;
        }
    }
    // the item's part of the row: 64-vector chunks [c0, c1)
    const int nchunk = (a.nvec + kWave - 1) / kWave;
    const int c0 = part * nchunk / a.parts;
    const int c1 = (part + 1) * nchunk / a.parts;
    for (int v0 = (c0 + wave % kWpt) * kWave + lane; v0 - lane < c1 * kWave; v0 += kWpt * kWave) {
        if (a.sync == kSyncChunkFlag && !chunk_ready(a, prow, k, (v0 - lane) / kWave, epoch))
            return;
        const bool coh = a.sync == kSyncChunkFlag;
        if (v0 - lane + kWave <= a.nvec) {
            if (coh) combine_whole<KC, true>(a, pj, prow, wrow, uint32_t(v0) * 16u, dst);
            else combine_whole<KC, false>(a, pj, prow, wrow, uint32_t(v0) * 16u, dst);
        } else {
            combine_tail(reinterpret_cast<const char*>(a.send_rows), a.stride, uint32_t(a.S),
                         prow, wrow, a.k, a.nvec, v0, dst, coh);
        }
    }
}

// ---------------------------------------------------------------- the launch
template <int KC, int ST>
__global__ __launch_bounds__(kBlock) void fused_kernel(FusedArgs a) {
    __shared__ int32_t hist[kWavesPerBlock][kMaxE];
    __shared__ int sh_tot[kMaxE];
    __shared__ int sh_pos[kMaxItemPicks];
    __shared__ int sh_wave_total[kWavesPerBlock];
    __shared__ int sh_word[2];
    __shared__ int sh_ticket;
    const int tid = threadIdx.x;
    const uint64_t epoch = a.hdr->epoch;          // constant during the call
    const int first_scan = a.nTiles;
    const int first_scatter = first_scan + a.nScan;
    const int first_combine = first_scatter + a.nScat * a.parts;
    const int total = first_combine + a.nComb * a.parts;

    // The barrier opens each round, BEFORE thread 0 claims the ticket: a
    // divergent thread-0 block must never follow another one (the end of a
    // hist item) with no barrier in between, or the compiler may merge the
    // two and build an inner loop that only lane 0 leaves -- the other 255
    // threads would then cycle on a stale ticket forever.  The ticket is made
    // wave-uniform so every branch on it is a scalar branch.
    int ticket;
    while (true) {
        __syncthreads();                  // everyone has read the last ticket
        if (tid == 0) sh_ticket = int(fetch_add(&a.hdr->work_ticket.v, 1u));
        __syncthreads();
        ticket = __builtin_amdgcn_readfirstlane(sh_ticket);
        if (ticket >= total) break;
        if (ticket < first_scan) {
            if (a.nScan == 0) do_layout1(a, uint32_t(epoch), hist, sh_tot, sh_wave_total);
            else do_hist(a, ticket, hist);
        }
        else if (ticket < first_scatter) do_scan(a, ticket - first_scan, uint32_t(epoch), sh_wave_total, sh_word);
        else if (ticket < first_combine) {
            const int u = ticket - first_scatter;
            do_scatter<ST>(a, u / a.parts, u % a.parts, epoch, sh_pos, sh_word);
        } else {
            const int u = ticket - first_combine;
            do_combine<KC, ST>(a, u / a.parts, u % a.parts, epoch, sh_pos, sh_word);
        }
    }

    // Every workgroup makes exactly one claim past the last item, after all
    // its work; the one whose claim came last of all (total + gridDim.x - 1)
    // therefore runs after every other workgroup has finished.  It derives
    // the counts, records the error word and resets the state.
    if (ticket != total + int(gridDim.x) - 1) return;
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
        if (ld_relaxed(&h->collision.v)) err = kDevSentinel;
        else if (ld_relaxed(&h->timeout.v)) err = kDevTimeout;
        else if (a.expert_offsets[a.E] != a.S) err = kDevBadExpert;
        h->error = err;
        h->collision.v = 0;
        h->timeout.v = 0;
        h->work_ticket.v = 0;
        h->hist_done.v = 0;
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
        hdr->collision.v = 0;
        hdr->work_ticket.v = 0;
        hdr->hist_done.v = 0;
        hdr->epoch = first_epoch;
        hdr->last_epoch = 0;
    }
}

// Sentinel mode, before each call: every row's leading 16 bytes get the
// reserved pattern again (the reset pass that sentinel polling needs after
// the rows of the previous call were consumed).
__global__ __launch_bounds__(kBlock) void sentinel_reset_kernel(uint8_t* rows, int64_t stride,
                                                                int64_t S)
{
    const u32x4 v = {kSentinelWord, kSentinelWord, kSentinelWord, kSentinelWord};
    for (int64_t s = int64_t(blockIdx.x) * kBlock + threadIdx.x; s < S;
         s += int64_t(gridDim.x) * kBlock)
        store16(rows + s * stride, v);
}

// The persistent grid: at most kFusedPerCu workgroups per CU, and no more
// than can be resident (cached per device and instantiation; atomic entries,
// as above).  Fewer workgroups than fit leave fewer concurrent streams of
// scattered row writes and fewer pollers, as in dispatch's capped grid
// (measured on MI355X at T=4096, H=7168, k=8, one call: 217.7 us with every
// resident workgroup (5 per CU), 212.1 / 209.6 / 206.5 us with 256 / 384 /
// 512 workgroups; the other sync modes alike).
constexpr int kFusedPerCu = 2;

// `which` numbers the instantiation (0-3) for the cache.
int resident_grid(const void* kernel, int which) {
    static std::atomic<int> cached[64][4];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    const int slot = dev < 64 ? dev : 63;
    const int have = cached[slot][which].load(std::memory_order_relaxed);
    if (have > 0) return have;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBlock, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    if (per_cu > kFusedPerCu) per_cu = kFusedPerCu;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    cached[slot][which].store(per_cu * cus, std::memory_order_relaxed);
    return per_cu * cus;
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
                        uint16_t* out, void* ws, uint32_t spin_limit, int grid, int sync,
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
    // one tile: its item scans the counts itself (no scan items)
    a.nScan = f.lay.nTiles == 1 ? 0 : (f.lay.nCnt + kFusedScanItems - 1) / kFusedScanItems;
    a.nComb = (T + kCombTok - 1) / kCombTok;
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
    a.sdone = reinterpret_cast<uint64_t*>(w + f.off_sdone);
    a.spin_limit = spin_limit ? spin_limit : kDefaultSpinLimit;
    a.sync = sync;

    if (sync == kSyncSentinel) {
        const int64_t blocks = (a.S + kBlock - 1) / kBlock;
        const uint32_t rg = blocks < 1024 ? uint32_t(blocks) : 1024u;
        EP_LAUNCH(sentinel_reset_kernel, dim3(rg), dim3(kBlock), 0, s, send_rows, a.stride, a.S);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    // the instantiation for the pick count and the scatter item size
    auto kernel_for = [k](int st) -> const void* {
        if (k == 8)
            return st == 4 ? reinterpret_cast<const void*>(&fused_kernel<8, 4>)
                           : reinterpret_cast<const void*>(&fused_kernel<8, 2>);
        return st == 4 ? reinterpret_cast<const void*>(&fused_kernel<0, 4>)
                       : reinterpret_cast<const void*>(&fused_kernel<0, 2>);
    };
    auto which = [k](int st) { return (k == 8 ? 0 : 2) + (st == 4 ? 1 : 0); };
    int g = grid > 0 ? grid : resident_grid(kernel_for(2), which(2));
    // Scatter items of 4 tokens for rows of at most 8 KiB, and for a batch
    // whose 2-token items would be fewer than the workgroups (it is split into
    // row parts below, item-event mode only); 2 tokens otherwise.
    const bool few = sync == kSyncItemEvents && (T + 1) / 2 < g;
    const int st = (a.nvec <= 512 || few) ? 4 : 2;
    if (grid <= 0 && st != 2) g = resident_grid(kernel_for(st), which(st));
    a.nScat = (T + st - 1) / st;
    // Row parts: a batch with fewer scatter items than workgroups splits each
    // item's rows into parts (64-vector chunks), so its few tokens still
    // spread over the GPU -- at T = 128 two-token items would keep 64
    // workgroups busy, and one workgroup moves only ~30-40 GB/s of scattered
    // rows.  Item-event readiness only: each part has its own event word.
    // the rows of the last tokens stay in the caches for the combine items
    a.t_keep = keep_from(T, H, k);
    a.parts = 1;
    if (sync == kSyncItemEvents && a.nScat < g) {
        const int nchunk = (a.nvec + kWave - 1) / kWave;
        int P = (g + a.nScat - 1) / a.nScat;
        if (P > kFusedMaxParts) P = kFusedMaxParts;
        if (P > nchunk) P = nchunk;
        a.parts = P;
    }
    const int items = a.nTiles + a.nScan + (a.nScat + a.nComb) * a.parts;
    if (g > items) g = items;
    if (k == 8 && st == 4)
        EP_LAUNCH((fused_kernel<8, 4>), dim3(g), dim3(kBlock), 0, s, a);
    else if (k == 8)
        EP_LAUNCH((fused_kernel<8, 2>), dim3(g), dim3(kBlock), 0, s, a);
    else if (st == 4)
        EP_LAUNCH((fused_kernel<0, 4>), dim3(g), dim3(kBlock), 0, s, a);
    else
        EP_LAUNCH((fused_kernel<0, 2>), dim3(g), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace ep
