// coalesce.hip -- rank-level token coalescing of the send records, and the
// cyclic exchange waves (the sender-side, one-GPU part of a multi-GPU
// exchange).
//
// RailWave sec. 3.1-3.2: the transfer records of a destination keep the
// backend's token coalescing, and one record may carry several destinations
// of the same token.  Here one record per (token t, destination rank r),
// r = expert / L with L = E/R local experts per rank, carrying the bit mask
// of r's local experts that t picked; records rank-major, then by ascending
// token.  A token that sends two of its k picks to one rank sends its row
// there once, so the send buffer shrinks from T*k rows to the number of
// distinct (token, rank) pairs.
//
// Three steps on one stream:
//   1. keys: a lane per pick (a token's picks in adjacent lanes) marks
//      whether the pick is its token's first pick of its rank (key = rank)
//      or a repeat (key = -1);
//   2. the dispatch layout (layout.hip) over the keys, with the R ranks as
//      its "experts": its stable counting sort gives the per-rank record
//      counts, offsets and each first pick's record row; the repeats are
//      skipped on purpose (expected total -1);
//   3. rows: a lane per pick gives every pick the row of its token's first
//      pick of the same rank and writes each record's token and
//      local-expert mask.
// Dispatching x with the first-pick positions (repeats -1, which ep_dispatch
// skips) then writes every record exactly once.
//
// The receiver's side (ep_expand_records): the records of one rank, each with
// its mask, expand into that rank's local experts' slots -- expert-major,
// then in record order (StrataCL appendix, level 2: expert windows).  It is
// a stable counting sort of the (record, set bit) pairs by expert, i.e. the
// dispatch layout over C "tokens" with L "picks" (key = the bit's expert, or
// -1 when clear) and L experts, followed by a dispatch of the record rows
// with those positions into a receive buffer of a given row count.
//
// RailWave sec. 3.2, eq. (10): the cyclic pairwise exchange sends, in wave
// k = 1..N-1, from node s to node (s + k) mod N, so every node has one
// outgoing and one incoming peer per wave and every ordered pair appears
// once per round.  That schedule is host logic (ep_exchange_waves).
#include "../../include/ep_route_topk.h"
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

// Lanes [g*k, g*k + k) of a wave hold the k picks of one token, for the
// g < 64/k tokens a wave takes (k <= 64); any lanes left over idle.  The
// picks of a token are read by consecutive lanes (coalesced), and a pick
// compares its rank with its token's other picks through lane shuffles.
struct PickLane {
    int64_t t;      // token
    int j;          // pick
    int base;       // lane of the token's pick 0
    bool active;
};

__device__ __forceinline__ PickLane pick_lane(int T, int k)
{
    const int per = kWave / k;
    const int lane = lane_id();
    const int g = lane / k;
    PickLane pl;
    pl.j = lane - g * k;
    pl.base = g < per ? g * k : 0;
    pl.t = (int64_t(blockIdx.x) * kBlock + threadIdx.x) / kWave * per + g;
    pl.active = g < per && pl.t < T;
    return pl;
}

// key = the pick's rank when it is the token's first pick of that rank (in
// pick order), else -1; an id outside [0, E) also gets -1.
__global__ __launch_bounds__(kBlock) void coalesce_keys_kernel(
    const int32_t* __restrict__ topk_idx, int T, int k, int E, int L,
    int32_t* __restrict__ keys)
{
    const PickLane pl = pick_lane(T, k);
    const int32_t e = pl.active ? topk_idx[pl.t * k + pl.j] : -1;
    const bool valid = uint32_t(e) < uint32_t(E);
    const int32_t r = valid ? e / L : -1;
    bool first = valid;
    for (int i = 0; i < k; ++i) {               // the same trip count in every lane
        const int32_t ri = __shfl(r, pl.base + i, kWave);
        if (i < pl.j && ri == r) first = false;
    }
    if (pl.active) keys[pl.t * k + pl.j] = first ? r : -1;
}

// send_pos holds the first picks' rows (the layout's positions); every pick
// takes the row of its token's first pick of the same rank, and each first
// pick writes its record's token and local-expert mask.  A row outside
// [0, T*k) is never written through.
__global__ __launch_bounds__(kBlock) void coalesce_rows_kernel(
    const int32_t* __restrict__ topk_idx, int T, int k, int E, int L,
    const int32_t* __restrict__ send_pos, int32_t* __restrict__ row_of_pick,
    int32_t* __restrict__ row_src, uint64_t* __restrict__ row_experts,
    WsHeader* __restrict__ hdr)
{
    const PickLane pl = pick_lane(T, k);
    const uint32_t S = uint32_t(T) * uint32_t(k);
    // both loads unconditional (an idle lane reads slot 0 and drops it), so
    // they are in flight together rather than one after the other
    const int64_t slot = pl.active ? pl.t * k + pl.j : 0;
    const int32_t e_raw = topk_idx[slot];
    const int32_t p_raw = send_pos[slot];
    const int32_t e = pl.active ? e_raw : -1;
    const bool valid = uint32_t(e) < uint32_t(E);
    const int32_t r = valid ? e / L : -1;
    const int32_t p = pl.active ? p_raw : -1;
    int j0 = -1;
    int32_t row = -1;
    uint64_t mask = 0;
    for (int i = 0; i < k; ++i) {
        const int32_t ri = __shfl(r, pl.base + i, kWave);
        const int32_t ei = __shfl(e, pl.base + i, kWave);
        const int32_t pi = __shfl(p, pl.base + i, kWave);
        if (valid && ri == r) {
            if (j0 < 0) {
                j0 = i;
                row = pi;
            }
            mask |= uint64_t(1) << (ei % L);
        }
    }
    if (pl.active) row_of_pick[pl.t * k + pl.j] = valid ? row : -1;
    if (valid && j0 == pl.j && uint32_t(row) < S) {
        row_src[row] = int32_t(pl.t);
        row_experts[row] = mask;
    }
    // the layout wrote its error word before this kernel started
    if (pl.active && !valid) hdr->error = kDevBadExpert;
}

// ---------------------------------------------------------------- receiver
// A thread per (record c, local expert i): key = i when record c feeds expert
// i (bit i of its mask), else -1.
__global__ __launch_bounds__(kBlock) void expand_keys_kernel(const uint64_t* __restrict__ masks,
                                                             int C, int L,
                                                             int32_t* __restrict__ keys)
{
    const int64_t q = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    if (q >= int64_t(C) * L) return;
    const int64_t c = q / L;
    const int i = int(q - c * L);
    keys[q] = ((masks[c] >> i) & 1u) ? i : -1;
}

// After the layout has written its error word: a mask bit at or past L (no
// such expert) or more slots than the receive buffer has rows is an error.
// Two such faults at once may report either one.
__global__ __launch_bounds__(kBlock) void expand_finish_kernel(
    const uint64_t* __restrict__ masks, int C, int L, const int32_t* __restrict__ expert_offsets,
    int64_t recv_rows, WsHeader* __restrict__ hdr)
{
    bool bad = false;
    if (L < 64)
        for (int64_t c = int64_t(blockIdx.x) * kBlock + threadIdx.x; c < C;
             c += int64_t(gridDim.x) * kBlock)
            bad |= (masks[c] >> L) != 0;
    if (bad) hdr->error = kDevBadExpert;
    if (blockIdx.x == 0 && threadIdx.x == 0 && int64_t(expert_offsets[L]) > recv_rows)
        hdr->error = kDevOverflow;
}

}  // namespace

hipError_t launch_expand_records(const uint16_t* rows, const uint64_t* masks, int C, int H, int L,
                                 int32_t* expert_counts, int32_t* expert_offsets, int32_t* pos,
                                 uint16_t* recv, int64_t recv_rows, void* ws, hipStream_t s)
{
    // the layout over (C records) x (L bits) with the L local experts as its
    // experts and one rank; its workspace shape is the coalescing pass's
    const CoalescePlan p = coalesce_plan(C, L, L);
    char* w = static_cast<char*>(ws);
    int32_t* keys = reinterpret_cast<int32_t*>(w + p.off_keys);
    int32_t* lay_rank_counts = reinterpret_cast<int32_t*>(w + p.off_rank_counts);
    int32_t* lay_rank_offsets = reinterpret_cast<int32_t*>(w + p.off_rank_offsets);
    const int64_t n = int64_t(C) * L;
    EP_LAUNCH(expand_keys_kernel, dim3(uint32_t((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, s,
              masks, C, L, keys);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_dispatch_layout_skips(keys, C, L, L, 1, expert_counts, expert_offsets,
                                     lay_rank_counts, lay_rank_offsets, pos, nullptr, w, -1, s);
    if (e != hipSuccess) return e;
    const uint32_t bound = uint32_t(recv_rows < n ? recv_rows : n);
    e = launch_dispatch_bounded(rows, C, H, L, pos, recv, bound, s);
    if (e != hipSuccess) return e;
    const int64_t blocks = (int64_t(C) + kBlock - 1) / kBlock;
    EP_LAUNCH(expand_finish_kernel, dim3(uint32_t(blocks < 1024 ? blocks : 1024)), dim3(kBlock),
              0, s, masks, C, L, expert_offsets, recv_rows, reinterpret_cast<WsHeader*>(w));
    return hipGetLastError();
}

hipError_t launch_rank_coalesce(const int32_t* topk_idx, int T, int k, int E, int R,
                                int32_t* rank_counts, int32_t* rank_offsets,
                                int32_t* row_of_pick, int32_t* send_pos, int32_t* row_src,
                                uint64_t* row_experts, void* ws, hipStream_t s)
{
    const CoalescePlan p = coalesce_plan(T, k, R);
    char* w = static_cast<char*>(ws);
    int32_t* keys = reinterpret_cast<int32_t*>(w + p.off_keys);
    int32_t* lay_rank_counts = reinterpret_cast<int32_t*>(w + p.off_rank_counts);
    int32_t* lay_rank_offsets = reinterpret_cast<int32_t*>(w + p.off_rank_offsets);
    const int L = E / R;
    const int64_t waves = (int64_t(T) + kWave / k - 1) / (kWave / k);
    const uint32_t grid = uint32_t((waves * kWave + kBlock - 1) / kBlock);
    EP_LAUNCH(coalesce_keys_kernel, dim3(grid), dim3(kBlock), 0, s, topk_idx, T, k, E, L, keys);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the ranks are the layout's experts (one per rank): its expert counts and
    // offsets are the per-rank record counts and offsets
    e = launch_dispatch_layout_skips(keys, T, k, R, R, rank_counts, rank_offsets,
                                     lay_rank_counts, lay_rank_offsets, send_pos, nullptr, w,
                                     -1, s);
    if (e != hipSuccess) return e;
    EP_LAUNCH(coalesce_rows_kernel, dim3(grid), dim3(kBlock), 0, s, topk_idx, T, k, E, L,
              send_pos, row_of_pick, row_src, row_experts, reinterpret_cast<WsHeader*>(w));
    return hipGetLastError();
}

void exchange_waves(int32_t N, int32_t* peer)
{
    for (int32_t k = 1; k < N; ++k)
        for (int32_t s = 0; s < N; ++s) peer[int64_t(k - 1) * N + s] = (s + k) % N;
}

}  // namespace ep
