// dispatch.hip -- permute token rows into the expert-contiguous send buffer.
//
// UBEP sec. 2.1 / sec. 2.3: each token's activation goes to every expert it
// picked, written straight into its final place in the receive region that
// is partitioned by (rank, expert) -- no staging copy.  Here:
// send[pos[t][j]] = x[t] for every pick (t, j).
//
// HBM-bound copy (1 read, k writes per row).  A wave owns one (token, row
// segment) item: each lane loads U 16-byte vectors of the row (coalesced,
// 1 KiB per wave instruction), then writes them to the k destination rows,
// so each row is read from HBM once.  The k row indices are wave-uniform
// scalar loads.  The stores are streaming and agent-coherent (nt sc1,
// through a descriptor over the destination row): they are written through
// the XCD's L2 instead of staying dirty in it, so the kernel ends with no
// write-back of ~32 MB of dirty lines in front of the next kernel (measured
// on MI355X at T=4096, H=7168, k=8: the route/layout/dispatch/combine step
// 213 -> 205 us).
#include <atomic>

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kWavesPerBlock = kBlock / kWave;

// One (token, segment) item whose vectors all lie inside the row: U loads
// per lane, then U stores per pick, no per-vector checks.  keep: the stores
// drop the streaming hint (rows the next kernel reads while still cached).
template <int U>
__device__ __forceinline__ void copy_whole(const char* __restrict__ src,
                                           char* __restrict__ send, int64_t row_bytes,
                                           const int32_t* __restrict__ prow, int k,
                                           uint32_t S, int v0, bool keep)
{
    const uint32_t lane_off = uint32_t(v0) * 16u;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load16(src + lane_off + u * kWave * 16);
    for (int j = 0; j < k; ++j) {
        const int32_t p = prow[j];
        if (uint32_t(p) >= S) continue;
        const __amdgpu_buffer_rsrc_t row = buffer_rsrc(send + int64_t(p) * row_bytes, row_bytes);
        if (keep) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                store16_coherent_keep(row, int(lane_off) + u * kWave * 16, v[u]);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) store16_coherent(row, int(lane_off) + u * kWave * 16, v[u]);
        }
    }
}

// The last, partial segment of a row: one vector at a time (plain stores,
// streaming unless `keep`: a descriptor built from this function's
// non-uniform arguments would cost a loop over the lanes).
__device__ __noinline__ void copy_tail(const char* __restrict__ src, char* __restrict__ send,
                                       int64_t row_bytes, const int32_t* __restrict__ prow,
                                       int k, uint32_t S, int v0, int U, int nvec, bool keep)
{
    for (int u = 0; u < U; ++u) {
        const int vi = v0 + u * kWave;
        if (vi >= nvec) break;
        const u32x4 v = load16(src + int64_t(vi) * 16);
        for (int j = 0; j < k; ++j) {
            const int32_t p = prow[j];
            if (uint32_t(p) >= S) continue;
            char* d = send + int64_t(p) * row_bytes + int64_t(vi) * 16;
            if (keep) store16(d, v);
            else store16_nt(d, v);
        }
    }
}

// Work items are (group of 4 tokens, row segment of kWave*U vectors) pairs,
// one wave per token, numbered segment-fastest: the workgroups resident at
// one time cover whole rows, so each destination row is written as one
// contiguous run (measured on MI355X at T=4096, H=7168, k=8: 1-2 us less
// than token-fastest order).  A 1-D grid of at most dispatch_grid_cap()
// workgroups (160 on MI355X) strides over the items in even rounds: fewer
// concurrent streams of scattered row writes keep better DRAM locality, and
// 96-128 workgroups already saturate the write path (measured at the same
// shape, streaming stores: dispatch alone 92.4 -> 87.7-89.0 us with 96-128
// workgroups against every item's; the whole route/layout/dispatch/combine
// step 205.5-207.2 -> 199.4-202.1 us); a few more hide x's read latency when
// x comes from HBM.
// Rows at or past S (T*k, or a smaller receive buffer's row count) are never
// written.
// Tokens from t_keep on store their rows cached (keep_from).
template <int U>
__global__ __launch_bounds__(kBlock) void dispatch_kernel(
    const uint16_t* __restrict__ x, int T, int nvec, int k,
    const int32_t* __restrict__ pos, uint16_t* __restrict__ send,
    uint32_t segs, uint32_t items, uint32_t S, int t_keep)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t row_bytes = int64_t(nvec) * 16;
    char* dst = reinterpret_cast<char*>(send);
    for (uint32_t b = blockIdx.x; b < items; b += gridDim.x) {
        const uint32_t group = b / segs;
        const int seg = int(b - group * segs);
        const int t = int(group) * kWavesPerBlock + wave;
        if (t >= T) continue;
        const char* src = reinterpret_cast<const char*>(x) + int64_t(t) * row_bytes;
        const int32_t* prow = pos + int64_t(t) * k;
        const int v0 = seg * kWave * U + lane_id();
        if ((seg + 1) * kWave * U <= nvec)
            copy_whole<U>(src, dst, row_bytes, prow, k, S, v0, t >= t_keep);
        else
            copy_tail(src, dst, row_bytes, prow, k, S, v0, U, nvec, t >= t_keep);
    }
}

template <int U>
hipError_t launch_u(const uint16_t* x, int T, int nvec, int k, const int32_t* pos,
                    uint16_t* send, uint32_t cap, uint32_t bound, int t_keep, hipStream_t s)
{
    const uint32_t segs = uint32_t((nvec + kWave * U - 1) / (kWave * U));
    const uint32_t items = uint32_t((T + kWavesPerBlock - 1) / kWavesPerBlock) * segs;
    // the fewest rounds of items that cap allows, spread evenly over the
    // smallest grid that keeps that many rounds: no nearly idle last round
    const uint32_t rounds = (items + cap - 1) / cap;
    const uint32_t grid = (items + rounds - 1) / rounds;
    EP_LAUNCH((dispatch_kernel<U>), dim3(grid), dim3(kBlock), 0, s, x, T, nvec, k, pos,
              send, segs, items, bound, t_keep);
    return hipGetLastError();
}

}  // namespace

// Cached per device; the cache entries are atomic, so concurrent first calls
// from several threads are safe (they store the same value).
uint32_t device_cu_count() {
    static std::atomic<uint32_t> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    const int slot = dev < 64 ? dev : 63;
    uint32_t v = cached[slot].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < 2)
            cus = 256;
        v = uint32_t(cus);
        cached[slot].store(v, std::memory_order_relaxed);
    }
    return v;
}

bool small_scatter(int T, int H, int k)
{
    return int64_t(T) * k * H * 2 <= kSmallScatterBytes;
}

bool keep_rows(int T, int H, int k)
{
    return int64_t(T) * k * H * 2 <= kKeepRowsBytes;
}

int keep_from(int T, int H, int k)
{
    const int64_t per_token = int64_t(k) * H * 2;
    if (int64_t(T) * per_token > kKeepMaxBytes) return T;
    const int64_t tail = kKeepTailBytes / per_token;
    return tail >= T ? 0 : int(T - tail);
}

hipError_t launch_dispatch(const uint16_t* x, int T, int H, int k, const int32_t* pos,
                           uint16_t* send, hipStream_t s)
{
    return launch_dispatch_bounded(x, T, H, k, pos, send, uint32_t(T) * uint32_t(k), s);
}

hipError_t launch_dispatch_bounded(const uint16_t* x, int T, int H, int k, const int32_t* pos,
                                   uint16_t* send, uint32_t bound, hipStream_t s)
{
    const int nvec = H / 8;                   // 16-byte vectors per row
    // A small batch is bound by latency, not by the write path: one vector per
    // lane and an uncapped grid put the most requests in flight (measured on
    // MI355X at T=128, H=7168, k=8: 8.2 -> 5.0 us).
    const int tk = keep_from(T, H, k);       // first token whose rows stay cached
    if (small_scatter(T, H, k))
        return launch_u<1>(x, T, nvec, k, pos, send, kMaxGrid, bound, tk, s);
    const uint32_t cap = dispatch_grid_cap();
    if (nvec % (kWave * 7) == 0) return launch_u<7>(x, T, nvec, k, pos, send, cap, bound, tk, s);
    if (nvec >= kWave * 8) return launch_u<8>(x, T, nvec, k, pos, send, cap, bound, tk, s);
    if (nvec >= kWave * 4) return launch_u<4>(x, T, nvec, k, pos, send, cap, bound, tk, s);
    return launch_u<1>(x, T, nvec, k, pos, send, cap, bound, tk, s);
}

}  // namespace ep
