// combine.hip -- top-k weighted gather-reduce back to token order.
//
// HyperParallel-MoE sec. 4.1: the top-k expert contributions of a token are
// accumulated according to its routing scores; RailWave "System Design"
// (Fig. 3): combine returns outputs to their original token positions with
// the metadata dispatch saved.  Here:
//   out[t] = bf16( sum_j w[t][j] * y[pos[t][j]] ),
// fp32 accumulation in the fixed order j = 0..k-1 (a product, then fused
// multiply-adds), one round-to-nearest-even to bf16 at the end.
//
// HBM-bound gather (k reads, 1 write per row).  A wave works on (token, row
// segment) items: per pick it issues coalesced 16-byte loads per lane from
// row pos[t][j]; the k row indices and weights are wave-uniform scalar loads.
// For the common k = 8 the pick loop is unrolled so all 8 loads of a lane
// can be in flight before the first FMA.  Large batches run batched
// (combine_batched_kernel: a batch's results are held in registers and
// stored together, so reads and writes do not interleave item by item);
// small batches and ragged rows take one item per wave (combine_kernel).
// The row loads are nontemporal: each expert-output row is read exactly
// once, and keeping them out of the Infinity Cache leaves it to the data the
// next kernels re-read (measured on MI355X at T=4096, H=7168, k=8: combine
// 108 -> 97 us and the following dispatch 111 -> 95 us).  The output rows
// are stored streaming and agent-coherent, through a descriptor over the
// token's row, so they do not stay dirty in the L2 for the next kernel to
// flush.
//
// The same kernel with every weight 1 is the backward of dispatch
// (HyperParallel-MoE sec. 2.2, Fig. 2(b): the backward Combine returns the
// input activations' gradient): x[t] went to every row pos[t][j], so
// grad_x[t] = bf16( sum_j grad_send[pos[t][j]] ), same order and rounding.
#include "ep_combine_dev.h"
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kWavesPerBlock = kBlock / kWave;
// With a runtime pick count, the row loads of this many picks are issued
// together before their FMAs (8 spills the batched kernel's registers).
constexpr int kPickGroup = 4;

template <int U>
__device__ __forceinline__ void load_pick(u32x4 (&r)[U], const char* __restrict__ y,
                                          int32_t p, uint32_t S, int64_t row_bytes,
                                          uint32_t lane_off)
{
    if (uint32_t(p) < S) {
        const char* src = y + int64_t(p) * row_bytes + lane_off;
#pragma unroll
        for (int u = 0; u < U; ++u) r[u] = load16_nt(src + u * kWave * 16);
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) r[u] = u32x4{0, 0, 0, 0};
    }
}

// A (token, segment) item whose vectors all lie inside the row.  KC > 0: the
// pick count is the compile-time KC, so all KC*U loads of a lane are issued
// before the first FMA; KC == 0: runtime k, one pick at a time.  UW: every
// weight is 1 and wrow is not read.
template <int U, int KC, bool UW>
__device__ __forceinline__ void combine_whole(const char* __restrict__ y,
                                              const int32_t* __restrict__ prow,
                                              const float* __restrict__ wrow, int k,
                                              uint32_t S, int64_t row_bytes,
                                              uint32_t lane_off, char* __restrict__ dst)
{
    float acc[U][8];
    if constexpr (KC > 0) {
        u32x4 r[KC][U];
#pragma unroll
        for (int j = 0; j < KC; ++j) load_pick<U>(r[j], y, prow[j], S, row_bytes, lane_off);
#pragma unroll
        for (int j = 0; j < KC; ++j) accumulate<U>(acc, r[j], UW ? 1.0f : wrow[j], j == 0);
    } else {
        // runtime k: kPickGroup picks' loads go out together (one memory round
        // trip per group, not per pick), then their FMAs in pick order
        for (int j0 = 0; j0 < k; j0 += kPickGroup) {
            u32x4 r[kPickGroup][U];
#pragma unroll
            for (int q = 0; q < kPickGroup; ++q)
                if (j0 + q < k) load_pick<U>(r[q], y, prow[j0 + q], S, row_bytes, lane_off);
#pragma unroll
            for (int q = 0; q < kPickGroup; ++q)
                if (j0 + q < k) accumulate<U>(acc, r[q], UW ? 1.0f : wrow[j0 + q], j0 + q == 0);
        }
    }
    store_acc_coherent<U>(buffer_rsrc(dst, row_bytes), lane_off, acc);
}

// The last, partial segment of a row: one vector at a time.  UW: every
// weight is 1 and wrow is not read.
template <bool UW>
__device__ __noinline__ void combine_tail(const char* __restrict__ y,
                                          const int32_t* __restrict__ prow,
                                          const float* __restrict__ wrow, int k, uint32_t S,
                                          int64_t row_bytes, int v0, int U, int nvec,
                                          char* __restrict__ dst)
{
    for (int u = 0; u < U; ++u) {
        const int vi = v0 + u * kWave;
        if (vi >= nvec) break;
        const uint32_t off = uint32_t(vi) * 16u;
        float acc[1][8];
        for (int j = 0; j < k; ++j) {
            u32x4 r[1];
            load_pick<1>(r, y, prow[j], S, row_bytes, off);
            accumulate<1>(acc, r, UW ? 1.0f : wrow[j], j == 0);
        }
        store_acc<1>(dst + off, acc);
    }
}

// Work items are (group of 4 tokens, row segment of kWave*U vectors) pairs,
// one wave per token, numbered segment-fastest: the workgroups resident at
// one time read whole expert-output rows and write whole output rows
// (measured on MI355X at T=4096, H=7168, k=8: about 4 us less than
// token-fastest order).  A 1-D grid strides over the items, so any T fits the
// launch limits.
template <int U, int KC, bool UW>
__global__ __launch_bounds__(kBlock) void combine_kernel(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ pos,
    const float* __restrict__ w, int T, int nvec, int k,
    uint16_t* __restrict__ out, uint32_t segs, uint32_t items)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t S = uint32_t(T) * uint32_t(k);
    const int64_t row_bytes = int64_t(nvec) * 16;
    const char* yb = reinterpret_cast<const char*>(y);
    for (uint32_t b = blockIdx.x; b < items; b += gridDim.x) {
        const uint32_t group = b / segs;
        const int seg = int(b - group * segs);
        const int t = int(group) * kWavesPerBlock + wave;
        if (t >= T) continue;
        const int32_t* prow = pos + int64_t(t) * k;
        const float* wrow = UW ? nullptr : w + int64_t(t) * k;
        char* dst = reinterpret_cast<char*>(out) + int64_t(t) * row_bytes;
        const int v0 = seg * kWave * U + lane_id();
        if ((seg + 1) * kWave * U <= nvec)
            combine_whole<U, KC, UW>(yb, prow, wrow, k, S, row_bytes, uint32_t(v0) * 16u, dst);
        else
            combine_tail<UW>(yb, prow, wrow, k, S, row_bytes, v0, U, nvec, dst);
    }
}

// ---------------------------------------------------------------- batched
// Large batches: a persistent grid of one workgroup per CU; wave gw of the NW
// waves takes items (token t, 1 KiB row segment s), numbered t*segs + s, in
// batches: batch m holds items m*B*NW + i*NW + gw for i < B.  The B items of
// a batch are all read and reduced first, their packed bf16 results held in
// registers, and only then stored.  Across the GPU the waves move through
// the batches together, so the output writes come in bursts between long
// runs of gathered reads instead of being interleaved with them (measured on
// MI355X at T=4096, H=7168, k=8: the expert-output reads alone take 68 us
// and the output writes alone 10 us, but 89-90 us when interleaved item by
// item; in batches of 28 on one workgroup per CU, 82-83 us).
//
// The batched path takes rows of whole 1 KiB segments (H % 512 == 0).
// Before a batch the wave's lanes check all of its picks against [0, S), 64
// at a time; a full batch with every pick inside runs with no per-pick
// condition (28 items' uniform conditions held at once would spill the
// scalar registers), any other batch checks each pick, and a pick outside
// counts as a row of zeros, exactly as in combine_kernel.
constexpr int kBatch = 28;

template <bool CHECK>
__device__ __forceinline__ u32x4 load_row_nt(const char* __restrict__ y, int32_t p, uint32_t S,
                                             int64_t row_bytes, uint32_t off)
{
    if (CHECK && uint32_t(p) >= S) return u32x4{0, 0, 0, 0};
    return load16_nt(y + int64_t(p) * row_bytes + off);
}

template <int KC, bool UW, bool CHECK>
__device__ __forceinline__ u32x4 reduce_item(const char* __restrict__ y,
                                             const int32_t* __restrict__ prow,
                                             const float* __restrict__ wrow, int k, uint32_t S,
                                             int64_t row_bytes, uint32_t off)
{
    float acc[1][8];
    if constexpr (KC > 0) {
        u32x4 r[KC][1];
#pragma unroll
        for (int j = 0; j < KC; ++j) r[j][0] = load_row_nt<CHECK>(y, prow[j], S, row_bytes, off);
#pragma unroll
        for (int j = 0; j < KC; ++j) accumulate<1>(acc, r[j], UW ? 1.0f : wrow[j], j == 0);
    } else {
        // runtime k: kPickGroup picks' loads go out together (one memory round
        // trip per group, not per pick), then their FMAs in pick order
        for (int j0 = 0; j0 < k; j0 += kPickGroup) {
            u32x4 r[kPickGroup][1];
#pragma unroll
            for (int q = 0; q < kPickGroup; ++q)
                if (j0 + q < k) r[q][0] = load_row_nt<CHECK>(y, prow[j0 + q], S, row_bytes, off);
#pragma unroll
            for (int q = 0; q < kPickGroup; ++q)
                if (j0 + q < k)
                    accumulate<1>(acc, r[q], UW ? 1.0f : wrow[j0 + q], j0 + q == 0);
        }
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[0][2 * q], acc[0][2 * q + 1]);
    return o;
}

template <int KC, bool UW, bool CHECK>
__device__ __forceinline__ u32x4 batch_item(const char* __restrict__ y,
                                            const int32_t* __restrict__ pos,
                                            const float* __restrict__ w, int k, uint32_t S,
                                            int64_t row_bytes, uint32_t segs, uint32_t it)
{
    const uint32_t t = it / segs, seg = it - t * segs;
    const uint32_t off = (seg * kWave + uint32_t(lane_id())) * 16u;
    return reduce_item<KC, UW, CHECK>(y, pos + int64_t(t) * k, UW ? nullptr : w + int64_t(t) * k,
                                      k, S, row_bytes, off);
}

__device__ __forceinline__ void batch_store(char* __restrict__ out, int64_t row_bytes,
                                            uint32_t segs, uint32_t it, u32x4 o)
{
    const uint32_t t = it / segs, seg = it - t * segs;
    store16_coherent(buffer_rsrc(out + int64_t(t) * row_bytes, row_bytes),
                     int((seg * kWave + uint32_t(lane_id())) * 16u), o);
}

// items + kBatch * (waves in the grid) < 2^32 (checked on the host).
template <int KC, bool UW>
__global__ __launch_bounds__(kBlock) void combine_batched_kernel(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ pos,
    const float* __restrict__ w, int T, int nvec, int k,
    uint16_t* __restrict__ out, uint32_t segs, uint32_t items)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t nw = gridDim.x * kWavesPerBlock;
    const uint32_t gw = blockIdx.x * kWavesPerBlock + uint32_t(wave);
    const uint32_t S = uint32_t(T) * uint32_t(k);
    const int64_t row_bytes = int64_t(nvec) * 16;
    const char* yb = reinterpret_cast<const char*>(y);
    char* ob = reinterpret_cast<char*>(out);
    for (uint32_t base = gw; base < items; base += kBatch * nw) {
        u32x4 o[kBatch];
        bool bad = false;
        for (int c = lane_id(); c < kBatch * k; c += kWave) {
            const uint32_t it = base + uint32_t(c / k) * nw;
            if (it < items) bad |= uint32_t(pos[int64_t(it / segs) * k + c % k]) >= S;
        }
        if (base + (kBatch - 1) * nw < items && ballot(bad) == 0) {
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                o[i] = batch_item<KC, UW, false>(yb, pos, w, k, S, row_bytes, segs, base + i * nw);
#pragma unroll
            for (int i = 0; i < kBatch; ++i) batch_store(ob, row_bytes, segs, base + i * nw, o[i]);
        } else {
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                if (base + i * nw < items)
                    o[i] = batch_item<KC, UW, true>(yb, pos, w, k, S, row_bytes, segs, base + i * nw);
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                if (base + i * nw < items) batch_store(ob, row_bytes, segs, base + i * nw, o[i]);
        }
    }
}

template <bool UW>
hipError_t launch_batched(const uint16_t* y, const int32_t* pos, const float* w, int T,
                          int nvec, int k, uint16_t* out, uint32_t grid, hipStream_t s)
{
    const uint32_t segs = uint32_t(nvec / kWave);
    const uint32_t items = uint32_t(T) * segs;
    // The common top-k values get a compile-time pick count: every pick's
    // load of an item is then unrolled, and the compiler overlaps the loads
    // of neighbouring items (measured on MI355X at T=4096, H=7168: runtime k
    // at k=6 took 120 us).
#define EP_BATCHED(KC) EP_LAUNCH((combine_batched_kernel<KC, UW>), dim3(grid), dim3(kBlock), 0, s, \
                                 y, pos, w, T, nvec, k, out, segs, items)
    switch (k) {
        case 8: EP_BATCHED(8); break;
        case 6: EP_BATCHED(6); break;
        case 4: EP_BATCHED(4); break;
        case 2: EP_BATCHED(2); break;
        default: EP_BATCHED(0); break;
    }
#undef EP_BATCHED
    return hipGetLastError();
}

template <int U, bool UW>
hipError_t launch_u(const uint16_t* y, const int32_t* pos, const float* w, int T,
                    int nvec, int k, uint16_t* out, hipStream_t s)
{
    const uint32_t segs = uint32_t((nvec + kWave * U - 1) / (kWave * U));
    const uint32_t items = uint32_t((T + kWavesPerBlock - 1) / kWavesPerBlock) * segs;
    const uint32_t grid = items < kMaxGrid ? items : kMaxGrid;
#define EP_ITEMS(KC) EP_LAUNCH((combine_kernel<U, KC, UW>), dim3(grid), dim3(kBlock), 0, s, \
                               y, pos, w, T, nvec, k, out, segs, items)
    switch (k) {
        case 8: EP_ITEMS(8); break;
        case 6: EP_ITEMS(6); break;
        case 4: EP_ITEMS(4); break;
        case 2: EP_ITEMS(2); break;
        default: EP_ITEMS(0); break;
    }
#undef EP_ITEMS
    return hipGetLastError();
}

// The batched kernel's preconditions: rows of whole 1 KiB segments and
// 32-bit item indexes with room for a batch past the end.
bool batchable(int T, int H, uint32_t grid)
{
    if (grid == 0 || (H / 8) % kWave != 0) return false;
    const uint64_t items = uint64_t(T) * uint64_t(H / 8 / kWave);
    const uint64_t span = uint64_t(kBatch) * grid * kWavesPerBlock;
    return items + span < (uint64_t(1) << 32);
}

// Gathers reading more than kSmallScatterBytes run batched where the rows
// allow it, on two workgroups per CU when every wave then takes a single
// batch, else on one; smaller ones are latency-bound and take the
// one-item-per-wave kernel on an uncapped grid.  Measured on MI355X, A/B on
// one box: T=4096, H=7168, k=8 (57,344 items: one round of 28-item batches
// on 512 workgroups, two on 256) combine 82.1-82.4 -> 79.0-79.2 us and
// 85.2 -> 82.9-83.2 us on two boxes; T=16384 (four rounds against eight)
// 328.6-329.2 -> 362.4-364.2 us, so a batch that needs more than one round
// stays on one workgroup per CU.  The unit-weight gather (dispatch_grad)
// moved 86.9-87.0 -> 87.6-89.2 us at T=4096, H=7168 and 49.4-49.6 ->
// 46.9-47.2 us at H=4096.
template <bool UW>
hipError_t launch_gather(const uint16_t* y, const int32_t* pos, const float* w, int T, int H,
                         int k, uint16_t* out, hipStream_t s)
{
    const uint32_t cus = device_cu_count();
    const uint64_t items = uint64_t(T) * uint64_t(H / 8 / kWave);
    const bool one_round = items <= uint64_t(kBatch) * 2 * cus * kWavesPerBlock;
    const uint32_t grid = one_round ? 2 * cus : cus;
    if (!small_scatter(T, H, k) && batchable(T, H, grid))
        return launch_batched<UW>(y, pos, w, T, H / 8, k, out, grid, s);
    // One vector per lane and pick: more, smaller items keep more waves
    // resident than two (measured at H=7168: about 1 us faster).
    return launch_u<1, UW>(y, pos, w, T, H / 8, k, out, s);
}

}  // namespace

hipError_t launch_combine_batched(const uint16_t* y, const int32_t* pos, const float* w, int T,
                                  int H, int k, uint16_t* out, uint32_t grid, hipStream_t s)
{
    if (!batchable(T, H, grid)) return hipErrorInvalidValue;
    return w ? launch_batched<false>(y, pos, w, T, H / 8, k, out, grid, s)
             : launch_batched<true>(y, pos, nullptr, T, H / 8, k, out, grid, s);
}

hipError_t launch_combine(const uint16_t* y, const int32_t* pos, const float* w,
                          int T, int H, int k, uint16_t* out, hipStream_t s)
{
    return launch_gather<false>(y, pos, w, T, H, k, out, s);
}

hipError_t launch_dispatch_grad(const uint16_t* grad_send, const int32_t* pos, int T, int H,
                                int k, uint16_t* grad_x, hipStream_t s)
{
    return launch_gather<true>(grad_send, pos, nullptr, T, H, k, grad_x, s);
}

}  // namespace ep
