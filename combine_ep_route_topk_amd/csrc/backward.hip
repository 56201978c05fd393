// backward.hip -- backward of combine: the gradients of the expert outputs
// and of the routing weights.
//
// HyperParallel-MoE sec. 2.2, Fig. 2(b): in the backward graph the backward
// Dispatch is the gradient of the forward Combine.  With the forward
// out[t] = sum_j w[t][j] * y[pos[t][j]]:
//   grad_y[pos[t][j]] = bf16( w[t][j] * grad_out[t] )   the exact product,
//                                                       rounded once (RNE);
//   grad_w[t][j]      = sum_h grad_out[t][h] * y[pos[t][j]][h]   in fp32.
// (The backward of dispatch is the unit-weight combine in combine.hip.)
//
// HBM-bound: per token one grad_out row and k expert-output rows are read and
// k gradient rows written, 2H(1 + 2k) bytes, plus 12k bytes of pos, weights
// and weight gradients.  Two launches, because one kernel that mixes the
// gathered reads of y with the scattered writes of grad_y runs well below
// either half on its own (measured on MI355X at T=4096, H=7168, k=8: one
// kernel 197 us; its read half 80 us, its write half 98 us at the same grid):
//   1. dots: one workgroup (4 waves) per token reads grad_out[t] and its k
//      rows and writes grad_w -- reads only, a grid as large as the token count;
//   2. scatter: grad_y[pos[t][j]] = w * grad_out[t], shaped like dispatch (a
//      wave per (token, row segment) item, segment-fastest, a grid capped
//      below the CU count: fewer concurrent streams of scattered row writes),
//      reading grad_out again, from the Infinity Cache where it fits.
// Measured at that shape: dots 79 us, scatter 91 us, 172 us for the pair.

#include "ep_combine_dev.h"
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kWavesPerBlock = kBlock / kWave;

// An f32 that rounds to the same bf16 as the exact product w*g.  The f32
// product p is rounded once already; rounding p to bf16 can go the wrong way
// only when p lies exactly half-way between two bf16 values while the exact
// product does not.  The FMA gives the exact remainder e = w*g - p (for
// products in the normal f32 range), and moving p one f32 step toward the
// exact product in that case makes the bf16 rounding break the tie the way
// the exact value does.
__device__ __forceinline__ float product_for_bf16(float w, float g)
{
    const float p = w * g;
    const float e = __builtin_fmaf(w, g, -p);
    uint32_t b = __float_as_uint(p);
    if ((b & 0xFFFFu) == 0x8000u && e != 0.0f)
        b += ((__float_as_uint(e) ^ b) >> 31) ? 0xFFFFFFFFu : 1u;   // toward the exact value
    return __uint_as_float(b);
}

__device__ __forceinline__ float wave_sum_f(float v)
{
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

// dot += the 8 products of the bf16 vectors g and y, in element order.
__device__ __forceinline__ float dot8(const float (&g)[8], u32x4 y, float dot)
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        dot = __builtin_fmaf(g[2 * q], bf16_lo(y[q]), dot);
        dot = __builtin_fmaf(g[2 * q + 1], bf16_hi(y[q]), dot);
    }
    return dot;
}

__device__ __forceinline__ void unpack8(u32x4 v, float (&f)[8])
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f[2 * q] = bf16_lo(v[q]);
        f[2 * q + 1] = bf16_hi(v[q]);
    }
}

// w * g[0..7] rounded to bf16 as the exact products would be.  Fast path: the
// f32 products, and a check whether any lane's product sits on a bf16 tie
// (low 16 bits 0x8000, about one product in 65536); only then does the wave
// redo the vector with product_for_bf16.
__device__ __forceinline__ u32x4 scaled(const float (&g)[8], float w)
{
    float p[8];
    bool tie = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        p[e] = w * g[e];
        tie |= uint16_t(__float_as_uint(p[e])) == 0x8000u;
    }
    if (ballot(tie) != 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = product_for_bf16(w, g[e]);
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(p[2 * q], p[2 * q + 1]);
    return o;
}

// ------------------------------------------------------------ 1. dots
// One token, the compile-time pick count KC: per segment all KC loads of a
// lane are issued before the first product.  Lanes past the row end and
// picks outside the buffer read zeros.
template <int KC>
__device__ __forceinline__ void dots_fixed_k(const char* __restrict__ g_row,
                                             const char* __restrict__ yb,
                                             const int32_t* __restrict__ prow, uint32_t S,
                                             int nvec, int64_t row_bytes, int wave,
                                             float (*sh)[kMaxK])
{
    int32_t p[KC];
    float dot[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) {
        p[j] = prow[j];
        dot[j] = 0.0f;
    }
    const u32x4 zero = {0, 0, 0, 0};
    const int segs = (nvec + kWave - 1) / kWave;
    for (int seg = wave; seg < segs; seg += kWavesPerBlock) {
        const int v = seg * kWave + lane_id();
        const bool lane_ok = v < nvec;
        const int64_t off = int64_t(v) * 16;
        float g[8];
        unpack8(lane_ok ? load16(g_row + off) : zero, g);
        u32x4 r[KC];
#pragma unroll
        for (int j = 0; j < KC; ++j)
            r[j] = (lane_ok && uint32_t(p[j]) < S) ? load16_nt(yb + int64_t(p[j]) * row_bytes + off)
                                                   : zero;
#pragma unroll
        for (int j = 0; j < KC; ++j) dot[j] = dot8(g, r[j], dot[j]);
    }
#pragma unroll
    for (int j = 0; j < KC; ++j) {
        const float d = wave_sum_f(dot[j]);
        // a pick outside [0, S) gets exactly 0, even where grad_out holds an
        // infinity (whose product with the zero row would be NaN)
        if (lane_id() == 0) sh[wave][j] = uint32_t(p[j]) < S ? d : 0.0f;
    }
}

// One token, runtime k: picks in groups of kDotGroup, each group over all of
// the wave's segments, its row loads issued together (the grad_out row is
// re-read from cache per group).  Per lane the dot of a pick sums the same
// products in the same order as dots_fixed_k; a pick outside [0, S) adds
// nothing and gets 0.
constexpr int kDotGroup = 4;

__device__ __noinline__ void dots_any_k(const char* __restrict__ g_row,
                                        const char* __restrict__ yb,
                                        const int32_t* __restrict__ prow, int k, uint32_t S,
                                        int nvec, int64_t row_bytes, int wave,
                                        float (*sh)[kMaxK])
{
    const u32x4 zero = {0, 0, 0, 0};
    const int segs = (nvec + kWave - 1) / kWave;
    for (int j0 = 0; j0 < k; j0 += kDotGroup) {
        int32_t p[kDotGroup];
        bool valid[kDotGroup];
        float dot[kDotGroup];
#pragma unroll
        for (int q = 0; q < kDotGroup; ++q) {
            p[q] = j0 + q < k ? prow[j0 + q] : -1;
            valid[q] = uint32_t(p[q]) < S;
            dot[q] = 0.0f;
        }
        for (int seg = wave; seg < segs; seg += kWavesPerBlock) {
            const int v = seg * kWave + lane_id();
            const bool lane_ok = v < nvec;
            const int64_t off = int64_t(v) * 16;
            float g[8];
            unpack8(lane_ok ? load16(g_row + off) : zero, g);
            u32x4 r[kDotGroup];
#pragma unroll
            for (int q = 0; q < kDotGroup; ++q)
                r[q] = (lane_ok && valid[q]) ? load16_nt(yb + int64_t(p[q]) * row_bytes + off)
                                             : zero;
#pragma unroll
            for (int q = 0; q < kDotGroup; ++q)
                if (valid[q] && lane_ok) dot[q] = dot8(g, r[q], dot[q]);
        }
#pragma unroll
        for (int q = 0; q < kDotGroup; ++q) {
            if (j0 + q >= k) break;
            const float d = wave_sum_f(dot[q]);
            if (lane_id() == 0) sh[wave][j0 + q] = valid[q] ? d : 0.0f;
        }
    }
}

// A workgroup per token (grid-stride): the 4 waves' dots, summed in wave
// order, so the result does not depend on timing.
template <int KC>
__global__ __launch_bounds__(kBlock) void combine_grad_dot_kernel(
    const uint16_t* __restrict__ grad_out, const uint16_t* __restrict__ y,
    const int32_t* __restrict__ pos, int T, int nvec, int k, float* __restrict__ grad_w)
{
    __shared__ float sh[kWavesPerBlock][kMaxK];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const uint32_t S = uint32_t(T) * uint32_t(k);
    const int64_t row_bytes = int64_t(nvec) * 16;
    const char* yb = reinterpret_cast<const char*>(y);
    for (int t = blockIdx.x; t < T; t += gridDim.x) {
        const char* g_row = reinterpret_cast<const char*>(grad_out) + int64_t(t) * row_bytes;
        const int32_t* prow = pos + int64_t(t) * k;
        if constexpr (KC > 0)
            dots_fixed_k<KC>(g_row, yb, prow, S, nvec, row_bytes, wave, sh);
        else
            dots_any_k(g_row, yb, prow, k, S, nvec, row_bytes, wave, sh);
        __syncthreads();
        if (tid < k) {
            float s = sh[0][tid];
#pragma unroll
            for (int q = 1; q < kWavesPerBlock; ++q) s += sh[q][tid];
            grad_w[int64_t(t) * k + tid] = s;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ 2. scatter
// One (token, segment) item whose vectors all lie inside the row: U loads
// per lane, then per pick U scaled vectors stored through a descriptor over
// the destination row (streaming, agent-coherent).
template <int U, bool KEEP>
__device__ __forceinline__ void scatter_whole(const char* __restrict__ g_row,
                                              char* __restrict__ gyb, int64_t row_bytes,
                                              const int32_t* __restrict__ prow,
                                              const float* __restrict__ wrow, int k,
                                              uint32_t S, int v0)
{
    const uint32_t lane_off = uint32_t(v0) * 16u;
    float g[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) unpack8(load16(g_row + lane_off + u * kWave * 16), g[u]);
    for (int j = 0; j < k; ++j) {
        const int32_t p = prow[j];
        if (uint32_t(p) >= S) continue;
        const float w = wrow[j];
        const __amdgpu_buffer_rsrc_t row = buffer_rsrc(gyb + int64_t(p) * row_bytes, row_bytes);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // KEEP: rows that dispatch_grad reads next while still cached
            const int off = int(lane_off) + u * kWave * 16;
            if constexpr (KEEP) store16_coherent_keep(row, off, scaled(g[u], w));
            else store16_coherent(row, off, scaled(g[u], w));
        }
    }
}

// The last, partial segment of a row: one vector at a time.
__device__ __noinline__ void scatter_tail(const char* __restrict__ g_row,
                                          char* __restrict__ gyb, int64_t row_bytes,
                                          const int32_t* __restrict__ prow,
                                          const float* __restrict__ wrow, int k, uint32_t S,
                                          int v0, int U, int nvec, bool keep)
{
    for (int u = 0; u < U; ++u) {
        const int vi = v0 + u * kWave;
        const bool lane_ok = vi < nvec;
        if (ballot(lane_ok) == 0) break;
        const u32x4 zero = {0, 0, 0, 0};
        float g[8];
        unpack8(lane_ok ? load16(g_row + int64_t(vi) * 16) : zero, g);
        for (int j = 0; j < k; ++j) {
            const int32_t p = prow[j];
            if (uint32_t(p) >= S) continue;
            const u32x4 o = scaled(g, wrow[j]);      // every lane: scaled() votes
            char* d = gyb + int64_t(p) * row_bytes + int64_t(vi) * 16;
            if (lane_ok) {
                if (keep) store16(d, o);
                else store16_nt(d, o);
            }
        }
    }
}

// Items are (group of 4 tokens, row segment of kWave*U vectors), one wave per
// token, numbered segment-fastest, as in dispatch.
template <int U, bool KEEP>
__global__ __launch_bounds__(kBlock) void combine_grad_scatter_kernel(
    const uint16_t* __restrict__ grad_out, const int32_t* __restrict__ pos,
    const float* __restrict__ w, int T, int nvec, int k, uint16_t* __restrict__ grad_y,
    uint32_t segs, uint32_t items)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t S = uint32_t(T) * uint32_t(k);
    const int64_t row_bytes = int64_t(nvec) * 16;
    char* gyb = reinterpret_cast<char*>(grad_y);
    for (uint32_t b = blockIdx.x; b < items; b += gridDim.x) {
        const uint32_t group = b / segs;
        const int seg = int(b - group * segs);
        const int t = int(group) * kWavesPerBlock + wave;
        if (t >= T) continue;
        const char* g_row = reinterpret_cast<const char*>(grad_out) + int64_t(t) * row_bytes;
        const int32_t* prow = pos + int64_t(t) * k;
        const float* wrow = w + int64_t(t) * k;
        const int v0 = seg * kWave * U + lane_id();
        if ((seg + 1) * kWave * U <= nvec)
            scatter_whole<U, KEEP>(g_row, gyb, row_bytes, prow, wrow, k, S, v0);
        else
            scatter_tail(g_row, gyb, row_bytes, prow, wrow, k, S, v0, U, nvec, KEEP);
    }
}

template <int U>
hipError_t launch_scatter(const uint16_t* grad_out, const int32_t* pos, const float* w, int T,
                          int nvec, int k, uint16_t* grad_y, uint32_t cap, bool keep,
                          hipStream_t s)
{
    const uint32_t segs = uint32_t((nvec + kWave * U - 1) / (kWave * U));
    const uint32_t items = uint32_t((T + kWavesPerBlock - 1) / kWavesPerBlock) * segs;
    // the fewest rounds of items that cap allows, spread evenly over the
    // smallest grid that keeps that many rounds: no nearly idle last round
    const uint32_t rounds = (items + cap - 1) / cap;
    const uint32_t grid = (items + rounds - 1) / rounds;
    if (keep)
        EP_LAUNCH((combine_grad_scatter_kernel<U, true>), dim3(grid), dim3(kBlock), 0, s, grad_out,
                  pos, w, T, nvec, k, grad_y, segs, items);
    else
        EP_LAUNCH((combine_grad_scatter_kernel<U, false>), dim3(grid), dim3(kBlock), 0, s, grad_out,
                  pos, w, T, nvec, k, grad_y, segs, items);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine_grad(const uint16_t* grad_out, const uint16_t* y,
                               const int32_t* pos, const float* w, int T, int H, int k,
                               uint16_t* grad_y, float* grad_w, hipStream_t s)
{
    const int nvec = H / 8;
    const uint32_t grid = uint32_t(T) < kMaxGrid ? uint32_t(T) : kMaxGrid;
    // The common top-k values get a compile-time pick count, so each lane's
    // row loads of all picks are in flight together; any other k goes pick
    // by pick.
#define EP_DOT(KC) EP_LAUNCH((combine_grad_dot_kernel<KC>), dim3(grid), dim3(kBlock), 0, s, \
                             grad_out, y, pos, T, nvec, k, grad_w)
    switch (k) {
        case 8: EP_DOT(8); break;
        case 6: EP_DOT(6); break;
        case 4: EP_DOT(4); break;
        case 2: EP_DOT(2); break;
        default: EP_DOT(0); break;
    }
#undef EP_DOT
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // At most thirteen sixteenths of the CU count, in even rounds: the
    // per-element multiply and tie check need more waves than dispatch's plain
    // copy to keep the write path busy, and a nearly idle last round of items
    // costs as much as a full one (measured on MI355X at T=4096, H=7168, k=8,
    // the whole combine_grad, 2048 items, fixed grids: 160 workgroups 183 us,
    // 176 178 us, 192 173.9-178.5 us (11 rounds, 128 busy in the last), 200
    // 179 us (48 busy), 208 172.3-173.8 us (10 rounds, 176 busy), 216 176 us,
    // 224 176.7-176.9 us (32 busy)).
    // a small batch: one vector per lane on an uncapped grid, as in dispatch
    const bool keep = keep_rows(T, H, k);
    if (small_scatter(T, H, k))
        return launch_scatter<1>(grad_out, pos, w, T, nvec, k, grad_y, kMaxGrid, keep, s);
    const uint32_t cap = scatter_grid_cap();
    if (nvec % (kWave * 7) == 0)
        return launch_scatter<7>(grad_out, pos, w, T, nvec, k, grad_y, cap, keep, s);
    if (nvec >= kWave * 8)
        return launch_scatter<8>(grad_out, pos, w, T, nvec, k, grad_y, cap, keep, s);
    if (nvec >= kWave * 4)
        return launch_scatter<4>(grad_out, pos, w, T, nvec, k, grad_y, cap, keep, s);
    return launch_scatter<1>(grad_out, pos, w, T, nvec, k, grad_y, cap, keep, s);
}

}  // namespace ep
