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
// and weight gradients.  One workgroup (4 waves) per token: wave w walks the
// row segments w, w + 4, ... of kWave 16-byte vectors.  Per segment a lane
// loads its grad_out vector and the k expert-output vectors (all k loads in
// flight at once for the common k = 8), writes the k scaled vectors, and adds
// the 8 products g*y of each pick to that pick's running dot.  The dots then
// go through a wave butterfly and a fixed-order sum over the 4 waves, so the
// result does not depend on timing.  Products of two bf16 values are exact in
// fp32; the dot's error is that of the additions only: per lane 8 per
// segment, then 6 butterfly steps and 3 cross-wave adds.
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

__device__ __forceinline__ u32x4 scaled(const float (&g)[8], float w)
{
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        o[q] = pack_bf16x2(product_for_bf16(w, g[2 * q]), product_for_bf16(w, g[2 * q + 1]));
    return o;
}

__device__ __forceinline__ void unpack8(u32x4 v, float (&f)[8])
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f[2 * q] = bf16_lo(v[q]);
        f[2 * q + 1] = bf16_hi(v[q]);
    }
}

// One token, the compile-time pick count KC: per segment all KC expert-output
// loads are issued before the first product.
template <int KC>
__device__ __forceinline__ void token_fixed_k(const char* __restrict__ g_row,
                                              const char* __restrict__ yb,
                                              char* __restrict__ gyb,
                                              const int32_t* __restrict__ prow,
                                              const float* __restrict__ wrow, uint32_t S,
                                              int nvec, int64_t row_bytes, int wave,
                                              float (*sh)[kMaxK])
{
    int32_t p[KC];
    float wv[KC];
    float dot[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) {
        p[j] = prow[j];
        wv[j] = wrow[j];
        dot[j] = 0.0f;
    }
    const int segs = (nvec + kWave - 1) / kWave;
    for (int seg = wave; seg < segs; seg += kWavesPerBlock) {
        const int v = seg * kWave + lane_id();
        const bool lane_ok = v < nvec;
        const uint32_t off = uint32_t(v) * 16u;
        const u32x4 zero = {0, 0, 0, 0};
        float g[8];
        unpack8(lane_ok ? load16(g_row + off) : zero, g);
        u32x4 r[KC];
#pragma unroll
        for (int j = 0; j < KC; ++j)
            r[j] = (lane_ok && uint32_t(p[j]) < S)
                       ? load16_nt(yb + int64_t(p[j]) * row_bytes + off) : zero;
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            dot[j] = dot8(g, r[j], dot[j]);
            if (uint32_t(p[j]) < S && lane_ok)
                store16_coherent(buffer_rsrc(gyb + int64_t(p[j]) * row_bytes, row_bytes),
                                 int(off), scaled(g, wv[j]));
        }
    }
#pragma unroll
    for (int j = 0; j < KC; ++j) {
        const float d = wave_sum_f(dot[j]);
        if (lane_id() == 0) sh[wave][j] = d;
    }
}

// One token, runtime k: pick by pick, each over all of the wave's segments
// (the grad_out row is re-read from cache per pick).  Per lane the dot of a
// pick sums the same products in the same order as token_fixed_k.
__device__ __noinline__ void token_any_k(const char* __restrict__ g_row,
                                         const char* __restrict__ yb, char* __restrict__ gyb,
                                         const int32_t* __restrict__ prow,
                                         const float* __restrict__ wrow, int k, uint32_t S,
                                         int nvec, int64_t row_bytes, int wave,
                                         float (*sh)[kMaxK])
{
    const int segs = (nvec + kWave - 1) / kWave;
    for (int j = 0; j < k; ++j) {
        const int32_t p = prow[j];
        const float w = wrow[j];
        const bool valid = uint32_t(p) < S;
        float dot = 0.0f;
        for (int seg = wave; seg < segs; seg += kWavesPerBlock) {
            const int v = seg * kWave + lane_id();
            if (v < nvec && valid) {
                const uint32_t off = uint32_t(v) * 16u;
                float g[8];
                unpack8(load16(g_row + off), g);
                dot = dot8(g, load16_nt(yb + int64_t(p) * row_bytes + off), dot);
                store16_coherent(buffer_rsrc(gyb + int64_t(p) * row_bytes, row_bytes),
                                 int(off), scaled(g, w));
            }
        }
        dot = wave_sum_f(dot);
        if (lane_id() == 0) sh[wave][j] = dot;
    }
}

template <int KC>
__global__ __launch_bounds__(kBlock) void combine_grad_kernel(
    const uint16_t* __restrict__ grad_out, const uint16_t* __restrict__ y,
    const int32_t* __restrict__ pos, const float* __restrict__ w, int T, int nvec, int k,
    uint16_t* __restrict__ grad_y, float* __restrict__ grad_w)
{
    __shared__ float sh[kWavesPerBlock][kMaxK];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const uint32_t S = uint32_t(T) * uint32_t(k);
    const int64_t row_bytes = int64_t(nvec) * 16;
    const char* yb = reinterpret_cast<const char*>(y);
    char* gyb = reinterpret_cast<char*>(grad_y);
    for (int t = blockIdx.x; t < T; t += gridDim.x) {
        const char* g_row = reinterpret_cast<const char*>(grad_out) + int64_t(t) * row_bytes;
        const int32_t* prow = pos + int64_t(t) * k;
        const float* wrow = w + int64_t(t) * k;
        if constexpr (KC > 0)
            token_fixed_k<KC>(g_row, yb, gyb, prow, wrow, S, nvec, row_bytes, wave, sh);
        else
            token_any_k(g_row, yb, gyb, prow, wrow, k, S, nvec, row_bytes, wave, sh);
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

}  // namespace

hipError_t launch_combine_grad(const uint16_t* grad_out, const uint16_t* y,
                               const int32_t* pos, const float* w, int T, int H, int k,
                               uint16_t* grad_y, float* grad_w, hipStream_t s)
{
    const uint32_t grid = uint32_t(T) < kMaxGrid ? uint32_t(T) : kMaxGrid;
    const int nvec = H / 8;
    if (k == 8)
        EP_LAUNCH((combine_grad_kernel<8>), dim3(grid), dim3(kBlock), 0, s,
                  grad_out, y, pos, w, T, nvec, k, grad_y, grad_w);
    else
        EP_LAUNCH((combine_grad_kernel<0>), dim3(grid), dim3(kBlock), 0, s,
                  grad_out, y, pos, w, T, nvec, k, grad_y, grad_w);
    return hipGetLastError();
}

}  // namespace ep
