// route_topk.hip -- top-k gating on gfx950.
//
// HyperParallel-MoE sec. 2.2: the router picks a small subset of experts per
// token by top-k routing and the experts' outputs are weighted by the routing
// scores.  Gating is a softmax; selection runs on the raw fp32 logits (the
// softmax is monotone, so the picks are the same and stay exact).
//
// Mapping: a group of LPT lanes (a power of two <= 64) owns one token; lane g
// of the group holds logits e = i*LPT + g, i < NV, so every load instruction
// reads LPT consecutive floats (coalesced).  Each of the k rounds takes a
// local best over the lane's untaken logits and a log2(LPT)-step xor-shuffle
// reduction on (value, index): larger value first, equal values -> lower
// index.  Lane j of the group keeps pick j, so the softmax over the picks is
// one more xor-shuffle sum.  All lanes of a group see bit-identical sums
// (each butterfly level adds the same two operands, only commuted).
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

__device__ __forceinline__ bool ranks_before(float a, int ia, float b, int ib) {
    return a > b || (a == b && ia < ib);
}

template <int NV, int LPT>
__global__ __launch_bounds__(kBlock) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int normalize,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w)
{
    const int g = threadIdx.x % LPT;
    const int64_t tok = (int64_t(blockIdx.x) * kBlock + threadIdx.x) / LPT;
    if (tok >= T) return;                   // whole LPT-lane groups leave together
    const float* row = logits + tok * E;

    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = i * LPT + g;
        v[i] = e < E ? row[e] : 0.0f;
    }
    uint32_t avail = 0;                     // bit i: logit i is in range and untaken
#pragma unroll
    for (int i = 0; i < NV; ++i)
        if (i * LPT + g < E) avail |= 1u << i;

    int my_pick = 0;
    float my_val = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = 0.0f;
        int bi = -1;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = i * LPT + g;
            if (((avail >> i) & 1u) && (bi < 0 || ranks_before(v[i], e, bv, bi))) {
                bv = v[i];
                bi = e;
            }
        }
#pragma unroll
        for (int d = LPT / 2; d >= 1; d >>= 1) {
            const float ov = __shfl_xor(bv, d, LPT);
            const int oi = __shfl_xor(bi, d, LPT);
            if (oi >= 0 && (bi < 0 || ranks_before(ov, oi, bv, bi))) {
                bv = ov;
                bi = oi;
            }
        }
        if (bi % LPT == g) avail &= ~(1u << (bi / LPT));
        if (g == j) {
            my_pick = bi;
            my_val = bv;
        }
    }

    // The first pick holds the largest logit m: exp(l - m) keeps every
    // softmax ratio and cannot overflow.
    const float m = __shfl(my_val, 0, LPT);
    const float ex = g < k ? expf(my_val - m) : 0.0f;
    float denom;
    if (normalize) {
        denom = ex;
#pragma unroll
        for (int d = LPT / 2; d >= 1; d >>= 1) denom += __shfl_xor(denom, d, LPT);
    } else {
        float z = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (i * LPT + g < E) z += expf(v[i] - m);
#pragma unroll
        for (int d = LPT / 2; d >= 1; d >>= 1) z += __shfl_xor(z, d, LPT);
        denom = z;
    }
    if (g < k) {
        topk_idx[tok * k + g] = my_pick;
        topk_w[tok * k + g] = ex / denom;
    }
}

template <int NV, int LPT>
hipError_t launch_t(const float* logits, int T, int E, int k, int normalize,
                    int32_t* idx, float* w, hipStream_t s)
{
    const int64_t threads = int64_t(T) * LPT;
    const int grid = int((threads + kBlock - 1) / kBlock);
    hipLaunchKernelGGL((route_topk_kernel<NV, LPT>), dim3(grid), dim3(kBlock), 0, s,
                       logits, T, E, k, normalize, idx, w);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int normalize,
                             int32_t* idx, float* w, hipStream_t s)
{
    if (E <= 1) return launch_t<1, 1>(logits, T, E, k, normalize, idx, w, s);
    if (E <= 2) return launch_t<1, 2>(logits, T, E, k, normalize, idx, w, s);
    if (E <= 4) return launch_t<1, 4>(logits, T, E, k, normalize, idx, w, s);
    if (E <= 8) return launch_t<1, 8>(logits, T, E, k, normalize, idx, w, s);
    if (E <= 16) return launch_t<1, 16>(logits, T, E, k, normalize, idx, w, s);
    if (E <= 32) return launch_t<1, 32>(logits, T, E, k, normalize, idx, w, s);
    if (E <= 64) return launch_t<1, 64>(logits, T, E, k, normalize, idx, w, s);
    if (E <= 128) return launch_t<2, 64>(logits, T, E, k, normalize, idx, w, s);
    if (E <= 256) return launch_t<4, 64>(logits, T, E, k, normalize, idx, w, s);
    if (E <= 512) return launch_t<8, 64>(logits, T, E, k, normalize, idx, w, s);
    return launch_t<16, 64>(logits, T, E, k, normalize, idx, w, s);
}

}  // namespace ep
