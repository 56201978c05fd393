// ep_combine_dev.h -- the combine arithmetic shared by ep_combine
// (combine.hip) and the fused flag-in-payload mode (fused.hip), so the two
// produce bit-identical outputs: per output element, an fp32 product for pick
// 0, then fused multiply-adds for picks 1..k-1 in order, then one
// round-to-nearest-even to bf16 (HyperParallel-MoE sec. 4.1: the top-k
// contributions are accumulated according to the routing scores).
#pragma once

#include "ep_device.h"

namespace ep {

// acc[u][0..7] (+)= wj * the 8 bf16 values of 16-byte vector r[u].
template <int U>
__device__ __forceinline__ void accumulate(float (&acc)[U][8], const u32x4 (&r)[U],
                                           float wj, bool first)
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float lo = bf16_lo(r[u][q]);
            const float hi = bf16_hi(r[u][q]);
            if (first) {
                acc[u][2 * q] = wj * lo;
                acc[u][2 * q + 1] = wj * hi;
            } else {
                acc[u][2 * q] = __builtin_fmaf(wj, lo, acc[u][2 * q]);
                acc[u][2 * q + 1] = __builtin_fmaf(wj, hi, acc[u][2 * q + 1]);
            }
        }
    }
}

// Rounds acc[u][0..7] to bf16 and stores vector u at byte offset
// off + u*kWave*16 of the row that descriptor `row` covers, streaming and
// agent-coherent (written through the L2, so no dirty output lines are left
// for the next kernel to wait on).
template <int U>
__device__ __forceinline__ void store_acc_coherent(__amdgpu_buffer_rsrc_t row, uint32_t off,
                                                   const float (&acc)[U][8])
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[u][2 * q], acc[u][2 * q + 1]);
        store16_coherent(row, int(off) + u * kWave * 16, o);
    }
}

// Rounds acc[u][0..7] to bf16 and stores vector u at dst + u*kWave*16.
template <int U>
__device__ __forceinline__ void store_acc(char* __restrict__ dst, const float (&acc)[U][8])
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[u][2 * q], acc[u][2 * q + 1]);
        store16(dst + u * kWave * 16, o);
    }
}

}  // namespace ep
