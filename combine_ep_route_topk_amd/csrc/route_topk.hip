// route_topk.hip -- top-k gating on gfx950.
//
// HyperParallel-MoE sec. 2.2: the router picks a small subset of experts per
// token by top-k routing and the experts' outputs are weighted by the routing
// scores.  Gating is a softmax; selection runs on the raw fp32 logits (the
// softmax is monotone, so the picks are the same and stay exact).
//
// Mapping: a group of G lanes (a power of two, G >= k) owns one token; lane g
// holds up to 16 logits of the row.  With E % 4 == 0 and 16-byte aligned
// logits, lane g loads 16-byte vectors: its key i holds expert
// ((i/4)*G + g)*4 + i%4, so each load instruction reads 4*G consecutive
// floats of a row and a lane issues 4 loads instead of 16 (measured on MI355X
// at T=4096, E=256, k=8: 10.1 -> 9.1 us warm, 14.4 -> 12.0 us cold); else
// key i holds expert i*G + g (nv = ceil(E/G) <= 16 keys).  A pick is one 64-bit key:
// the logit's bits made order-preserving as an unsigned integer (with -0.0
// read as +0.0, since the two compare equal) in the high half and ~e in the
// low half, so the largest key is the largest logit with the lowest expert
// id.  Each of the k rounds takes every lane's largest untaken key and a
// group-wide maximum through DPP row moves (quad permutes, half-row and row
// mirrors: VALU instructions, no LDS round trip), a 16-lane swizzle for G=32
// and a lane-0/lane-32 read for G=64.  A key is untaken when it lies below
// the previous round's pick (keys are unique); lane j keeps pick j.  The
// softmax sum uses the same pattern: every lane adds the same pairs of
// operands, so all lanes hold bit-identical sums.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kMaxNv = 16;

__device__ __forceinline__ uint32_t order_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0;                    // -0.0 ranks as +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_order_bits(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
    return (uint64_t(dpp32<CTRL>(uint32_t(v >> 32))) << 32) | dpp32<CTRL>(uint32_t(v));
}
__device__ __forceinline__ uint64_t swap16_64(uint64_t v) {     // lane ^ 16
    const uint32_t lo = uint32_t(__builtin_amdgcn_ds_swizzle(int(uint32_t(v)), 0x401F));
    const uint32_t hi = uint32_t(__builtin_amdgcn_ds_swizzle(int(uint32_t(v >> 32)), 0x401F));
    return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
    const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), l));
    const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), l));
    return (uint64_t(hi) << 32) | lo;
}

constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;

template <int G>
__device__ __forceinline__ uint64_t group_max(uint64_t k) {
    if constexpr (G >= 2) { const uint64_t o = dpp64<kQuadXor1>(k); k = o > k ? o : k; }
    if constexpr (G >= 4) { const uint64_t o = dpp64<kQuadXor2>(k); k = o > k ? o : k; }
    if constexpr (G >= 8) { const uint64_t o = dpp64<kHalfMirror>(k); k = o > k ? o : k; }
    if constexpr (G >= 16) { const uint64_t o = dpp64<kMirror>(k); k = o > k ? o : k; }
    if constexpr (G >= 32) { const uint64_t o = swap16_64(k); k = o > k ? o : k; }
    if constexpr (G >= 64) {
        const uint64_t a = readlane64(k, 0), b = readlane64(k, 32);
        k = a > b ? a : b;
    }
    return k;
}

template <int G>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (G >= 2) x += __uint_as_float(dpp32<kQuadXor1>(__float_as_uint(x)));
    if constexpr (G >= 4) x += __uint_as_float(dpp32<kQuadXor2>(__float_as_uint(x)));
    if constexpr (G >= 8) x += __uint_as_float(dpp32<kHalfMirror>(__float_as_uint(x)));
    if constexpr (G >= 16) x += __uint_as_float(dpp32<kMirror>(__float_as_uint(x)));
    if constexpr (G >= 32)
        x += __uint_as_float(uint32_t(__builtin_amdgcn_ds_swizzle(int(__float_as_uint(x)), 0x401F)));
    if constexpr (G >= 64) {
        const float a = __uint_as_float(uint32_t(__builtin_amdgcn_readlane(int(__float_as_uint(x)), 0)));
        const float b = __uint_as_float(uint32_t(__builtin_amdgcn_readlane(int(__float_as_uint(x)), 32)));
        x = a + b;
    }
    return x;
}

// The expert that lane g's key i holds.
template <int G, bool VEC>
__device__ __forceinline__ int slot_expert(int i, int g) {
    return VEC ? ((i >> 2) * G + g) * 4 + (i & 3) : i * G + g;
}

template <int G, bool VEC>
__global__ __launch_bounds__(kBlock) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int normalize,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w)
{
    const int g = threadIdx.x % G;
    const int64_t tok = (int64_t(blockIdx.x) * kBlock + threadIdx.x) / G;
    // Out-of-range groups keep running (on row 0, with every key dropped) so
    // that every DPP move reads an active lane; they just store nothing.
    const bool live = tok < T;
    const float* row = logits + (live ? tok : 0) * E;
    const int nv = (E + G - 1) / G;

    // Every load is unconditional, from a clamped in-bounds address (a key
    // past E reads element 0 of the row and is then dropped): a guarded load
    // becomes a branch with a full wait for memory inside it, so the loads
    // would go out one round trip at a time instead of all together.
    float v[kMaxNv];
    uint64_t key[kMaxNv];
    if constexpr (VEC) {                 // E % 4 == 0: a vector is all inside or all past E
        float4 f[kMaxNv / 4];
#pragma unroll
        for (int i = 0; i < kMaxNv; i += 4) {
            const int e0 = slot_expert<G, true>(i, g);
            f[i / 4] = *reinterpret_cast<const float4*>(row + (e0 < E ? e0 : 0));
        }
#pragma unroll
        for (int i = 0; i < kMaxNv; i += 4) {
            const int e0 = slot_expert<G, true>(i, g);
            const bool ok = live && e0 < E;
            v[i] = f[i / 4].x;
            v[i + 1] = f[i / 4].y;
            v[i + 2] = f[i / 4].z;
            v[i + 3] = f[i / 4].w;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                key[i + c] = ok ? (uint64_t(order_bits(v[i + c])) << 32) |
                                      uint32_t(~uint32_t(e0 + c))
                                : 0;
        }
    } else {
#pragma unroll
        for (int i = 0; i < kMaxNv; ++i) {
            const int e = slot_expert<G, false>(i, g);
            v[i] = row[i < nv && e < E ? e : 0];
        }
#pragma unroll
        for (int i = 0; i < kMaxNv; ++i) {
            const int e = slot_expert<G, false>(i, g);
            const bool ok = live && i < nv && e < E;
            key[i] = ok ? (uint64_t(order_bits(v[i])) << 32) | uint32_t(~uint32_t(e)) : 0;
        }
    }

    // Keys are unique (each carries its expert id), so round j's pick is the
    // largest key below round j-1's pick: no key is modified between rounds.
    uint64_t my_key = 0, top_key = 0, prev = ~uint64_t(0);
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < kMaxNv; ++i) best = key[i] < prev && key[i] > best ? key[i] : best;
        best = group_max<G>(best);
        prev = best;
        if (j == 0) top_key = best;
        if (g == j) my_key = best;
    }

    // The first pick holds the largest logit m: exp(l - m) keeps every
    // softmax ratio and cannot overflow.
    const float m = from_order_bits(uint32_t(top_key >> 32));
    const float my_val = from_order_bits(uint32_t(my_key >> 32));
    const int my_pick = int(~uint32_t(my_key));
    const float ex = g < k ? expf(my_val - m) : 0.0f;
    float denom;
    if (normalize) {
        denom = group_sum<G>(ex);
    } else {
        float z = 0.0f;
#pragma unroll
        for (int i = 0; i < kMaxNv; ++i)
            if ((VEC || i < nv) && slot_expert<G, VEC>(i, g) < E) z += expf(v[i] - m);
        denom = group_sum<G>(z);
    }
    if (live && g < k) {
        topk_idx[tok * k + g] = my_pick;
        topk_w[tok * k + g] = ex / denom;
    }
}

template <int G>
hipError_t launch_g(const float* logits, int T, int E, int k, int normalize,
                    int32_t* idx, float* w, hipStream_t s)
{
    const int64_t threads = int64_t(T) * G;
    const int grid = int((threads + kBlock - 1) / kBlock);
    if (E % 4 == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0)
        EP_LAUNCH((route_topk_kernel<G, true>), dim3(grid), dim3(kBlock), 0, s,
                  logits, T, E, k, normalize, idx, w);
    else
        EP_LAUNCH((route_topk_kernel<G, false>), dim3(grid), dim3(kBlock), 0, s,
                  logits, T, E, k, normalize, idx, w);
    return hipGetLastError();
}

int pow2_at_least(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int normalize,
                             int32_t* idx, float* w, hipStream_t s)
{
    // smallest group that holds the k picks and at most kMaxNv logits per lane
    int G = pow2_at_least(k);
    const int need = pow2_at_least((E + kMaxNv - 1) / kMaxNv);
    if (need > G) G = need;
    switch (G) {
        case 1: return launch_g<1>(logits, T, E, k, normalize, idx, w, s);
        case 2: return launch_g<2>(logits, T, E, k, normalize, idx, w, s);
        case 4: return launch_g<4>(logits, T, E, k, normalize, idx, w, s);
        case 8: return launch_g<8>(logits, T, E, k, normalize, idx, w, s);
        case 16: return launch_g<16>(logits, T, E, k, normalize, idx, w, s);
        case 32: return launch_g<32>(logits, T, E, k, normalize, idx, w, s);
        default: return launch_g<64>(logits, T, E, k, normalize, idx, w, s);
    }
}

}  // namespace ep
