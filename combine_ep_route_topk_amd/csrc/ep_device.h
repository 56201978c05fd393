// ep_device.h -- device helpers shared by the gfx950 kernels of
// libep_route_topk: vector types, bf16 <-> f32, wave64 primitives and
// agent-scope (whole-GPU, all 8 XCDs) atomics.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;                 // CDNA wavefront width

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16
// A bf16 value widens to f32 exactly: its bits are the high half of the f32.
__device__ __forceinline__ float bf16_lo(uint32_t packed) {
    return __uint_as_float(packed << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t packed) {
    return __uint_as_float(packed & 0xFFFF0000u);
}
// Two f32 -> two bf16 (round to nearest even, NaN stays NaN) in one
// v_cvt_pk_bf16_f32; element 0 lands in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

// ---------------------------------------------------------------- 16-byte I/O
__device__ __forceinline__ u32x4 load16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store16(void* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}
// Streaming store: the line is not expected to be re-read soon by this CU.
__device__ __forceinline__ void store16_nt(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ u32x4 load16_nt(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ---------------------------------------------------------------- coherent stores
// A buffer descriptor over `bytes` bytes at `base` (raw, unstrided): buffer
// accesses through it are bounds-checked by the hardware against `bytes`.
constexpr uint32_t kRawBufferWord3 = 0x00020000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, int(bytes), kRawBufferWord3);
}
// 16-byte store with the agent-scope coherence bit (sc1) and the streaming
// hint (nt): it is written through this XCD's L2 instead of staying dirty
// there, so once it has completed it is visible to agent-scope loads on
// every XCD -- the same guarantee an agent-scope atomic store (also sc1)
// has.  `off` is a byte offset inside the descriptor's range.
constexpr int kCpolNtSc1 = 2 | 16;
__device__ __forceinline__ void store16_coherent(__amdgpu_buffer_rsrc_t r, int off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCpolNtSc1);
}
// The same store without the streaming hint: still written through at agent
// scope, but the line may stay in the caches for a reader that comes soon
// (a small batch whose rows the next kernel reads while they still fit).
constexpr int kCpolSc1 = 16;
__device__ __forceinline__ void store16_coherent_keep(__amdgpu_buffer_rsrc_t r, int off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCpolSc1);
}
// 16-byte load with the same bits: served at agent scope (it sees every
// store from any XCD that has completed) and not kept in this XCD's L2, so
// no L2 invalidate (acquire fence) is needed before it.  The descriptor's
// base must be wave-uniform.
__device__ __forceinline__ u32x4 load16_coherent(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolNtSc1));
}
// Wait until every store this wave issued has completed (s_waitcnt vmcnt(0)
// on gfx9-family ISAs, where stores count in vmcnt); the compiler may move
// no memory access across it.
__device__ __forceinline__ void wait_own_stores() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------- wave64
__device__ __forceinline__ int lane_id() { return __lane_id(); }
__device__ __forceinline__ uint64_t lanes_below() {
    return (uint64_t(1) << lane_id()) - 1;   // lane 0 -> 0
}
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// Inclusive prefix sum over the 64 lanes of a wave (Hillis-Steele, 6 steps).
__device__ __forceinline__ int wave_inclusive_sum(int v) {
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

// ---------------------------------------------------------------- atomics
// Agent scope = visible to every CU of this GPU (all XCDs); on gfx950 the
// compiler lowers these with the L2 write-back / invalidate the memory model
// requires.
__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_relaxed64(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed64(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t fetch_add(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t fetch_add_acq_rel(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_release() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}
__device__ __forceinline__ void fence_acquire() {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}
__device__ __forceinline__ void backoff() { __builtin_amdgcn_s_sleep(2); }

}  // namespace ep
