// Host emulation of the HIP device subset used by the ep kernels: each
// workgroup runs on one OS thread as kBlock lane fibers (ucontext); wave ops
// rendezvous the 64 fibers of a wave; __syncthreads rendezvouses all fibers.
#pragma once
#include <ucontext.h>
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <cmath>
#include <thread>
#include <vector>
#include <functional>
#include <stdexcept>

#define __global__
#define __device__
#define __align__(n) __attribute__((aligned(n)))
#define __host__
#define __forceinline__ inline
#define __noinline__ __attribute__((noinline))
#define __launch_bounds__(x)
#define __shared__ static thread_local
#define __restrict__ __restrict

typedef int hipError_t;
typedef void* hipStream_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1, hipErrorInvalidDevice = 101,
       hipErrorInvalidSymbol = 13, hipErrorNotSupported = 801 };
struct alignas(16) int4 { int x, y, z, w; };
inline int4 make_int4(int a, int b, int c, int d) { return int4{a, b, c, d}; }
struct alignas(16) float4 { float x, y, z, w; };
inline float4 make_float4(float a, float b, float c, float d) { return float4{a, b, c, d}; }
struct dim3 { unsigned x, y, z; dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {} };

namespace emu {
struct Lane;
struct Group;
struct U3 { unsigned x, y, z; };
extern thread_local Group* g_group;
extern thread_local int g_lane_tid;   // threadIdx.x of the running fiber
extern thread_local U3 g_block;
extern U3 g_grid;
extern long g_op_limit;

enum OpKind { OP_NONE, OP_BALLOT, OP_SHFL, OP_READLANE, OP_READFIRST, OP_SYNC, OP_EXIT, OP_WAITCNT };

// One store that a lane has issued and that has not completed yet (weak
// memory mode): up to 16 bytes at `addr`; `coherent` for stores with the
// agent-coherence bit (sc1) and atomic stores, which write through to memory.
struct Pending {
    uintptr_t addr;
    uint8_t bytes[16];
    int n;
    bool coherent;
};

struct Group {
    int nthreads;
    std::vector<std::vector<Pending>> pending;   // per lane, in issue order
    std::vector<ucontext_t> ctx;
    std::vector<std::vector<char>> stacks;
    ucontext_t sched;
    std::vector<int> op;          // pending op per fiber
    std::vector<uint64_t> val;    // operand per fiber
    std::vector<int> arg;         // src lane / width etc.
    std::vector<uint64_t> res;
    std::vector<long> seq;        // count of wave ops per fiber (to detect mismatch)
    std::function<void()> body;
    long steps = 0;
};

void yield_op(int kind, uint64_t v, int a);
uint64_t result();

// ---- weak memory mode (off unless emu_set_weak() turned it on) ----
// Each simulated XCD (workgroup b runs on XCD b % 8) has a private
// write-back cache; plain stores complete into it and reach memory only when
// an agent-scope release writes the cache back, or at the end of the kernel.
// Coherent (sc1) stores and atomic stores write through to memory; coherent
// and atomic loads read memory; plain loads may return a stale cached copy
// until an agent-scope acquire invalidates the cache.  Every store first sits
// in its lane's queue and completes out of order: at random while the lane
// runs, at s_waitcnt vmcnt(0) or a release, before a load of the same lane
// to the same bytes (one wave's accesses to one address stay in order), or
// -- so that a parked lane's stores still complete, as they do on the
// hardware -- in the background.
bool weak_active();
void mem_store(void* p, const void* src, int n, bool coherent);
void mem_load(void* dst, const void* p, int n, bool coherent);
void waitcnt(int bits);
void fence(int order, const char* scope);
void complete_all();
}  // namespace emu

struct EmuIdx { unsigned operator()() const; };
#define threadIdx (emu::U3{(unsigned)emu::g_lane_tid, 0u, 0u})
#define blockIdx (emu::g_block)
#define gridDim (emu::g_grid)

inline int __lane_id() { return emu::g_lane_tid % 64; }
inline uint64_t __ballot(int p) { emu::yield_op(emu::OP_BALLOT, p ? 1 : 0, 0); return emu::result(); }
template <class T> inline T emu_shfl_idx(T v, int src, int width) {
    static_assert(sizeof(T) <= 8, "");
    uint64_t bits = 0; std::memcpy(&bits, &v, sizeof(T));
    int self = __lane_id();
    int base = self & ~(width - 1);
    int s = base + (src & (width - 1));
    emu::yield_op(emu::OP_SHFL, bits, s);
    uint64_t r = emu::result(); T out; std::memcpy(&out, &r, sizeof(T)); return out;
}
template <class T> inline T __shfl(T v, int src, int width = 64) { return emu_shfl_idx(v, src, width); }
template <class T> inline T __shfl_xor(T v, int m, int width = 64) {
    int self = __lane_id(); int idx = self ^ m;
    if (idx >= ((self + width) & ~(width - 1))) idx = self;
    uint64_t bits = 0; std::memcpy(&bits, &v, sizeof(T));
    emu::yield_op(emu::OP_SHFL, bits, idx);
    uint64_t r = emu::result(); T out; std::memcpy(&out, &r, sizeof(T)); return out;
}
template <class T> inline T __shfl_up(T v, unsigned d, int width = 64) {
    int self = __lane_id(); int idx = self - (int)d;
    if (idx < (self & ~(width - 1))) idx = self;
    uint64_t bits = 0; std::memcpy(&bits, &v, sizeof(T));
    emu::yield_op(emu::OP_SHFL, bits, idx);
    uint64_t r = emu::result(); T out; std::memcpy(&out, &r, sizeof(T)); return out;
}
template <class T> inline T emu_readlane(T v, int l) { return emu_shfl_idx(v, l, 64); }
template <class T> inline T emu_readfirst(T v) { return emu_shfl_idx(v, 0, 64); }
#define __builtin_amdgcn_readlane(v, l) emu_readlane((v), (l))
// DPP row moves and the ds_swizzle patterns the kernels use, as shuffles.
inline int emu_dpp_src(int lane, int ctrl) {
    if (ctrl <= 0xFF) return (lane & ~3) | ((ctrl >> (2 * (lane & 3))) & 3);   // quad_perm
    if (ctrl == 0x140) return (lane & ~15) | (15 - (lane & 15));               // row_mirror
    if (ctrl == 0x141) return (lane & ~7) | (7 - (lane & 7));                  // row_half_mirror
    std::fprintf(stderr, "[emu] unsupported DPP control %#x\n", ctrl);
    std::abort();
}
inline int emu_update_dpp(int old, int src, int ctrl, int, int, bool) {
    (void)old;
    return emu_shfl_idx(src, emu_dpp_src(__lane_id(), ctrl), 64);
}
inline int emu_ds_swizzle(int v, int pattern) {
    if (pattern & 0x8000) { std::fprintf(stderr, "[emu] unsupported swizzle %#x\n", pattern); std::abort(); }
    const int and_m = pattern & 0x1F, or_m = (pattern >> 5) & 0x1F, xor_m = (pattern >> 10) & 0x1F;
    const int lane = __lane_id();
    const int src = (lane & ~31) | ((((lane & 31) & and_m) | or_m) ^ xor_m);
    return emu_shfl_idx(v, src, 64);
}
#define __builtin_amdgcn_update_dpp(o, s, c, r, b, bc) emu_update_dpp((o), (s), (c), (r), (b), (bc))
#define __builtin_amdgcn_ds_swizzle(v, p) emu_ds_swizzle((v), (p))
inline unsigned __float_as_uint(float f) { unsigned u; std::memcpy(&u, &f, 4); return u; }
#define __builtin_amdgcn_readfirstlane(v) emu_readfirst((v))
inline void __syncthreads() { emu::yield_op(emu::OP_SYNC, 0, 0); }
#define __builtin_amdgcn_s_sleep(n) emu::yield_op(emu::OP_NONE, 0, 0)
#define __builtin_amdgcn_fence(order, scope) emu::fence((order), (scope))
inline int __popcll(unsigned long long x) { return __builtin_popcountll(x); }
inline int __ffsll(unsigned long long x) { return __builtin_ffsll((long long)x); }
inline int __clz(int x) { return x == 0 ? 32 : __builtin_clz((unsigned)x); }
inline int __clzll(long long x) { return x == 0 ? 64 : __builtin_clzll((unsigned long long)x); }
// The GPU's constant-rate wall clock: here the host's steady clock in 10 ns ticks.
#include <chrono>
inline long long wall_clock64() {
    return std::chrono::duration_cast<std::chrono::nanoseconds>(
               std::chrono::steady_clock::now().time_since_epoch()).count() / 10;
}
inline float __uint_as_float(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
#define __HIP_MEMORY_SCOPE_AGENT 3
inline bool emu_order_releases(int o) {
    return o == __ATOMIC_RELEASE || o == __ATOMIC_ACQ_REL || o == __ATOMIC_SEQ_CST;
}
inline bool emu_order_acquires(int o) {
    return o == __ATOMIC_ACQUIRE || o == __ATOMIC_ACQ_REL || o == __ATOMIC_SEQ_CST;
}
template <class T> inline T emu_atomic_load(const T* p, int o) {
    emu::yield_op(emu::OP_NONE, 0, 0);   // let other fibers / threads progress
    if (!emu::weak_active()) return __atomic_load_n(p, __ATOMIC_SEQ_CST);
    T v;
    emu::mem_load(&v, p, int(sizeof(T)), true);
    if (emu_order_acquires(o)) emu::fence(__ATOMIC_ACQUIRE, "agent");
    return v;
}
template <class T, class U> inline void emu_atomic_store(T* p, U v, int o) {
    if (!emu::weak_active()) { __atomic_store_n(p, (T)v, __ATOMIC_SEQ_CST); return; }
    if (emu_order_releases(o)) emu::fence(__ATOMIC_RELEASE, "agent");
    const T t = (T)v;
    emu::mem_store(p, &t, int(sizeof(T)), true);
}
template <class T, class U> inline T emu_atomic_fetch_add(T* p, U v, int o) {
    if (!emu::weak_active()) return __atomic_fetch_add(p, (T)v, __ATOMIC_SEQ_CST);
    // performed at memory; the lane's own earlier stores stay queued unless
    // the order asks for a release
    if (emu_order_releases(o)) emu::fence(__ATOMIC_RELEASE, "agent");
    const T r = __atomic_fetch_add(p, (T)v, __ATOMIC_SEQ_CST);
    if (emu_order_acquires(o)) emu::fence(__ATOMIC_ACQUIRE, "agent");
    return r;
}
#define __hip_atomic_load(p, o, s) emu_atomic_load((p), (o))
#define __hip_atomic_store(p, v, o, s) emu_atomic_store((p), (v), (o))
#define __hip_atomic_fetch_add(p, v, o, s) emu_atomic_fetch_add((p), (v), (o))
template <class T, class U> inline T atomicAdd(T* p, U v) { return __atomic_fetch_add(p, (T)v, __ATOMIC_SEQ_CST); }

// Buffer descriptors and buffer stores: the emulation keeps base and size
// and aborts on an access outside the range (the hardware would drop it).
struct emu_buffer_rsrc { char* base; uint32_t n; };
#define __amdgpu_buffer_rsrc_t emu_buffer_rsrc
inline emu_buffer_rsrc emu_make_buffer_rsrc(void* p, int, int n, unsigned) {
    return emu_buffer_rsrc{static_cast<char*>(p), uint32_t(n)};
}
// The cache-policy bit of a buffer access that makes it agent-coherent (sc1).
constexpr int kEmuCpolSc1 = 16;
// Negative control: stores with the sc1 bit behave as plain stores.
#ifdef EMU_MUTATE_SC1_STORES_PLAIN
constexpr bool kEmuSc1StoresCoherent = false;
#else
constexpr bool kEmuSc1StoresCoherent = true;
#endif
template <class V> inline void emu_buffer_store(V v, emu_buffer_rsrc r, int off, int aux) {
    if (off < 0 || uint64_t(uint32_t(off)) + sizeof(V) > r.n) {
        std::fprintf(stderr, "[emu] buffer store at %d outside a %u-byte range\n", off, r.n);
        std::abort();
    }
    if (emu::weak_active())
        emu::mem_store(r.base + off, &v, int(sizeof(V)), kEmuSc1StoresCoherent && (aux & kEmuCpolSc1));
    else
        std::memcpy(r.base + off, &v, sizeof(V));
}
struct emu_v4u32 { uint32_t v[4]; };
inline emu_v4u32 emu_buffer_load_b128(emu_buffer_rsrc r, int off, int aux) {
    if (off < 0 || uint64_t(uint32_t(off)) + 16 > r.n) {
        std::fprintf(stderr, "[emu] buffer load at %d outside a %u-byte range\n", off, r.n);
        std::abort();
    }
    emu_v4u32 v;
    if (emu::weak_active())
        emu::mem_load(&v, r.base + off, 16, (aux & kEmuCpolSc1) != 0);
    else
        std::memcpy(&v, r.base + off, 16);
    return v;
}
#define __builtin_amdgcn_make_buffer_rsrc(p, s, n, f) emu_make_buffer_rsrc((void*)(p), (s), (n), (f))
#define __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, aux) emu_buffer_load_b128((r), (off), (aux))
#define __builtin_amdgcn_raw_buffer_store_b128(v, r, off, soff, aux) emu_buffer_store((v), (r), (off), (aux))
#define __builtin_amdgcn_s_waitcnt(x) emu::waitcnt((x))
// Nontemporal accesses are plain (cached) accesses with a hint.
template <class V> inline void emu_nt_store(V v, V* p) {
    if (emu::weak_active()) emu::mem_store(p, &v, int(sizeof(V)), false);
    else std::memcpy(p, &v, sizeof(V));
}
template <class V> inline V emu_nt_load(const V* p) {
    V v;
    if (emu::weak_active()) emu::mem_load(&v, p, int(sizeof(V)), false);
    else std::memcpy(&v, p, sizeof(V));
    return v;
}
#define __builtin_nontemporal_store(v, p) emu_nt_store((v), (p))
#define __builtin_nontemporal_load(p) emu_nt_load((p))

inline hipError_t hipGetLastError() { return hipSuccess; }
inline hipError_t hipGetDevice(int* d) { *d = 0; return 0; }
// A __device__ variable is an ordinary host object here, so its address is
// the symbol's address.
#define HIP_SYMBOL(x) (&(x))
inline hipError_t hipGetSymbolAddress(void** p, const void* sym) {
    *p = const_cast<void*>(sym);
    return 0;
}
inline hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int* n, const void*, int, int) { *n = 2; return 0; }
enum { hipDeviceAttributeMultiprocessorCount = 1 };
inline hipError_t hipDeviceGetAttribute(int* v, int, int) { *v = 4; return 0; }

namespace emu {
void launch(dim3 grid, dim3 block, std::function<void()> body);
}
#define hipLaunchKernelGGL(K, G, B, SH, S, ...) emu::launch(dim3(G), dim3(B), [=]() { K(__VA_ARGS__); })

enum hipMemcpyKind { hipMemcpyHostToDevice = 1, hipMemcpyDeviceToHost = 2, hipMemcpyDeviceToDevice = 3 };
inline hipError_t hipStreamSynchronize(hipStream_t) { return 0; }
inline hipError_t hipMemcpy(void* d, const void* s, size_t n, hipMemcpyKind) { std::memcpy(d, s, n); return 0; }
inline const char* hipGetErrorString(hipError_t) { return "emu"; }
