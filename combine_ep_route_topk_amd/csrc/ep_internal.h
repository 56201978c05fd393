// ep_internal.h -- workspace layouts, tuning constants and kernel launchers
// shared by the host API (api.hip) and the kernel files of libep_route_topk.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ep_route_topk.h"

namespace ep {

// One-shot measurement hook (ep_set_timing_events): when set, the next
// entry point's first kernel launch records `start` from its own dispatch
// packet and every launch records `stop`, so the pair brackets exactly the
// entry point's kernels.  Thread-local; api.hip clears it after each call.
struct LaunchTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
LaunchTiming& launch_timing();

#define EP_LAUNCH(K, G, B, SHM, S, ...)                                                \
    do {                                                                               \
        ::ep::LaunchTiming& ep_t_ = ::ep::launch_timing();                             \
        if (ep_t_.start || ep_t_.stop) {                                               \
            hipExtLaunchKernelGGL(K, G, B, SHM, S, ep_t_.start, ep_t_.stop, 0,         \
                                  __VA_ARGS__);                                        \
            ep_t_.start = nullptr;                                                     \
        } else {                                                                       \
            hipLaunchKernelGGL(K, G, B, SHM, S, __VA_ARGS__);                          \
        }                                                                              \
    } while (0)

// ----------------------------------------------------------------- tuning
constexpr int kBlock = 256;          // threads per workgroup (4 waves of 64)
constexpr int kTileSlots = 1024;     // slots per layout tile (histogram unit)
constexpr int kScanItems = 2048;     // (expert, tile) counters per scan block
// Up to this many (expert, tile) counters the layout computes every tile's
// bases inside the positions launch (each workgroup re-reads all counters)
// instead of a separate device-wide scan.
constexpr int kRedundantScanMax = 32768;
// Counters per scan item of the persistent fused mode: one item covers the
// 8192 counters of a T=4096, k=8, E=256 layout, so its look-back chain is empty.
constexpr int kFusedScanItems = 8192;
// Most parts a small batch's rows are split into in the fused mode's
// item-event readiness (so that its few tokens still spread over the GPU).
#ifndef EP_FUSED_MAX_PARTS
#define EP_FUSED_MAX_PARTS 4
#endif
constexpr int kFusedMaxParts = EP_FUSED_MAX_PARTS;
constexpr int kMaxE = 1024;
constexpr int kMaxK = 64;
// Cap on the 1-D grid of the row kernels, which stride over their items.
constexpr uint32_t kMaxGrid = uint32_t(1) << 20;

// Error codes stored in a workspace's error word (host maps them to ep_status).
enum : uint32_t { kDevOk = 0, kDevBadExpert = 1, kDevTimeout = 2, kDevSentinel = 3,
                  kDevOverflow = 4 };

// Magic words marking initialised workspaces.
constexpr uint32_t kLayoutMagic = 0x45504C57u;   // "EPLW"
constexpr uint32_t kFusedMagic = 0x45504657u;    // "EPFW"

// One 32-bit word alone in a 128-byte line.  The counters that many
// workgroups poll or update at once each get their own line: a line that
// every waiting wave re-reads serialises all requests to it, and an atomic on
// a word sharing that line queues behind them.
struct alignas(128) LineWord {
    uint32_t v;
    uint32_t pad[31];
};

// Common 1 KiB header at the start of every workspace.
struct WsHeader {
    // line 0: written once per call, read by the host
    uint32_t magic;
    uint32_t error;         // result of the last call (kDev*)
    uint64_t epoch;         // fused mode: epoch of the NEXT call
    uint64_t last_epoch;    // fused mode: epoch of the last call
    uint32_t pad0[26];
    LineWord scan_ticket;   // decoupled-lookback block ticket
    LineWord timeout;       // set by any expired bounded wait
    LineWord work_ticket;   // fused mode: next work item to claim
    LineWord hist_done;     // fused mode: histogram tiles finished
    LineWord collision;    // fused sentinel mode: a payload held the reserved pattern
    LineWord reserved[2];
};
static_assert(sizeof(WsHeader) == 1024, "header is eight 128-byte lines");
static_assert(offsetof(WsHeader, error) == 4, "the host reads magic and error as two words");

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Layout of the dispatch-layout workspace (also the first part of the fused
// workspace).  All offsets are from the workspace base, 256-byte aligned.
struct LayoutPlan {
    int64_t S;          // slots = T*k
    int nTiles;         // histogram tiles
    int nCnt;           // E * nTiles (expert-major counters)
    int nScan;          // scan blocks
    size_t off_status;  // u32 [nScan]      lookback status words
    size_t off_cnt;     // i32 [nCnt]       per-(expert, tile) counts
    size_t off_base;    // i32 [nCnt]       per-(expert, tile) first row
    size_t off_rank;    // i32 [S]          rank of a slot inside its (tile, expert)
    size_t bytes;
};

inline LayoutPlan layout_plan(int T, int k, int E) {
    LayoutPlan p{};
    p.S = int64_t(T) * k;
    p.nTiles = int((p.S + kTileSlots - 1) / kTileSlots);
    p.nCnt = E * p.nTiles;
    p.nScan = (p.nCnt + kScanItems - 1) / kScanItems;
    size_t off = sizeof(WsHeader);
    p.off_status = off; off += align256(sizeof(uint32_t) * p.nScan);
    p.off_cnt = off;    off += align256(sizeof(int32_t) * p.nCnt);
    p.off_base = off;   off += align256(sizeof(int32_t) * p.nCnt);
    p.off_rank = off;   off += align256(sizeof(int32_t) * p.S);
    p.bytes = off;
    return p;
}

// Fused workspace: the layout part (its cnt and rank arrays are used), then
// 64-bit epoch-tagged look-back status words and Data-as-Flag base words.
struct FusedPlan {
    LayoutPlan lay;
    size_t off_status64;  // u64 [nScan]  (epoch32 << 32 | flag << 30 | value)
    size_t off_fbase;     // u64 [nCnt]   (epoch32 << 32 | base) published bases
    size_t off_sdone;     // u64 [ceil(T/2) * kFusedMaxParts] epoch of the call once a
                          //     scatter item (or one part of it) is done
    size_t bytes;
};

inline FusedPlan fused_plan(int T, int k, int E) {
    FusedPlan f{};
    f.lay = layout_plan(T, k, E);
    size_t off = f.lay.bytes;
    f.off_status64 = off; off += align256(sizeof(uint64_t) * f.lay.nScan);
    f.off_fbase = off;    off += align256(sizeof(uint64_t) * f.lay.nCnt);
    f.off_sdone = off;
    off += align256(sizeof(uint64_t) * ((size_t(T) + 1) / 2) * kFusedMaxParts);
    f.bytes = off;
    return f;
}

// Rank-coalescing workspace: the layout's (over R "experts"), then each
// pick's key, then the layout's per-rank outputs (which duplicate its
// per-expert ones when every rank holds one expert).
struct CoalescePlan {
    LayoutPlan lay;
    size_t off_keys;          // i32 [T*k]
    size_t off_rank_counts;   // i32 [R]
    size_t off_rank_offsets;  // i32 [R+1]
    size_t bytes;
};

// The receiver's expansion uses the same shape of workspace: the layout's
// over (C records, L bits, L experts), the keys, and one rank's outputs.
inline CoalescePlan coalesce_plan(int T, int k, int R) {
    CoalescePlan c{};
    c.lay = layout_plan(T, k, R);
    size_t off = c.lay.bytes;
    c.off_keys = off;         off += align256(sizeof(int32_t) * c.lay.S);
    c.off_rank_counts = off;  off += align256(sizeof(int32_t) * size_t(R));
    c.off_rank_offsets = off; off += align256(sizeof(int32_t) * (size_t(R) + 1));
    c.bytes = off;
    return c;
}

// Default bound of a device-side wait, in polling rounds (each round is one
// agent-scope load plus a short sleep, roughly a microsecond).
constexpr uint32_t kDefaultSpinLimit = uint32_t(1) << 20;

// Bytes per 16-byte-vector chunk that carries its own readiness word in the
// fused mode's sub-row flag variant (one wave-wide row segment).
constexpr int kChunkBytes = 1024;
// A fused send row: payload (2H bytes), the 16-byte trailer, then one 8-byte
// flag per kChunkBytes chunk of the payload, padded to 1 KiB, so that a
// wave's 1 KiB store lands in one 1 KiB unit of memory (measured on MI355X at
// T=4096, H=7168, k=8, the fused call: 189.9-190.4 us padded to 128 bytes,
// 187.3-187.5 us to 1 KiB, 195.6 us to 4 KiB; at T=16384 with a skewed
// incast, 718.8-719.7 / 719.3-722.6 / 713.6-714.2 us).
inline size_t fused_row_stride(int H) {
    const size_t chunks = (size_t(2) * H + kChunkBytes - 1) / kChunkBytes;
    return (size_t(2) * H + 16 + 8 * chunks + 1023) / 1024 * 1024;
}

// ----------------------------------------------------------------- launchers
// The CU count of the current device (cached per device).
uint32_t device_cu_count();
// Grid cap of dispatch's row scatter: five eighths of the CU count of the
// current device.  With the cached tail of rows (keep_from) a larger grid
// costs little in back-to-back steps and hides more of x's read latency when
// x comes from HBM (measured on MI355X at T=4096, H=7168, k=8, A/B on two
// boxes, dispatch in the step / after a 1 GiB read: 128 workgroups
// 83.6-85.2 / 114.7-115.5 us, 160 85.4-86.2 / 101.7-102.2 us).
inline uint32_t dispatch_grid_cap() { return device_cu_count() * 5 / 8; }
// Grid cap of the backward combine's gradient scatter: thirteen sixteenths of
// the CU count (its per-element multiply and tie check need more waves than
// dispatch's plain copy).
inline uint32_t scatter_grid_cap() { return device_cu_count() * 13 / 16; }
// Scatters writing (gathers reading) at most this many bytes are
// latency-bound: they run one vector per lane on an uncapped grid instead.
// A build may set it lower (the host emulation's tests build with 0, so that
// every size takes the large-batch kernels).
#ifndef EP_SMALL_SCATTER_BYTES
#define EP_SMALL_SCATTER_BYTES (int64_t(64) << 20)
#endif
constexpr int64_t kSmallScatterBytes = EP_SMALL_SCATTER_BYTES;
bool small_scatter(int T, int H, int k);
// Cached rows.  Dispatch (and the fused scatter) stores the rows of its last
// tokens -- up to kKeepTailBytes of them -- without the streaming hint, so
// combine, which reads the rows in token order, finds that tail in the
// caches, and streams the rest; batches of more than kKeepMaxBytes of rows
// stream all.  Measured on MI355X, dispatch then combine, A/B on one box:
// T=4096, H=7168, k=8 (448 MiB of rows) 175.9-176.2 -> 168.7-168.8 us with a
// 128 MiB tail (96 MiB 169.1-169.7, 160 MiB 170.7-171.1; every row cached
// 210 us, since they overflow the 256 MB Infinity Cache and evict x);
// T=4096, H=4096 (256 MiB) 95.8-97.0 with every row cached -> 91.8-92.1 us
// with the tail; T=16384, H=7168 (1.75 GiB) 667.3-667.7 -> 742.4-743.5 us
// with the tail.
constexpr int64_t kKeepTailBytes = int64_t(128) << 20;
constexpr int64_t kKeepMaxBytes = int64_t(512) << 20;
// The first token whose rows a scatter of T tokens x k rows x H bf16 keeps
// cached (T: none).
int keep_from(int T, int H, int k);
// The backward's gradient scatter keeps all of its rows cached for
// dispatch_grad, or none: up to kKeepRowsBytes (measured at T=4096, H=4096,
// k=8, 256 MiB: combine_grad 100.4-102.1 -> 99.2-99.4 us, dispatch_grad
// 51.3-51.6 -> 49.7-50.1 us).  A cached tail chosen per token at run time
// made its scatter kernel slower at every size (T=4096, H=7168: combine_grad
// 173.0-173.2 -> 183.2-183.5 us, with no row cached at T=16384 as well).
constexpr int64_t kKeepRowsBytes = int64_t(256) << 20;
bool keep_rows(int T, int H, int k);

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int normalize,
                             int32_t* topk_idx, float* topk_w, hipStream_t s);

hipError_t launch_dispatch_layout(const int32_t* topk_idx, int T, int k, int E, int R,
                                  int32_t* expert_counts, int32_t* expert_offsets,
                                  int32_t* rank_counts, int32_t* rank_offsets,
                                  int32_t* pos, int32_t* slot_src, void* ws,
                                  hipStream_t s);
// The layout workspace that the library itself holds, one per GPU, for the
// entry point that allocates nothing: kLayoutScratchBytes bytes, 256-byte
// aligned, kept until the process ends.  *ptr receives the current device's
// copy (looked up once per device).
constexpr size_t kLayoutScratchBytes = size_t(16) << 20;
hipError_t layout_scratch(void** ptr);
// The layout with a chosen expected slot total: the device error word reports
// an id outside [0, E) only when expect >= 0 and fewer than `expect` slots
// were counted.  expect = -1 lets slots with a negative id be skipped on
// purpose (the rank-coalescing pass marks a token's repeated ranks so).
hipError_t launch_dispatch_layout_skips(const int32_t* topk_idx, int T, int k, int E, int R,
                                        int32_t* expert_counts, int32_t* expert_offsets,
                                        int32_t* rank_counts, int32_t* rank_offsets,
                                        int32_t* pos, int32_t* slot_src, void* ws,
                                        int64_t expect, hipStream_t s);

hipError_t launch_rank_coalesce(const int32_t* topk_idx, int T, int k, int E, int R,
                                int32_t* rank_counts, int32_t* rank_offsets,
                                int32_t* row_of_pick, int32_t* send_pos, int32_t* row_src,
                                uint64_t* row_experts, void* ws, hipStream_t s);
hipError_t launch_expand_records(const uint16_t* rows, const uint64_t* masks, int C, int H, int L,
                                 int32_t* expert_counts, int32_t* expert_offsets, int32_t* pos,
                                 uint16_t* recv, int64_t recv_rows, void* ws, hipStream_t s);
// Host: peer[(w-1)*N + s] = (s + w) mod N for w = 1..N-1.
void exchange_waves(int32_t N, int32_t* peer);

hipError_t launch_dispatch(const uint16_t* x, int T, int H, int k, const int32_t* pos,
                           uint16_t* send, hipStream_t s);
// Dispatch into a buffer of `bound` rows: positions at or past it are skipped.
hipError_t launch_dispatch_bounded(const uint16_t* x, int T, int H, int k, const int32_t* pos,
                                   uint16_t* send, uint32_t bound, hipStream_t s);

hipError_t launch_combine(const uint16_t* y, const int32_t* pos, const float* w,
                          int T, int H, int k, uint16_t* out, hipStream_t s);

// The batched combine on a grid of `grid` workgroups, whatever the batch
// size (w == nullptr: every weight 1).  Requires H % 512 == 0; returns
// hipErrorInvalidValue otherwise.  launch_combine picks it for large batches.
hipError_t launch_combine_batched(const uint16_t* y, const int32_t* pos, const float* w, int T,
                                  int H, int k, uint16_t* out, uint32_t grid, hipStream_t s);
hipError_t launch_combine_grad(const uint16_t* grad_out, const uint16_t* y,
                               const int32_t* pos, const float* w, int T, int H, int k,
                               uint16_t* grad_y, float* grad_w, hipStream_t s);

hipError_t launch_dispatch_grad(const uint16_t* grad_send, const int32_t* pos, int T, int H,
                                int k, uint16_t* grad_x, hipStream_t s);

hipError_t launch_fused_init(void* ws, uint64_t first_epoch, hipStream_t s);

// How a combine item of the fused mode learns that its rows are complete.
enum FusedSync : int {
    kSyncItemEvents = 0,   // event word per scatter item, then the rows' trailers
    kSyncRowFlag = 1,      // the rows' trailers only (Token-Flag Fusion per row)
    kSyncChecksum = 2,     // per scatter item a checksum of the rows' markers
    kSyncSentinel = 3,     // each row's leading 16 bytes leave a reserved pattern
    kSyncChunkFlag = 4,    // a flag per 1 KiB chunk of each row (sub-row TFF)
};
constexpr int kNumFusedSync = 5;
// The sentinel mode's reserved pattern: every 32-bit word of a row's leading
// 16 bytes holds two bf16 signalling NaNs 0x7FA5 until the row is written.
constexpr uint32_t kSentinelWord = 0x7FA57FA5u;

hipError_t launch_fused(const uint16_t* x, const int32_t* topk_idx, const float* topk_w,
                        int T, int H, int k, int E, int R, int32_t* expert_counts,
                        int32_t* expert_offsets, int32_t* rank_counts,
                        int32_t* rank_offsets, int32_t* pos, uint8_t* send_rows,
                        uint16_t* out, void* ws, uint32_t spin_limit, int grid, int sync,
                        hipStream_t s);

hipError_t launch_slices(const int32_t* eo, int E, int P, int64_t* start, int32_t* expert,
                         int64_t* offset, hipStream_t s);

hipError_t launch_window_copy(const void* src, void* dst, int64_t row_bytes, int64_t S,
                              const ep_task* tasks, const int64_t* core_begin,
                              const int64_t* slice_start, int C, uint64_t* core_clock,
                              uint32_t* bad, hipStream_t s);

int64_t lpt_unit_count(const int32_t* rank_offsets, int R, int64_t unit_rows);

int64_t lpt_partition(const int32_t* rank_offsets, int R, int64_t row_bytes, int64_t unit_rows,
                      const int32_t* tier_of_peer, const double* alpha, const double* beta,
                      const int32_t* cap, int C, ep_task* tasks, int64_t max_tasks,
                      int64_t* core_begin, double* core_load);

}  // namespace ep
