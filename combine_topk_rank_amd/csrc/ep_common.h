// ep_common.h — definitions shared by the HIP sources of the dispatch/combine
// library (device-side ring view, workspace carving, shape validation).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ep.h"
#include "ep_ring_proto.h"

namespace ep {

constexpr int kWave = 64;          // CDNA wavefront width (UCCL-EP article s5.1: 32 -> 64)
constexpr int kBlock = 256;        // threads per workgroup: 4 wavefronts
constexpr int kLayoutTile = 256;   // tokens per layout workgroup
constexpr int kMsgRows = 8;        // rows per WRITE message (UCCL-EP s4.1 packing, s5.3 batch 8)
constexpr int kMaxR = 64;          // a rank set is one 64-bit mask
constexpr int kMaxE = 4096;        // per-expert LDS histogram bound
constexpr int kMaxK = 32;          // experts of a token sit in lanes 0..k-1
constexpr int kMaxH = 1 << 24;     // rows stay far below 2^31 bytes (buffer records)
constexpr int kPad = 8;            // 64-byte stride between per-channel counters
// Bound on a grid-barrier wait, in s_memrealtime ticks (100 MHz): one second.
constexpr unsigned long long kBarrierTimeoutTicks = 100000000ull;

// Device view of a TransferCmd ring.
struct RingDev {
    RingSlot* slots;                       // host-pinned, [channels][depth]
    const unsigned long long* host_tail;   // host-pinned, consumer position, stride kPad
    unsigned long long* head;              // device, ticket counter, stride kPad
    unsigned long long* tail_cache;        // device, last consumer position seen, stride kPad
    unsigned long long* poll;              // device, 1 while a lane reads host_tail, stride kPad
    const unsigned long long* completed;   // host-pinned, commands completed, stride kPad
    int32_t depth;
    int32_t channels;
    int32_t max_inflight;
    int32_t pad_;
    unsigned long long timeout_ticks;      // in s_memrealtime ticks
};

// CheckCompletion (UCCL-EP article s2.2): whether the command with `ticket`
// on channel c has completed, from the consumer's per-channel count of
// completed commands (commands of a channel complete in ticket order).
// Never waits.
__device__ inline bool ring_check_completion(const RingDev& g, int c, unsigned long long ticket) {
    return __hip_atomic_load(g.completed + (size_t)c * kPad, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_SYSTEM) > ticket;
}

// Carved workspace.
// Workspace header: grid barrier words, one per 128-byte line (the top
// arrival count, kBarGroups group counts, the generation), then the
// dispatch's arrival counters, also one per line (a top counter and 8 group
// counters).
constexpr size_t kArriveStride = 32;   // words
constexpr int kBarGroups = 8;
constexpr int kBarFlatMax = 128;   // grids up to this size count arrivals in one level
constexpr size_t kBarGen = (1 + kBarGroups) * kArriveStride;   // word of the generation
constexpr size_t kBarrierBytes = 10 * kArriveStride * 4;
constexpr size_t kWsHeader = kBarrierBytes + 16 * kArriveStride * 4;
static_assert((kBarGen + 1) * 4 <= kBarrierBytes, "barrier words fit their section");
static_assert(kBarrierBytes % 256 == 0 && kWsHeader % 256 == 0,
              "workspace sections stay 256-byte aligned");

struct Workspace {
    uint32_t* barrier;        // grid barrier words (zero at first use)
    uint32_t* arrive;         // [9 lines] dispatch arrival counters (zero between calls)
    int32_t* blk_rank_cnt;    // [NB, R] per-layout-block rank counts
    int32_t* blk_exp_cnt;     // [NB, E] per-layout-block expert counts
    int32_t* wave_rank_cnt;   // [ceil(T/64), R] per-64-token rank counts (one-kernel dispatch)
    int32_t* msg_base;        // [R+1]   first message index of each rank
    int32_t* msg_arrivals;    // [max_msgs] rows (x chunks) written per message
    int32_t* msgs_done;       // [E]     messages of a rank (or, per-expert mode, an expert) published
    int64_t max_msgs;
    int64_t counters_n;       // msg_arrivals .. msgs_done, contiguous
    int32_t layout_blocks;
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int32_t layout_blocks(int32_t T) {
    return (int32_t)(T <= 0 ? 1 : ceil_div(T, kLayoutTile));
}

inline int64_t wave_blocks(int32_t T) { return T <= 0 ? 1 : ceil_div(T, kWave); }

// Messages of one call, at most: per rank, ceil(rows / 8) with at most
// min(k, R) rows a token; per expert (per-expert mode), ceil(rows / 8) with k
// rows a token.  Both are below ceil(T * k / 8) + E.
inline int64_t max_messages(const ep_shape_t& s) {
    return ceil_div((int64_t)s.T * s.k, kMsgRows) + s.E;
}

size_t workspace_bytes(const ep_shape_t& s);
Workspace carve_workspace(const ep_shape_t& s, void* base);
int validate_shape(const ep_shape_t* s);
size_t row_bytes(int32_t H, int32_t fmt);

// Remember the last failing HIP call of this thread (ep_last_error).
void record_hip_error(hipError_t e, const char* what);
// Remember why a call was rejected on the host (ep_last_error).
void record_error(const char* what);

#define EP_HIP_CHECK(expr)                                  \
    do {                                                    \
        hipError_t e_ = (expr);                             \
        if (e_ != hipSuccess) {                             \
            ::ep::record_hip_error(e_, #expr);              \
            return EP_ERR_HIP;                              \
        }                                                   \
    } while (0)

// Launch errors surface through hipGetLastError, which also returns errors
// left by unrelated earlier calls of the thread: clear it before a launch.
inline void clear_hip_error() { (void)hipGetLastError(); }

// First error wins.
__device__ inline void set_error(int32_t* st, int code) {
    atomicCAS(st, 0, code);
}

__device__ inline int32_t read_status(const int32_t* st) {
    return __hip_atomic_load(st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Broadcast lane `l` (wave-uniform) of a 32-bit value.
__device__ inline int32_t bcast(int32_t v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ inline float bcastf(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Raw buffer resource over `bytes` bytes at p (the untyped-access word 3 of
// CDNA3/CDNA4 buffer descriptors).  Buffer instructions drop accesses whose
// offset falls outside [0, bytes).
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(void* p, int32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(p, 0, bytes, 0x00020000);
}
// Cache-policy bits of gfx94x/gfx950 buffer instructions.  A store with
// sc0 sc1 has system scope: it is written through the L2 to memory and is
// complete (vmcnt) only once it is coherent for every agent, so a completed
// system-scope store needs no L2 write-back before another agent (a CPU, a
// NIC reading over PCIe) may be told about it.  nt marks it streaming.
constexpr int kCacheSc0 = 1, kCacheNt = 2, kCacheSc1 = 16;
constexpr int kStoreSystem = kCacheSc0 | kCacheSc1;

// Wait until this wavefront's outstanding vector memory operations, stores
// included, have completed (s_waitcnt vmcnt(0); gfx9 encoding with expcnt
// and lgkmcnt left at their maxima).  A workgroup barrier does not wait for
// stores, so a release fence executed by one wavefront after the barrier
// covers another wavefront's stores only if that wavefront waited first.
__device__ inline void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Grid-wide barrier for a grid whose workgroups are all resident.  Grids of
// more than kBarFlatMax workgroups count arrivals in two levels so that no
// single word takes every atomic: workgroup b counts into group counter
// b % kBarGroups, the last of a group into the top counter.  Smaller grids
// count straight into the top counter, which saves the group level's atomic
// round trip and cache maintenance on the path of the last arrival (about
// 0.6-0.9 us of a 17-65 workgroup layout).  The last of all bumps the
// generation, which releases the others.  Each workgroup reads the generation before it
// arrives (thread 0 passes what it loaded with grid_barrier_generation, as
// early as it likes: the generation cannot move before this workgroup
// arrives).  Every counter is reset by the arrival that completes it, so the
// words stay consistent from one call to the next for any grid size (they
// start at zero).  The wait is bounded by about a second of wall clock; on
// timeout the status is set and false is returned.  Stores made before the
// barrier by any workgroup are visible to loads made after it by every
// workgroup; with SYSTEM they are also released at system scope (visible to
// other agents, e.g. a CPU or NIC).
__device__ inline uint32_t grid_barrier_generation(const uint32_t* bar) {
    return __hip_atomic_load(&bar[kBarGen], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool SYSTEM>
__device__ bool grid_barrier(uint32_t* bar, uint32_t nblocks, int32_t* st, uint32_t gen) {
    __shared__ int s_ok;
    wait_vm();   // this workgroup's stores complete before thread 0 releases them
    __syncthreads();
    if (threadIdx.x == 0) {
        int ok = 1;
        if (SYSTEM)
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
        else
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const uint32_t g = blockIdx.x % kBarGroups;
        const uint32_t ng = nblocks < (uint32_t)kBarGroups ? nblocks : (uint32_t)kBarGroups;
        const uint32_t in_g = (nblocks - g + kBarGroups - 1) / kBarGroups;
        uint32_t* cg = bar + (size_t)(1 + g) * kArriveStride;
        bool last = false;
        if (nblocks <= (uint32_t)kBarFlatMax) {
            if (__hip_atomic_fetch_add(&bar[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                nblocks - 1) {
                __hip_atomic_store(&bar[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
                last = true;
            }
        } else if (__hip_atomic_fetch_add(cg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   in_g - 1) {
            __hip_atomic_store(cg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // what the group's workgroups released goes on with the top arrival
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
            if (__hip_atomic_fetch_add(&bar[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                ng - 1) {
                __hip_atomic_store(&bar[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
                last = true;
            }
        }
        if (last) {
            __hip_atomic_store(&bar[kBarGen], gen + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
            while (__hip_atomic_load(&bar[kBarGen], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   gen) {
                if (__builtin_amdgcn_s_memrealtime() - t0 > kBarrierTimeoutTicks) {
                    set_error(st, EP_ERR_TIMEOUT);
                    ok = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_ok = ok;
    }
    __syncthreads();
    return s_ok != 0;
}

}  // namespace ep
