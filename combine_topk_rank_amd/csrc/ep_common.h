// ep_common.h — definitions shared by the HIP sources of the dispatch/combine
// library (device-side ring view, workspace carving, shape validation).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ep.h"

namespace ep {

constexpr int kWave = 64;          // CDNA wavefront width (UCCL-EP article s5.1: 32 -> 64)
constexpr int kBlock = 256;        // threads per workgroup: 4 wavefronts
constexpr int kLayoutTile = 256;   // tokens per layout workgroup
constexpr int kMsgRows = 8;        // rows per WRITE message (UCCL-EP s4.1 packing, s5.3 batch 8)
constexpr int kMaxR = 64;          // a rank set is one 64-bit mask
constexpr int kMaxE = 4096;        // per-expert LDS histogram bound
constexpr int kMaxK = 32;          // experts of a token sit in lanes 0..k-1
constexpr int kPad = 8;            // 64-byte stride between per-channel counters
// Bound on a grid-barrier wait, in s_memrealtime ticks (100 MHz): one second.
constexpr unsigned long long kBarrierTimeoutTicks = 100000000ull;

// One FIFO slot as it sits in the ring: four 64-bit words, each
//   bits  0..15  tag = low 16 bits of (ticket + 1)
//   bits 16..63  48 bits of the command:
//     w0: type (8) | op (8) | num_tokens (16) | 0 (16)
//     w1: dst_rank (16) | size_or_value (32)
//     w2: src_offset (48)
//     w3: dst_offset (48)
// The GPU writes the words with two plain 16-byte stores followed by a
// system-scope release, in any order and with no flag write; a consumer that reads the four words (8-byte
// loads are single-copy atomic) and finds the expected tag in all of them has
// the whole command.  A stale slot holds the tag of ticket - depth + 1, which
// differs as long as depth < 65536.  The consumer decodes slots into
// ep_transfer_cmd_t.
struct RingSlot {
    uint64_t w[4];
};
static_assert(sizeof(RingSlot) == 32, "ring slot is 32 bytes");
constexpr uint64_t kMaxRingOffset = (1ull << 48) - 1;
constexpr int32_t kMaxRingDepth = 65535;

// Device view of a TransferCmd ring.
struct RingDev {
    RingSlot* slots;                       // host-pinned, [channels][depth]
    const unsigned long long* host_tail;   // host-pinned, consumer position, stride kPad
    unsigned long long* head;              // device, ticket counter, stride kPad
    unsigned long long* tail_cache;        // device, last consumer position seen, stride kPad
    unsigned long long* poll;              // device, 1 while a lane reads host_tail, stride kPad
    int32_t depth;
    int32_t channels;
    int32_t max_inflight;
    int32_t pad_;
    unsigned long long timeout_ticks;      // in s_memrealtime ticks
};

// Carved workspace.
struct Workspace {
    uint32_t* barrier;        // [2] grid barrier: arrivals, generation (zero at first use)
    int32_t* blk_rank_cnt;    // [NB, R] per-layout-block rank counts
    int32_t* blk_exp_cnt;     // [NB, E] per-layout-block expert counts
    int32_t* msg_base;        // [R+1]   first message index of each rank
    int32_t* msg_arrivals;    // [max_msgs] rows (x chunks) written per message
    int32_t* rank_msgs_done;  // [R]     messages of a rank published
    int64_t max_msgs;
    int64_t counters_n;       // msg_arrivals .. rank_msgs_done, contiguous
    int32_t layout_blocks;
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int32_t layout_blocks(int32_t T) {
    return (int32_t)(T <= 0 ? 1 : ceil_div(T, kLayoutTile));
}

inline int64_t max_messages(const ep_shape_t& s) {
    int64_t kr = s.k < s.R ? s.k : s.R;
    return ceil_div((int64_t)s.T * kr, kMsgRows) + s.R;
}

size_t workspace_bytes(const ep_shape_t& s);
Workspace carve_workspace(const ep_shape_t& s, void* base);
int validate_shape(const ep_shape_t* s);
size_t row_bytes(int32_t H, int32_t fmt);

// Remember the last failing HIP call of this thread (ep_last_error).
void record_hip_error(hipError_t e, const char* what);

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
__device__ inline uint64_t bcast64(uint64_t v, int l) {
    uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}
__device__ inline float bcastf(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Number of set bits of `m` below this lane.
__device__ inline int lane_prefix(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

}  // namespace ep
