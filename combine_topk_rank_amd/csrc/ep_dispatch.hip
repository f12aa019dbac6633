// ep_dispatch.hip — pack/permute of token rows into rank-contiguous send
// buffers (bf16, or OCP e4m3 with per-128 float scales) and emission of
// batched TransferCmd descriptors into the FIFO a CPU proxy drains.
//
// UCCL-EP article:
//   s4.1 the dispatch kernel prepares the token data, synchronises, then posts
//        the transfer and goes on without waiting;  small tokens are packed,
//        several per message (s5.3: batch of 8);
//   s2.2 the FIFO: lock-free head reservation with atomics, a producer blocks
//        while 256 commands are in flight;
//   s2.3 WRITE fields (dst_rank, src_offset, dst_offset, size);
//   s3.1/s3.2 the Atomic message with an op and a 28-bit value;
//   s4.2 one FIFO per channel.
//
// Work decomposition (token-major): wavefront g handles chunk g % nchunks of
// token g / nchunks.  It reads its chunk of x once (16-byte loads) and stores
// it to every destination slot of the token (16-byte stores; 8-byte stores of
// codes for fp8), so x is read once and the packed rows written once.  Rows
// are stored with system-scope stores, which are written through to memory:
// once a wavefront's stores are complete, another agent (the NIC a proxy
// drives, here the CPU) may read them.  A message is the <= 8 consecutive
// rows [o_r + 8m, ...) of rank r; those rows come from different tokens.
//
// Large batches publish as messages complete.  Workgroups loop over groups
// of consecutive wavefronts; after each group, wavefront 0 counts the group's
// rows into their messages' arrival counters (one atomic per message and
// group) and the last arrival of a message publishes its WRITE; the last
// WRITE of a rank also publishes the rank's ATOMIC (its row count), whose
// ticket is taken after every WRITE ticket of the rank, so the proxy, which
// pops in ticket order, sees the count after the rows.  Small batches publish
// in closed form: the last workgroup to finish emits every command from the
// per-rank counts.

#include <atomic>

#include "ep_common.h"
#include "ep_route.h"

namespace ep {
RingDev ring_device_view(ep_ring_t* r);

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));


struct PackArgs {
    const u32x4* x;               // [T, H/8] 16-byte vectors
    const int32_t* idx;           // [T, k]
    const float* w;               // [T, k]
    const int32_t* rank_off;      // [R+1]
    const int32_t* send_slot;     // [T, R]
    uint8_t* send_buf;            // [cap, row_bytes]
    int32_t* slot_src;            // [cap]
    int32_t* slot_local_idx;      // [cap, k]
    float* slot_local_w;          // [cap, k]
    const int32_t* msg_base;      // [R+1]
    int32_t* msg_arrivals;        // [max_msgs]
    int32_t* msgs_done;           // [E] messages of a rank / an expert published
    int32_t* st;
    RingDev ring;
    int64_t max_msgs;             // entries of msg_arrivals
    int64_t cap;
    int64_t row_bytes;
    int32_t T, H, E, R, k, epr;
    int32_t nv;                   // 16-byte vectors per x row (H/8)
    int32_t nchunks;              // wavefronts per token
    int32_t has_ring;
    int64_t ngroups;              // groups of a workgroup's wavefronts (one per pass)
    uint32_t* arrive;             // arrival counters (workspace, zero between calls)
    // per-expert mode
    const int32_t* exp_off;       // [E+1]
    const int32_t* expert_slot;   // [T, k]
    float* slot_w;                // [cap]
    // one-kernel small batches: the layout outputs
    int32_t* cnt_rank_out;        // [R]
    int32_t* cnt_exp_out;         // [E]
    int32_t* rank_off_out;        // [R+1]
    int32_t* exp_off_out;         // [E+1]
    uint8_t* in_rank_out;         // [T, R]
    int32_t* send_slot_out;       // [T, R]
    int32_t* msg_base_out;        // [R+1] (workspace)
    int64_t counters_n;           // msg_arrivals .. msgs_done
    // one-kernel large batches
    uint32_t* bar;                // grid barrier words (workspace)
    int32_t* wave_cnt;            // [ceil(T/64), R] per-64-token rank counts (workspace)
    int32_t* exp_part;            // [nparts, E] partial expert counts (workspace)
    int32_t nparts;               // workgroup b adds into part b % nparts (<= kExpParts)
    int32_t expert_wg;            // 1: one workgroup more counts the experts
    int32_t npass;                // groups per pack workgroup, at most
};

// ------------------------------------------------------------------ ring

// Write one command into its slot: four tagged 8-byte words in two 16-byte
// stores; the tags make the order in which the words land irrelevant.  With
// SYS the stores have system scope and go through to host memory by
// themselves; otherwise they are cached and the caller releases each round
// of writes at system scope (see ring_publish_n).  The rows the command
// points to were complete at system scope before its ticket was taken.
template <bool SYS>
__device__ inline void ring_write(const RingDev& g, int c, unsigned long long ticket, uint32_t type,
                                  uint32_t op, uint32_t ntok, uint32_t dst_rank, uint32_t size_val,
                                  uint64_t src_off, uint64_t dst_off) {
    RingSlot* slot = g.slots + (size_t)c * g.depth + (size_t)(ticket % (unsigned long long)g.depth);
    uint64_t w[4];
    ring_slot_words(ticket, type, op, ntok, dst_rank, size_val, src_off, dst_off, w);
    if (SYS) {
        // A descriptor per slot: lanes with different slots get separate
        // store instructions (the compiler loops over the distinct
        // descriptors), so each 16-byte store travels to host memory on its
        // own.  One descriptor over all slots with per-lane offsets, one
        // instruction for all lanes, made every dispatch far slower (train
        // step 192 -> 307 us, skewed 636 -> 980 us).
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(slot, (int32_t)sizeof(RingSlot));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, (u64x2{w[0], w[1]})), rs,
                                               0, 0, kStoreSystem);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, (u64x2{w[2], w[3]})), rs,
                                               16, 0, kStoreSystem);
    } else {
        u64x2* p = reinterpret_cast<u64x2*>(slot);
        p[0] = u64x2{w[0], w[1]};
        p[1] = u64x2{w[2], w[3]};
    }
}

// Reserve n consecutive tickets on channel c (one atomic per reservation).
__device__ inline unsigned long long ring_reserve(const RingDev& g, int c, unsigned n) {
    return atomicAdd(g.head + (size_t)c * kPad, (unsigned long long)n);
}

struct RingCmd {
    uint32_t type, op, ntok, dst_rank, size_val;
    uint64_t src_off, dst_off;
};

// Up to N commands per lane, all on the lane's channel c (the first n of
// them, n <= N): wait until each ticket may be written -- fewer than
// max_inflight commands of the channel published but not yet drained --
// write it, and make it visible to the CPU.  The waits and the writes share
// one wave-uniform loop, so a command whose ticket is ready is written at once
// even while other commands of the wavefront still wait (they may wait on
// it).  A command is given up when the ring's timeout passes (status set) or
// when another producer has already failed.  SYS: system-scope slot stores
// (best for a few commands per wavefront: each lane's 16-byte stores travel
// on their own); otherwise cached stores and one system-scope release per
// round (best for runs of consecutive slots, which leave the L2 as lines).
// `seen0`, when not ~0, is the cached consumer position of channel c as the
// caller already loaded it (saves this call a load).
template <int N, bool SYS>
__device__ void ring_publish_n(const RingDev& g, int n, int c, const unsigned long long* ticket,
                               const RingCmd* cmd, int32_t* st, unsigned long long seen0 = ~0ull) {
    if (!__ballot(n > 0)) return;
    const unsigned long long lim = (unsigned long long)g.max_inflight;
    unsigned long long* cache = g.tail_cache + (size_t)c * kPad;
    unsigned long long* poll = g.poll + (size_t)c * kPad;
    const unsigned long long* htail = g.host_tail + (size_t)c * kPad;
    unsigned long long seen = 0, t0 = 0;
    uint32_t pending = (1u << n) - 1u;
    bool polled = false;
    if (pending)
        seen = seen0 != ~0ull ? seen0
                              : __hip_atomic_load(cache, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (__ballot(pending != 0)) {
        bool progress = false;
        if (pending) {
            // the lowest pending ticket decides whether the cache is refreshed
            unsigned long long lo = ~0ull;
#pragma unroll
            for (int i = 0; i < N; ++i)
                if (((pending >> i) & 1u) && ticket[i] < lo) lo = ticket[i];
            if (lo >= seen + lim) {
                // The cached consumer position says full.  One lane per
                // channel at a time reads the real one over PCIe and
                // refreshes the cache; the others read the cache.
                if (atomicCAS(poll, 0ull, 1ull) == 0ull) {
                    unsigned long long h =
                        __hip_atomic_load(htail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                    atomicMax(cache, h);
                    atomicExch(poll, 0ull);
                }
                unsigned long long cv =
                    __hip_atomic_load(cache, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (cv > seen) seen = cv;
            }
#pragma unroll
            for (int i = 0; i < N; ++i) {
                if (((pending >> i) & 1u) && ticket[i] < seen + lim) {
                    ring_write<SYS>(g, c, ticket[i], cmd[i].type, cmd[i].op, cmd[i].ntok,
                                    cmd[i].dst_rank, cmd[i].size_val, cmd[i].src_off,
                                    cmd[i].dst_off);
                    pending &= ~(1u << i);
                    progress = true;
                }
            }
            if (pending && !progress) {
                if (read_status(st) != 0) {
                    pending = 0;
                } else {
                    const unsigned long long now = __builtin_amdgcn_s_memrealtime();
                    if (!polled) {
                        polled = true;
                        t0 = now;
                    } else if (now - t0 > g.timeout_ticks) {
                        set_error(st, EP_ERR_RING_TIMEOUT);
                        pending = 0;
                    }
                }
            }
        }
        if (__ballot(progress)) {
            // one system-scope release pushes this round's slots out of the
            // L2 to host memory, where the proxy polls them
            if (!SYS) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
        } else if (__ballot(pending != 0)) {
            __builtin_amdgcn_s_sleep(16);
        }
    }
}

// One command per lane (lanes with `have`).
template <bool SYS>
__device__ inline void ring_publish(const RingDev& g, bool have, int c, unsigned long long ticket,
                                    uint32_t type, uint32_t op, uint32_t ntok, uint32_t dst_rank,
                                    uint32_t size_val, uint64_t src_off, uint64_t dst_off,
                                    int32_t* st) {
    const RingCmd cmd{type, op, ntok, dst_rank, size_val, src_off, dst_off};
    ring_publish_n<1, SYS>(g, have ? 1 : 0, c, &ticket, &cmd, st);
}

// Wavefront 0 of a workgroup, after the rows of its current group (kWaves
// consecutive wavefronts, hence consecutive tokens) are released: lane r
// takes rank r.  slot[w][r] is the slot of rank r written by wavefront w of
// the group (-1 for none).  The group's slots of rank r ascend with w and
// are consecutive, so they fall into at most three consecutive messages;
// each message gets one arrival atomic carrying the group's row count (x
// chunks).  A message whose count completes is published (WRITE); the
// rank's last message also publishes the rank's ATOMIC.
//
// The chain of memory round trips is kept short: the rank's rows and first
// message (RankView) are loaded once per launch; the status word and the
// channel's cached consumer position are loaded with the arrival atomics; the
// WRITEs go out before the count of the rank's published messages returns,
// which only the ATOMIC waits for.
struct RankView {
    int32_t o[kMaxR], cnt[kMaxR], mbase[kMaxR];   // rank r's first row, rows, first message
};

// Fill the workgroup's RankView (LDS); wavefront 0, once per launch.
__device__ inline void load_rank_view(const PackArgs& a, RankView& v) {
    const int lane = lane_id();
    if (lane < a.R) {
        const int32_t o = a.rank_off[lane];
        v.o[lane] = o;
        v.cnt[lane] = a.rank_off[lane + 1] - o;
        v.mbase[lane] = a.msg_base[lane];
    }
}

// Up to N commands per lane, command i on its own channel c[i] (those with
// bit i of `have`): as ring_publish_n, each command written as soon as its ticket is
// inside its channel's window, so no command of the wavefront waits for
// another of the same wavefront.  System-scope slot stores.  `seen0`, when
// not NULL, holds the cached consumer position of each command's channel as
// the caller already loaded it.
template <int N>
__device__ void ring_publish_v(const RingDev& g, uint32_t have, const int* c,
                               const unsigned long long* ticket, const RingCmd* cmd, int32_t* st,
                               const unsigned long long* seen0 = nullptr) {
    if (!__ballot(have != 0)) return;
    const unsigned long long lim = (unsigned long long)g.max_inflight;
    unsigned long long seen[N];
    uint32_t pending = have;
#pragma unroll
    for (int i = 0; i < N; ++i)
        seen[i] = !((pending >> i) & 1u) ? 0ull
                  : seen0                ? seen0[i]
                                         : __hip_atomic_load(g.tail_cache + (size_t)c[i] * kPad,
                                                             __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT);
    bool polled = false;
    unsigned long long t0 = 0;
    while (__ballot(pending != 0)) {
        bool progress = false;
        if (pending) {
#pragma unroll
            for (int i = 0; i < N; ++i) {
                if (!((pending >> i) & 1u) || ticket[i] < seen[i] + lim) continue;
                // the cached consumer position says full: one lane per channel
                // at a time reads the real one over PCIe and refreshes the cache
                unsigned long long* poll = g.poll + (size_t)c[i] * kPad;
                unsigned long long* cache = g.tail_cache + (size_t)c[i] * kPad;
                if (atomicCAS(poll, 0ull, 1ull) == 0ull) {
                    const unsigned long long h = __hip_atomic_load(
                        g.host_tail + (size_t)c[i] * kPad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                    atomicMax(cache, h);
                    atomicExch(poll, 0ull);
                }
                const unsigned long long cv =
                    __hip_atomic_load(cache, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (cv > seen[i]) seen[i] = cv;
            }
#pragma unroll
            for (int i = 0; i < N; ++i) {
                if (((pending >> i) & 1u) && ticket[i] < seen[i] + lim) {
                    ring_write<true>(g, c[i], ticket[i], cmd[i].type, cmd[i].op, cmd[i].ntok,
                                     cmd[i].dst_rank, cmd[i].size_val, cmd[i].src_off,
                                     cmd[i].dst_off);
                    pending &= ~(1u << i);
                    progress = true;
                }
            }
            if (pending && !progress) {
                if (read_status(st) != 0) {
                    pending = 0;
                } else {
                    const unsigned long long now = __builtin_amdgcn_s_memrealtime();
                    if (!polled) {
                        polled = true;
                        t0 = now;
                    } else if (now - t0 > g.timeout_ticks) {
                        set_error(st, EP_ERR_RING_TIMEOUT);
                        pending = 0;
                    }
                }
            }
        }
        if (!__ballot(progress) && __ballot(pending != 0)) __builtin_amdgcn_s_sleep(16);
    }
}

// ATOMIC{ADD, cnt} for ranks that receive no rows (nothing to order after).
__device__ void publish_empty_ranks(const PackArgs& a, const RankView& rv) {
    const int lane = lane_id();
    bool have = false;
    int c = 0;
    unsigned long long tk = 0;
    if (lane < a.R && rv.cnt[lane] == 0) {
        have = true;
        c = lane % a.ring.channels;
        tk = ring_reserve(a.ring, c, 1);
    }
    ring_publish<true>(a.ring, have, c, tk, EP_CMD_ATOMIC, EP_ATOMIC_ADD, 0, (uint32_t)lane, 0, 0,
                       0, a.st);
}

template <int W>
__device__ void publish_group(const PackArgs& a, const RankView& rv,
                              const int32_t (*slot)[kMaxR]) {
    const int lane = lane_id();
    const bool has = lane < a.R;
    const int C = a.ring.channels;
    const int32_t o = has ? rv.o[lane] : 0, cnt = has ? rv.cnt[lane] : 0;
    const int32_t mbase = has ? rv.mbase[lane] : 0;
    // rows per message, relative to the first message m0 the group touches
    int32_t m0 = -1, cnt3[3] = {0, 0, 0};
    bool bad = false;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        const int32_t sl = has ? slot[w][lane] : -1;
        if (sl >= 0) {
            if (sl < o || sl >= o + cnt) {
                bad = true;   // send_slot does not belong to rank_offset
            } else {
                const int32_t m = (sl - o) / kMsgRows;
                if (m0 < 0) m0 = m;
                const int32_t d = m - m0;
                if (d == 0) ++cnt3[0];
                else if (d == 1) ++cnt3[1];
                else if (d == 2) ++cnt3[2];
                else bad = true;   // slots of a rank not ascending through the group
            }
        }
    }
    bool hit[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        hit[i] = m0 >= 0 && cnt3[i] > 0;
        if (hit[i] && mbase + m0 + i >= a.max_msgs) bad = true;   // message table too small
    }
    // An inconsistent group is reported before it counts any row or takes
    // any ticket: none of its messages is ever published.
    if (__ballot(bad)) {
        if (bad) set_error(a.st, EP_ERR_INVALID_ARG);
        return;
    }
    // the status, the cached consumer positions and the (at most three)
    // arrival atomics go out together: one latency
    const int32_t st0 = read_status(a.st);
    unsigned long long tc = 0;
    if (lane < C)
        tc = __hip_atomic_load(a.ring.tail_cache + (size_t)lane * kPad, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    int32_t old3[3] = {0, 0, 0};
#pragma unroll
    for (int i = 0; i < 3; ++i)
        if (hit[i]) old3[i] = atomicAdd(&a.msg_arrivals[mbase + m0 + i], cnt3[i]);
    // completed messages, in ascending order, in registers (no indexed
    // private array)
    int32_t done_m[3] = {0, 0, 0};
    int ndone = 0;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        if (!hit[i]) continue;
        const int32_t m = m0 + i;
        const int32_t nrows = min(kMsgRows, cnt - m * kMsgRows);
        if (old3[i] + cnt3[i] == nrows * a.nchunks) {
            a.msg_arrivals[mbase + m] = 0;   // every arrival is in: leave the counter clean
#pragma unroll
            for (int q = 0; q <= i; ++q)
                if (ndone == q) done_m[q] = m;
            ++ndone;
        }
    }
    if (!__ballot(ndone > 0)) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const int c = lane % C;
    const unsigned long long seen = (unsigned long long)__shfl((long long)tc, c);
    unsigned long long tk[3] = {0, 0, 0};
    int nw = 0;
    int32_t done = 0;
    if (ndone > 0 && st0 == 0) {
        const unsigned long long t0 = ring_reserve(a.ring, c, (unsigned)ndone);
#pragma unroll
        for (int i = 0; i < 3; ++i) tk[i] = t0 + i;
        nw = ndone;
        // Count the messages into the rank once their WRITE tickets exist (the
        // added value depends on the ticket); the rank's last messages
        // reserve the ATOMIC's ticket, which then follows every WRITE ticket
        // of the rank.
        const int32_t add = ndone + (int32_t)(t0 >> 62);
        done = atomicAdd(&a.msgs_done[lane], add);
    }
    const uint64_t rb = (uint64_t)a.row_bytes;
    RingCmd cmd[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int32_t m = done_m[i];
        const int32_t nrows = min(kMsgRows, cnt - m * kMsgRows);
        cmd[i] = RingCmd{EP_CMD_WRITE, 0, (uint32_t)nrows, (uint32_t)lane, (uint32_t)(nrows * rb),
                         (uint64_t)(o + m * kMsgRows) * rb, (uint64_t)(m * kMsgRows) * rb};
    }
    ring_publish_n<3, true>(a.ring, nw, c, tk, cmd, a.st, seen);
    bool atom = false;
    unsigned long long ta = 0;
    if (nw > 0 && done + ndone == (cnt + kMsgRows - 1) / kMsgRows) {
        a.msgs_done[lane] = 0;
        ta = ring_reserve(a.ring, c, 1);
        atom = true;
    }
    ring_publish<true>(a.ring, atom, c, ta, EP_CMD_ATOMIC, EP_ATOMIC_ADD, 0, (uint32_t)lane,
                       (uint32_t)cnt, 0, 0, a.st);
}

// Closed-form command stream (every row written and released first).  Per
// channel c, its ranks r = c, c + C, ... ascending; per rank, the WRITEs of
// its messages 0, 1, ..., then its ATOMIC (also for a rank with no rows).
// The streams are concatenated channel-major; lane l of a wavefront takes
// the l-th rank of that order (R <= 64).
struct ClosedOrder {
    int32_t r;        // rank at this lane's position (lanes < R)
    int32_t c;        // its channel
    int32_t o, cnt;   // its rows in the send buffer
    int32_t items;    // its commands: ceil(cnt / 8) WRITEs + 1 ATOMIC
    int32_t start;    // its first command in the concatenated order
    int32_t cstart;   // first command of its channel
    int32_t total;    // all commands (wave-uniform)
};

__device__ inline ClosedOrder closed_order(const PackArgs& a, const int32_t* ro) {
    const int lane = lane_id();
    const int C = a.ring.channels, R = a.R;
    const int q = R / C, rem = R % C;   // channels < rem hold q + 1 ranks
    ClosedOrder z{};
    int i = 0;
    if (lane < R) {
        if (lane < rem * (q + 1)) {
            z.c = lane / (q + 1);
            i = lane % (q + 1);
        } else {
            const int l2 = lane - rem * (q + 1);
            z.c = rem + l2 / q;
            i = l2 % q;
        }
        z.r = z.c + i * C;
        z.o = ro[z.r];
        z.cnt = ro[z.r + 1] - z.o;
        z.items = (z.cnt + kMsgRows - 1) / kMsgRows + 1;
    }
    int32_t incl = z.items;
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
    }
    z.start = incl - z.items;
    z.cstart = __shfl(z.start, lane - i);   // the channel's first rank sits i lanes back
    z.total = bcast(incl, kWave - 1);
    return z;
}

// Publish command g of the concatenated closed-form order (lanes with
// `have`); base[c] is the first ticket of channel c.
__device__ void closed_publish(const PackArgs& a, const ClosedOrder& z,
                               const unsigned long long* base, const unsigned long long* seen,
                               int32_t g, bool have) {
    int j = 0;   // position holding command g
    for (int p = 1; p < a.R; ++p)
        if (bcast(z.start, p) <= g) j = p;
    const int32_t local = g - __shfl(z.start, j);
    const int32_t c = __shfl(z.c, j), r = __shfl(z.r, j);
    const int32_t o = __shfl(z.o, j), cnt = __shfl(z.cnt, j);
    const int32_t nmsg = __shfl(z.items, j) - 1;
    const int32_t cstart = __shfl(z.cstart, j);
    const unsigned long long ticket = have ? base[c] + (unsigned long long)(g - cstart) : 0;
    const bool write = local < nmsg;
    const int32_t rows = write ? min(kMsgRows, cnt - local * kMsgRows) : 0;
    const uint64_t rb = (uint64_t)a.row_bytes;
    const RingCmd cmd{write ? (uint32_t)EP_CMD_WRITE : (uint32_t)EP_CMD_ATOMIC,
                      write ? 0u : (uint32_t)EP_ATOMIC_ADD, (uint32_t)rows, (uint32_t)r,
                      write ? (uint32_t)(rows * rb) : (uint32_t)cnt,
                      write ? (uint64_t)(o + local * kMsgRows) * rb : 0,
                      write ? (uint64_t)(local * kMsgRows) * rb : 0};
    // the channel's cached consumer position came with the reservation
    ring_publish_n<1, false>(a.ring, have ? 1 : 0, c, &ticket, &cmd, a.st,
                             have ? seen[c] : ~0ull);
}

// One ticket reservation per channel for all of its commands (wavefront-wide;
// lane of a channel's first rank reserves), bases stored to base[c]; the
// channel's first command and command count go to cstart[c] and cnum[c].
__device__ void closed_reserve(const PackArgs& a, const ClosedOrder& z, unsigned long long* base,
                               unsigned long long* seen, int32_t* cstart, int32_t* cnum) {
    const int lane = lane_id();
    const int C = a.ring.channels, R = a.R;
    const int q = R / C, rem = R % C;
    const int nr = z.c < rem ? q + 1 : q;   // ranks of this lane's channel
    const int nxt = lane + nr;              // the next channel's first rank, if any
    const int32_t nxt_start = __shfl(z.start, nxt < kWave ? nxt : kWave - 1);
    if (lane < R && z.start == z.cstart) {   // lane of a channel's first rank
        const int32_t n = (nxt < R ? nxt_start : z.total) - z.cstart;
        // the cached consumer position travels with the reservation (one
        // latency for both); the writes check their tickets against it
        const unsigned long long sn = __hip_atomic_load(
            a.ring.tail_cache + (size_t)z.c * kPad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        base[z.c] = ring_reserve(a.ring, z.c, (unsigned)n);
        seen[z.c] = sn;
        cstart[z.c] = z.cstart;
        cnum[z.c] = n;
    }
}

// The whole closed-form stream, by every thread of a workgroup of NT
// threads.  The channels advance together: in each round thread i takes
// channel i % nch and the next command of that channel's stream, so every
// channel's window fills (and its proxy drains) from the start instead of
// one channel after another.
template <int NT>
__device__ void closed_publish_all(const PackArgs& a, const ClosedOrder& z,
                                   const unsigned long long* base, const unsigned long long* seen,
                                   const int32_t* cstart, const int32_t* cnum) {
    const int nch = a.ring.channels < a.R ? a.ring.channels : a.R;
    const int per_round = NT / nch;
    int32_t nmax = 0;
    for (int c = 0; c < nch; ++c) nmax = cnum[c] > nmax ? cnum[c] : nmax;
    const int c = (int)threadIdx.x % nch;
    const int32_t jt = (int32_t)threadIdx.x / nch;
    for (int32_t j0 = 0; j0 < nmax; j0 += per_round) {
        const int32_t j = j0 + jt;
        const bool have = jt < per_round && j < cnum[c];
        closed_publish(a, z, base, seen, have ? cstart[c] + j : 0, have);
    }
}

// Count this workgroup out after its rows were released at system scope;
// true in the last workgroup to finish.  Grids of more than flat_max
// workgroups use two levels to spread the contention: workgroups b = g (mod
// kArriveGroups) share counter g (consecutive workgroups go to different
// XCDs, so a group tends to sit on one), and the last of each group counts
// into the top counter.  Smaller grids count straight into the top counter:
// one atomic round trip and one cache write-back less for the last arrival,
// whose publication is what the batch waits for.  The rank-mode small
// batches, whose workgroups finish spread over microseconds, take that up to
// 256 workgroups (decode step 22.6 -> 21.9 us); the per-expert one-kernel
// dispatch only up to 128 (at 224 workgroups its decode step was 2 us
// slower with one counter).  Every counter is reset by the arrival that
// completes it, so the words are zero between calls.
constexpr int kArriveGroups = 8;
constexpr uint32_t kArriveFlatRank = 256, kArriveFlatDefault = 128;
__device__ bool arrive_last(uint32_t* ctr, uint32_t flat_max = kArriveFlatDefault) {
    const uint32_t nb = gridDim.x;
    if (nb <= flat_max) {
        if (__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != nb - 1)
            return false;
        __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        return true;
    }
    const uint32_t g = blockIdx.x % kArriveGroups;
    const uint32_t ng = nb < kArriveGroups ? nb : kArriveGroups;   // groups in use
    const uint32_t in_g = (nb - g + kArriveGroups - 1) / kArriveGroups;
    uint32_t* cg = ctr + (size_t)(1 + g) * kArriveStride;
    if (__hip_atomic_fetch_add(cg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != in_g - 1)
        return false;
    __hip_atomic_store(cg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // what the group's workgroups released is carried on to the top counter
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
    if (__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != ng - 1)
        return false;
    __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return true;
}

// Refresh the producers' cached consumer positions from host memory (one
// PCIe read per channel), so that publication later in the kernel does not
// find a stale "full" and wait for a read then.
__device__ void refresh_tail_cache(const PackArgs& a) {
    const int c = lane_id();
    if (c < a.ring.channels) {
        const unsigned long long h = __hip_atomic_load(a.ring.host_tail + (size_t)c * kPad,
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        atomicMax(a.ring.tail_cache + (size_t)c * kPad, h);
    }
}

// The same in two halves, for a wavefront that also copies rows: the PCIe
// read is issued first and its value applied after the wavefront's rows,
// so the read's latency does not delay them.
__device__ inline unsigned long long tail_read(const PackArgs& a) {
    const int c = lane_id();
    return c < a.ring.channels
               ? __hip_atomic_load(a.ring.host_tail + (size_t)c * kPad, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_SYSTEM)
               : 0ull;
}
__device__ inline void tail_apply(const PackArgs& a, unsigned long long h) {
    const int c = lane_id();
    if (c < a.ring.channels) atomicMax(a.ring.tail_cache + (size_t)c * kPad, h);
}

// ------------------------------------------------------------------ fp8
// Round to nearest even with saturation to +-448: clamp, then the gfx950
// OCP e4m3 conversion (round to nearest even).
template <bool HI>
__device__ inline uint32_t e4m3x2(float a, float b, uint32_t old) {
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

__device__ inline float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf16hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Largest magnitude among the four bf16 values of two words, as the bf16
// bit pattern.  Magnitudes of bf16 values order like unsigned integers, an
// infinity (0x7F80) above every finite value and NaN patterns above that.
__device__ inline uint32_t max_bf16_mag(uint32_t a, uint32_t b) {
    const uint32_t a0 = a & 0x7FFFu, a1 = (a >> 16) & 0x7FFFu;
    const uint32_t b0 = b & 0x7FFFu, b1 = (b >> 16) & 0x7FFFu;
    const uint32_t x = a0 > a1 ? a0 : a1;
    const uint32_t y = b0 > b1 ? b0 : b1;
    return x > y ? x : y;
}

// The same with NaN patterns left out (they count as zero): a NaN has no
// magnitude to compare, so it does not take part in a block's maximum.
__device__ inline uint32_t max_bf16_mag_num(uint32_t a, uint32_t b) {
    uint32_t m[4] = {a & 0x7FFFu, (a >> 16) & 0x7FFFu, b & 0x7FFFu, (b >> 16) & 0x7FFFu};
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) r = (m[i] <= 0x7F80u && m[i] > r) ? m[i] : r;
    return r;
}

// Codes of the eight values of u (bytes in element order) whose product
// x * inv is NaN -- x is NaN, or x is infinite in a block whose maximum is
// infinite (inv = 0) -- become the NaN code 0x7F with the sign of x; the
// clamp before the conversion would have turned them into -448.
__device__ inline u32x2 nan_codes(const u32x4 u, float inv, u32x2 q) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    uint32_t out[2] = {q.x, q.y};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t b = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        const float p = __uint_as_float(b << 16) * inv;
        if (p != p) {
            const int sh = 8 * (e & 3);
            out[e >> 2] = (out[e >> 2] & ~(0xFFu << sh)) | ((0x7Fu | ((b >> 8) & 0x80u)) << sh);
        }
    }
    return u32x2{out[0], out[1]};
}

// max over the 16 lanes of a row group (a 128-element block is 16 lanes x 8)
__device__ inline float group16_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 1));
    v = fmaxf(v, __shfl_xor(v, 2));
    v = fmaxf(v, __shfl_xor(v, 4));
    v = fmaxf(v, __shfl_xor(v, 8));
    return v;
}

// ------------------------------------------------------------------ kernel
// Wavefronts per pack workgroup: they share one system-scope release for
// their rows and one wavefront publishes their descriptors.
constexpr int kPackWaves = 16;
constexpr int kPackWavesFp8 = 8;
// Below this many whole-chunk wavefronts, pack uses 2-vector chunks in
// workgroups of kPackWavesSmall wavefronts.
constexpr int64_t kPackSmallWaves = 1024;
constexpr int kPackWavesSmall = 4;
// Vectors per lane for rows of up to 896 vectors (H = 7168): 14 = one
// wavefront per row, 7 = two.
constexpr int kPackVplH7168 = 14;
constexpr int kPackVplFp8H7168 = 14;
// Pack workgroups per compute unit by default: with fewer workgroups than
// groups, each workgroup loops, so rows complete (and descriptors are
// published) in several generations instead of all at the end of the kernel.
// Half the compute units with 16 wavefronts each; the rank-mode streaming
// pack goes up to all of them for large batches (stream_grid_cap).
constexpr int kPackGridPerCuNum = 1, kPackGridPerCuDen = 2;

// Store chunk `chunk` of token t's row into every destination slot of the
// wavefront: destination d (bit d of dmask) goes to slot bcast(s_lane, d).
// bf16 copies 16-byte vectors; fp8 quantises the chunk once and stores codes
// and scales.  Slots at or beyond the capacity are skipped.  All lanes of the
// wavefront call this together.
// This wavefront's chunk of row t of x: vectors v0 + lane + 64 i.
template <int VPL>
__device__ inline void load_row_chunk(const PackArgs& a, int64_t t, int chunk, u32x4 (&v)[VPL]) {
    const int lane = lane_id();
    const int v0 = chunk * VPL * kWave;
    const u32x4* xr = a.x + t * a.nv;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        int vi = v0 + lane + i * kWave;
        if (vi < a.nv) v[i] = xr[vi];
        else v[i] = u32x4{0, 0, 0, 0};
    }
}

// The same with buffer loads bounded by the row's bytes, for the one-kernel
// dispatches: vectors past the row read as zero with no branch, so nothing
// forces a wait for the data before its first use.  With the branch of
// load_row_chunk the compiler waits for the loads at once, so a prefetch
// issued ahead of the routing loads held them up; the one-kernel large
// dispatch also needs fewer registers with these (train 197.8 -> 196.3 us
// per step, skewed 691 -> 681 us).  The two-kernel bf16 pack keeps
// load_row_chunk.
// t and chunk are the same on every lane, but the compiler cannot see that
// (they derive from threadIdx.x / 64): read from the first lane, the buffer
// descriptor is scalar, and each load is one instruction instead of a loop
// over the distinct descriptors of the lanes.
template <int VPL>
__device__ inline void prefetch_row_chunk(const PackArgs& a, int64_t t, int chunk,
                                          u32x4 (&v)[VPL]) {
    const int lane = lane_id();
    t = (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)t >> 32)) << 32) |
                  (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)t));
    chunk = __builtin_amdgcn_readfirstlane(chunk);
    const int v0 = chunk * VPL * kWave;
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(const_cast<u32x4*>(a.x + t * a.nv), a.nv * (int32_t)sizeof(u32x4));
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (v0 + lane + i * kWave) * (int)sizeof(u32x4),
                                                     0, 0);
}

template <int VPL, int FMT>
__device__ inline void store_row_chunk_v(const PackArgs& a, int chunk, int32_t s_lane,
                                         uint64_t dmask, const u32x4 (&v)[VPL]);

template <int VPL, int FMT>
__device__ inline void store_row_chunk(const PackArgs& a, int64_t t, int chunk, int32_t s_lane,
                                       uint64_t dmask) {
    u32x4 v[VPL];
    load_row_chunk<VPL>(a, t, chunk, v);
    store_row_chunk_v<VPL, FMT>(a, chunk, s_lane, dmask, v);
}

// The stores of store_row_chunk, for a chunk already loaded into v.
template <int VPL, int FMT>
__device__ inline void store_row_chunk_v(const PackArgs& a, int chunk, int32_t s_lane,
                                         uint64_t dmask, const u32x4 (&v)[VPL]) {
    const int lane = lane_id();
    const int v0 = chunk * VPL * kWave;

    if (FMT == EP_FMT_BF16) {
        for (uint64_t m = dmask; m; m &= m - 1) {
            const int r = __builtin_ctzll(m);
            const int32_t s = bcast(s_lane, r);
            if (s >= a.cap) continue;
            const __amdgpu_buffer_rsrc_t dst =
                buffer_rsrc(a.send_buf + (int64_t)s * a.row_bytes, (int32_t)a.row_bytes);
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                int vi = v0 + lane + i * kWave;
                if (vi < a.nv)
                    __builtin_amdgcn_raw_buffer_store_b128(v[i], dst, vi * 16, 0,
                                                           kStoreSystem | kCacheNt);
            }
        }
    } else {
        // quantise once: per 128-element block, a = max(amax, 1e-4),
        // codes = e4m3(x * (448 / a)), scale = a / 448.  The block max is
        // taken on the bf16 bits (magnitudes order like unsigned integers),
        // so no float copy of the row stays live.  A lane holding an
        // infinity or a NaN (rare) takes the slow steps: NaNs stay out of
        // the maximum, NaN products get the NaN code.
        u32x2 q[VPL];
        float scale[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const u32x4 u = v[i];
            const uint32_t m01 = max_bf16_mag(u.x, u.y);
            const uint32_t m23 = max_bf16_mag(u.z, u.w);
            uint32_t mw = m01 > m23 ? m01 : m23;
            const bool nonfinite = mw >= 0x7F80u;
            if (mw > 0x7F80u) {
                const uint32_t n01 = max_bf16_mag_num(u.x, u.y);
                const uint32_t n23 = max_bf16_mag_num(u.z, u.w);
                mw = n01 > n23 ? n01 : n23;
            }
            float am = __uint_as_float(mw << 16);
            am = group16_max(am);
            const float av = fmaxf(am, 1e-4f);
            const float inv = 448.0f / av;
            scale[i] = av / 448.0f;
            uint32_t lo = e4m3x2<false>(bf16lo(u.x) * inv, bf16hi(u.x) * inv, 0);
            lo = e4m3x2<true>(bf16lo(u.y) * inv, bf16hi(u.y) * inv, lo);
            uint32_t hi = e4m3x2<false>(bf16lo(u.z) * inv, bf16hi(u.z) * inv, 0);
            hi = e4m3x2<true>(bf16lo(u.w) * inv, bf16hi(u.w) * inv, hi);
            q[i] = u32x2{lo, hi};
            if (nonfinite) q[i] = nan_codes(u, inv, q[i]);
        }
        // The tail of the row, [H, row_bytes), is 4-byte words: the scales of
        // blocks 0 .. H/128 - 1, then zeros.  This chunk writes the words of
        // its 4 VPL blocks, lane b holding block v0/16 + b (block 4i + l/16
        // of the chunk sits in lane l of vector i); the last chunk also
        // writes the zero words after them.  One store per destination
        // instead of one per vector, and whole 128-byte lines.
        static_assert(VPL <= 16, "a chunk's scales fit one wavefront");
        const int nblk = a.H / 128;
        const int nword = (int)((a.row_bytes - a.H) / 4);
        const int w0 = v0 / 16;
        const int wend = v0 + VPL * kWave >= a.nv ? nword : w0 + 4 * VPL;
        float sg = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const float g = __shfl(scale[i], (lane & 3) * 16);
            if ((lane >> 2) == i) sg = g;
        }
        if (w0 + lane >= nblk) sg = 0.0f;
        for (uint64_t m = dmask; m; m &= m - 1) {
            const int r = __builtin_ctzll(m);
            const int32_t s = bcast(s_lane, r);
            if (s >= a.cap) continue;
            const __amdgpu_buffer_rsrc_t row =
                buffer_rsrc(a.send_buf + (int64_t)s * a.row_bytes, (int32_t)a.row_bytes);
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                int vi = v0 + lane + i * kWave;
                if (vi < a.nv)
                    __builtin_amdgcn_raw_buffer_store_b64(q[i], row, vi * 8, 0, kStoreSystem);
            }
            for (int wi = w0 + lane, j = 0; wi < wend; wi += kWave, ++j)
                __builtin_amdgcn_raw_buffer_store_b32(j == 0 ? __float_as_uint(sg) : 0u, row,
                                                      a.H + wi * 4, 0, kStoreSystem);
        }
    }

}

// Metadata of token t's slots (one per destination rank, lane r holding the
// slot of rank r): the source token, and per choice j the expert's index on
// the slot's rank (or -1) and its gate (or 0).  Slots at or beyond the
// capacity are skipped.  All lanes of the wavefront call this together.
__device__ inline void store_slot_metadata(const PackArgs& a, int64_t t, int32_t s_lane,
                                           uint64_t dmask) {
    const int lane = lane_id();
    int e = -1;
    float wt = 0.0f;
    if (lane < a.k) {
        e = a.idx[t * a.k + lane];
        wt = a.w[t * a.k + lane];
    }
    for (uint64_t m = dmask; m; m &= m - 1) {
        const int r = __builtin_ctzll(m);
        const int32_t s = bcast(s_lane, r);
        if (s >= a.cap) continue;
        if (lane < a.k) {
            const bool local = e >= 0 && e < a.E && (unsigned)(e - r * a.epr) < (unsigned)a.epr;
            a.slot_local_idx[(int64_t)s * a.k + lane] = local ? e - r * a.epr : -1;
            a.slot_local_w[(int64_t)s * a.k + lane] = local ? wt : 0.0f;
        }
        if (lane == 0) a.slot_src[s] = (int32_t)t;
    }
}

// How a pack kernel publishes descriptors.
//   kPubNone:   no ring.
//   kPubStream: as messages complete, overlapping the copy.  After each
//     group, the workgroup's wavefronts hand their (slot, rank) pairs to
//     wavefront 0 through LDS; it releases the group's rows at system scope,
//     counts them into their messages' arrival counters, and the last
//     arrival of a message publishes the WRITE (the last of a rank, also the
//     rank's ATOMIC).
//   kPubClosed (small batches): every workgroup writes and releases its
//     rows and counts itself out; the last one to finish reserves each
//     channel's tickets at once and publishes the whole command stream in
//     closed form from the counts.  No per-message counters, no waiting.
enum { kPubNone = 0, kPubStream = 1, kPubClosed = 2 };

template <int VPL, int FMT, int WAVES, int PUB>
__global__ __launch_bounds__(WAVES * kWave) void pack_kernel(PackArgs a) {
    constexpr int kWaves = WAVES;
    // group's slot of rank r per wavefront, two buffers by pass parity
    __shared__ int32_t s_slot[2][kWaves][kMaxR];
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);
    const int64_t P = a.rank_off[a.R];
    const bool cap_ok = P <= a.cap;
    if (blockIdx.x == 0 && wave == 0) {
        if (!cap_ok && lane == 0) set_error(a.st, EP_ERR_CAPACITY);
        if (PUB != kPubNone) refresh_tail_cache(a);
    }
    // stream publication runs when the ring exists and the rows fit; every
    // wavefront hands its slots over after each group, but wavefront 0
    // publishes only if no error (e.g. a bad expert id found by the layout)
    // was reported before the kernel started -- then no command goes out,
    // as in the closed form
    const bool streaming = PUB == kPubStream && cap_ok;
    bool pub_ok = false;   // wavefront 0 only
    if (streaming && wave == 0) pub_ok = bcast(read_status(a.st), 0) == 0;
    __shared__ RankView rv;   // read by wavefront 0 only, which wrote it
    if (streaming && wave == 0) load_rank_view(a, rv);
    if (pub_ok && blockIdx.x == 0) publish_empty_ranks(a, rv);
    // groups of kWaves wavefronts, taken in launch order; a workgroup that
    // finishes a group (rows, then descriptors) moves on to the next one
    int pass = 0;
    for (int64_t grp = blockIdx.x; grp < a.ngroups; grp += gridDim.x, pass ^= 1) {
    const int64_t gw = grp * kWaves + wave;
    const int64_t t = gw / a.nchunks;
    const int chunk = (int)(gw - t * a.nchunks);
    const bool active = t < a.T;   // wavefront-uniform

    int32_t s_lane = -1;
    uint64_t dmask = 0;
    if (active) {
        // fp8 rows: the chunk's loads go out before the slot entry's (one
        // memory latency for both; fp8 step 170.1 -> 169.0 us in alternating
        // runs).  bf16 rows keep the order below (skewed was 3 us slower).
        u32x4 v[VPL];
        if (FMT != EP_FMT_BF16) prefetch_row_chunk<VPL>(a, t, chunk, v);
        if (lane < a.R) s_lane = a.send_slot[t * a.R + lane];
        dmask = __ballot(s_lane >= 0);
        if (PUB == kPubClosed && s_lane >= 0 && (s_lane < a.rank_off[lane] || s_lane >= a.rank_off[lane + 1]))
            set_error(a.st, EP_ERR_INVALID_ARG);   // send_slot not from this rank_offset

        if (FMT != EP_FMT_BF16)
            store_row_chunk_v<VPL, FMT>(a, chunk, s_lane, dmask, v);
        else
            store_row_chunk<VPL, FMT>(a, t, chunk, s_lane, dmask);

        // per-slot metadata, written by the token's first chunk
        if (chunk == 0) store_slot_metadata(a, t, s_lane, dmask);
    }

    if (!streaming) continue;   // uniform over the workgroup
    // hand this wavefront's slots (rank r on lane r) to wavefront 0
    if (lane < a.R) s_slot[pass][wave][lane] = s_lane;
    // The rows went out with system-scope stores: once complete they are
    // visible to every agent, so no write-back precedes the arrivals.
    wait_vm();
    __syncthreads();
    if (wave == 0 && pub_ok) {
        // The arrivals and the descriptors of the group.  Meanwhile the
        // other wavefronts go on with the next group, whose slots go to the
        // other buffer; this one is written again only after the next
        // barrier, which wavefront 0 reaches once it is done here.
        publish_group<kWaves>(a, rv, s_slot[pass]);
    }
    }

    if (PUB == kPubClosed) {
        // Once its system-scope row stores are complete, the workgroup
        // counts itself out; the last workgroup to finish then publishes
        // every command.
        __shared__ int s_last;
        __shared__ unsigned long long s_base[kMaxR];
        const ClosedOrder z = closed_order(a, a.rank_off);   // loads issued before the wait
        wait_vm();   // this wavefront's rows are complete
        __syncthreads();
        if (threadIdx.x == 0) {
            // publish only if no error was raised: then no ticket is taken
            s_last = arrive_last(a.arrive, kArriveFlatRank) && cap_ok && read_status(a.st) == 0;
        }
        __syncthreads();
        if (!s_last) return;
        __shared__ int32_t s_cstart[kMaxR], s_cnum[kMaxR];
        __shared__ unsigned long long s_seen[kMaxR];
        if (wave == 0) closed_reserve(a, z, s_base, s_seen, s_cstart, s_cnum);
        __syncthreads();
        closed_publish_all<kWaves * kWave>(a, z, s_base, s_seen, s_cstart, s_cnum);
    }
}

// ------------------------------------------------- one-kernel small batches
// Routing layout and pack of a batch of at most kFusedMaxT tokens in one
// launch (UCCL-EP article s4.1: the low-latency path is for small decode
// batches; its cost is latency, and a separate layout kernel is one more
// chain of memory round trips and one more launch).  The layout is tiny
// (T * k ids), so every workgroup computes all of it in LDS: wavefront w
// builds the rank masks of tokens 64w .. 64w + 63 and its per-rank ballots;
// the rank totals, offsets and every token's slots follow from the ballots.
// No workgroup waits for another before copying.  Workgroup 0 also writes
// the layout outputs that are not per token (counts, offsets, the expert
// histogram and its scan, the message bases); the first chunk of each token
// writes its send_slot and is_token_in_rank rows.  The rows, metadata and
// closed-form publication are those of the small-batch pack.
constexpr int kFusedMaxT = kPackWavesSmall * kWave;

template <int VPL, int FMT, int KMAX>
__global__ __launch_bounds__(kPackWavesSmall* kWave) void fused_small_kernel(PackArgs a) {
    constexpr int kWaves = kPackWavesSmall;
    static_assert(kWaves * kWave == kBlock, "the expert scan takes a kBlock-thread workgroup");
    __shared__ uint64_t s_ball[kWaves][kMaxR];   // bit i: token 64w + i goes to rank r
    __shared__ int32_t s_cnt[kWaves][kMaxR];     // tokens of wavefront w on rank r
    __shared__ int32_t s_wbase[kWaves][kMaxR];   // first slot of rank r for wavefront w's tokens
    __shared__ int32_t s_ro[kMaxR + 1];          // rank offsets
    __shared__ int32_t s_hist[kMaxE];            // expert histogram (workgroup 0)
    __shared__ int32_t s_part[kBlock];
    __shared__ int s_last;
    __shared__ unsigned long long s_base[kMaxR];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const bool first = blockIdx.x == 0;
    const int R = a.R;

    // this wavefront's chunk of its first group, loaded before the layout so
    // that the two memory latencies overlap
    u32x4 v[VPL];
    {
        const int64_t gw = (int64_t)blockIdx.x * kWaves + wave;
        const int64_t t = gw / a.nchunks;
        if (blockIdx.x < a.ngroups && t < a.T)
            prefetch_row_chunk<VPL>(a, t, (int)(gw - t * a.nchunks), v);
    }

    // layout, in every workgroup
    if (first)
        for (int e = tid; e < a.E; e += kBlock) s_hist[e] = 0;
    __syncthreads();
    const uint64_t mask = token_rank_mask<KMAX>(a.idx, (int64_t)wave * kWave + lane, a.T, a.E,
                                                a.k, a.epr, a.st, first ? s_hist : nullptr);
    wave_rank_counts(mask, R, s_cnt[wave], s_ball[wave]);
    __syncthreads();
    if (wave == 0) {
        int32_t tot = 0;
        if (lane < R)
            for (int w = 0; w < kWaves; ++w) tot += s_cnt[w][lane];
        const int32_t msgs = (tot + kMsgRows - 1) / kMsgRows;
        int32_t incl = tot, mincl = msgs;
        for (int d = 1; d < kWave; d <<= 1) {
            const int32_t o = __shfl_up(incl, d);
            const int32_t mo = __shfl_up(mincl, d);
            if (lane >= d) {
                incl += o;
                mincl += mo;
            }
        }
        const int32_t off = incl - tot;
        if (lane < R) {
            s_ro[lane] = off;
            int32_t run = off;
            for (int w = 0; w < kWaves; ++w) {
                s_wbase[w][lane] = run;
                run += s_cnt[w][lane];
            }
        }
        if (lane == R - 1) s_ro[R] = incl;
        if (first) {
            if (lane < R) {
                a.cnt_rank_out[lane] = tot;
                a.rank_off_out[lane] = off;
                a.msg_base_out[lane] = mincl - msgs;
            }
            if (lane == R - 1) {
                a.rank_off_out[R] = incl;
                a.msg_base_out[R] = mincl;
            }
        }
    }
    __syncthreads();

    // rows: wavefront g of the grid takes chunk g % nchunks of token g / nchunks
    const int64_t P = s_ro[R];
    const bool cap_ok = P <= a.cap;
    const bool refresh = first && wave == 0 && a.has_ring;   // wavefront-uniform
    unsigned long long tail_h = 0;
    if (first && wave == 0) {
        if (!cap_ok && lane == 0) set_error(a.st, EP_ERR_CAPACITY);
        if (refresh) tail_h = tail_read(a);
    }
    for (int64_t grp = blockIdx.x; grp < a.ngroups; grp += gridDim.x) {
        const int64_t gw = grp * kWaves + wave;
        const int64_t t = gw / a.nchunks;
        const int chunk = (int)(gw - t * a.nchunks);
        if (t >= a.T) continue;   // wavefront-uniform
        if (grp != blockIdx.x) prefetch_row_chunk<VPL>(a, t, chunk, v);
        const int tw = (int)(t / kWave), tl = (int)(t % kWave);
        int32_t s_lane = -1;
        uint32_t bit = 0;
        if (lane < R) {
            const uint64_t b = s_ball[tw][lane];
            bit = (uint32_t)((b >> tl) & 1ull);
            if (bit) s_lane = s_wbase[tw][lane] + (int32_t)__popcll(b & ((1ull << tl) - 1ull));
        }
        const uint64_t dmask = __ballot(s_lane >= 0);
        store_row_chunk_v<VPL, FMT>(a, chunk, s_lane, dmask, v);
        if (chunk == 0) {
            store_slot_metadata(a, t, s_lane, dmask);
            if (lane < R) {
                a.send_slot_out[t * R + lane] = s_lane;
                a.in_rank_out[t * R + lane] = (uint8_t)bit;
            }
        }
    }
    if (first) {
        // expert counts and offsets, while the rows' stores complete
        for (int e = tid; e < a.E; e += kBlock) a.cnt_exp_out[e] = s_hist[e];
        block_exclusive_scan_store(s_hist, a.E, a.exp_off_out, s_part);
        // the per-message counters of the streaming pack start at zero, as
        // after a layout call
        for (int64_t i = tid; i < a.counters_n; i += kBlock) a.msg_arrivals[i] = 0;
    }

    // closed-form publication by the last workgroup to finish its rows
    if (!a.has_ring) return;   // grid-uniform
    if (refresh) tail_apply(a, tail_h);
    const ClosedOrder z = closed_order(a, s_ro);
    wait_vm();   // this wavefront's rows are complete
    __syncthreads();
    if (tid == 0) s_last = arrive_last(a.arrive, kArriveFlatRank) && cap_ok && read_status(a.st) == 0;
    __syncthreads();
    if (!s_last) return;
    __shared__ int32_t s_cstart[kMaxR], s_cnum[kMaxR];
    __shared__ unsigned long long s_seen[kMaxR];
    if (wave == 0) closed_reserve(a, z, s_base, s_seen, s_cstart, s_cnum);
    __syncthreads();
    closed_publish_all<kWaves * kWave>(a, z, s_base, s_seen, s_cstart, s_cnum);
}

// ------------------------------------------------- one-kernel large batches
// Routing layout and pack of a large batch in one launch, for chunkings with
// one wavefront per token.  The pack's work order is kept (workgroup b takes
// groups b, b + G, ... of kWaves consecutive tokens, so messages complete all
// through the copy and publication overlaps it); only the layout moves into
// the kernel, split so that no workgroup does more than a few ballots:
//   1. for each of its groups, the workgroup takes the 64-token block the
//      group lies in and computes its per-rank ballots (one wavefront per
//      block); the block's first group also stores the block's rank counts
//      to a [ceil(T/64), R] table;
//   2. grid barrier (the G pack workgroups are resident at once);
//   3. every workgroup sums the table: the rank totals (hence the offsets,
//      identical everywhere) and, per group, the rows of each rank in the
//      blocks before the group's block; a token's slot is then
//        o_r + (rows of r in earlier blocks) + popcount(ballot_r below it);
//   4. the pack of the two-kernel path, reading slots from LDS; each token's
//      first wavefront also writes its send_slot and is_token_in_rank rows.
// Each wavefront loads its row chunk of pass 0 before the barrier, so the
// copy's first reads overlap the layout.
// The per-expert counts and their scan: when the pack's grid leaves room on
// the chip, one workgroup more computes them from topk_idx meanwhile (off the
// critical path; it takes no part in the barrier).  When the pack fills the
// chip, they come from the ballots' ids: the workgroup that takes a block's
// first group also counts the block's choices per expert in LDS and adds its
// non-zero counts, after the barrier, to one of a few partial histograms in
// the workspace (workgroup b to part b mod nparts, so that few workgroups add
// to one counter); the last workgroup to have added its counts sums the parts
// into the output and writes their exclusive scan.  The slots are those of
// the layout kernel: integer counts and prefix sums, no atomic decides an
// order.
constexpr int kFusedLargeMaxPasses = 16;
constexpr int kExpParts = 8;   // partial expert histograms, at most

// Per-expert counts of all T * k choices and their exclusive scan (one
// workgroup of NT >= kBlock threads).
template <int NT>
__device__ void expert_counts(const PackArgs& a, int32_t* s_hist, int32_t* s_part) {
    const int tid = threadIdx.x;
    for (int e = tid; e < a.E; e += NT) s_hist[e] = 0;
    __syncthreads();
    const int64_t n = (int64_t)a.T * a.k;
    constexpr int kBatch = 8;
    for (int64_t i0 = tid; i0 < n; i0 += (int64_t)NT * kBatch) {
        int32_t v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t i = i0 + (int64_t)u * NT;
            v[u] = i < n ? a.idx[i] : -1;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (v[u] >= 0 && v[u] < a.E) atomicAdd(&s_hist[v[u]], 1);
    }
    __syncthreads();
    for (int e = tid; e < a.E; e += NT) a.cnt_exp_out[e] = s_hist[e];
    block_exclusive_scan_store(s_hist, a.E, a.exp_off_out, s_part);
}

// After every workgroup's expert counts are added in (one wavefront of each
// workgroup, once its own atomics are complete): the last one to arrive sums
// the parts into num_tokens_per_expert (lane l takes experts l, l + 64, ...,
// so the loads of a part are coalesced, and a lane's loads of all parts are
// in flight together), keeps the totals in `tot` (LDS) and writes their
// exclusive scan (lane l taking a contiguous run of experts).
__device__ void expert_offsets_if_last(const PackArgs& a, int32_t* tot) {
    const int lane = lane_id();
    int last = 0;
    if (lane == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        last = arrive_last(a.arrive) ? 1 : 0;   // acquires every part's atomics
    }
    if (!bcast(last, 0)) return;
    const int E = a.E, np = a.nparts;
    for (int e = lane; e < E; e += kWave) {
        int32_t v[kExpParts];
#pragma unroll
        for (int q = 0; q < kExpParts; ++q) v[q] = q < np ? a.exp_part[(int64_t)q * E + e] : 0;
        int32_t c = 0;
#pragma unroll
        for (int q = 0; q < kExpParts; ++q) c += v[q];
        tot[e] = c;
        a.cnt_exp_out[e] = c;
    }
    const int per = (E + kWave - 1) / kWave;
    const int lo = lane * per, hi = min(lo + per, E);
    int32_t sum = 0;
    for (int e = lo; e < hi; ++e) sum += tot[e];
    int32_t incl = sum;
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    int32_t run = incl - sum;
    for (int e = lo; e < hi; ++e) {
        a.exp_off_out[e] = run;
        run += tot[e];
    }
    if (lane == kWave - 1) a.exp_off_out[E] = incl;
}

// The rows of one pass of the one-kernel large batch: this wavefront's
// token of group b + p*G (its row chunk in *v when already loaded), its
// slots from the block's ballots, its rows and metadata.  Returns the slot
// of rank `lane` (or -1).
template <int VPL, int FMT, int WAVES>
__device__ __forceinline__ int32_t fused_rows(const PackArgs& a, int p, int64_t b, int64_t G,
                                              const uint64_t (*s_ball)[kMaxR],
                                              const int32_t (*s_base)[kMaxR],
                                              const u32x4 (*v)[VPL]) {
    const int lane = lane_id(), wave = (int)(threadIdx.x / kWave), R = a.R;
    const int64_t t = (b + (int64_t)p * G) * WAVES + wave;
    int32_t s_lane = -1;
    if (t < a.T) {   // wavefront-uniform
        if (lane < R) {
            const uint64_t bb = s_ball[p][lane];
            const int tl = (int)(t % kWave);
            const bool in = (bb >> tl) & 1ull;
            if (in) s_lane = s_base[p][lane] + (int32_t)__popcll(bb & ((1ull << tl) - 1ull));
            a.send_slot_out[t * R + lane] = s_lane;
            a.in_rank_out[t * R + lane] = (uint8_t)in;
        }
        const uint64_t dmask = __ballot(s_lane >= 0);
        if (v) {
            store_row_chunk_v<VPL, FMT>(a, 0, s_lane, dmask, *v);
        } else {
            u32x4 w[VPL];
            prefetch_row_chunk<VPL>(a, t, 0, w);   // branch-free loads (fewer registers here)
            store_row_chunk_v<VPL, FMT>(a, 0, s_lane, dmask, w);
        }
        store_slot_metadata(a, t, s_lane, dmask);
    }
    return s_lane;
}

// One workgroup per CU: WAVES / 4 wavefronts per SIMD.  Built for k <= KMAX.
template <int VPL, int FMT, int WAVES, int PUB, int KMAX>
__global__ __launch_bounds__(WAVES * kWave, WAVES / 4) void fused_large_kernel(PackArgs a) {
    constexpr int kWaves = WAVES;
    constexpr int kT = WAVES * kWave;
    constexpr int kPass = kFusedLargeMaxPasses;
    static_assert(kWave % kWaves == 0, "a group lies inside one 64-token block");
    static_assert(kWaves >= 2, "wavefront 1 finishes the expert offsets");
    static_assert(kT >= kBlock, "the expert scan takes at least kBlock threads");
    __shared__ uint64_t s_ball[kPass][kMaxR];   // pass p: ballots of its group's block
    __shared__ int32_t s_base[kPass][kMaxR];    // pass p: slot of the block's first row of r
    __shared__ int32_t s_tot[kMaxR];            // rows of rank r
    __shared__ int32_t s_slot[2][kWaves][kMaxR];
    __shared__ RankView rv;
    __shared__ int32_t s_hist[kMaxE];           // choices per expert (this workgroup's blocks)
    __shared__ int32_t s_part[kT];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int R = a.R;
    const bool count_here = !a.expert_wg;         // uniform over the grid
    const int64_t G = (int64_t)gridDim.x - (count_here ? 0 : 1);   // pack workgroups
    const int64_t b = blockIdx.x;
    if (b == G) {
        expert_counts<kT>(a, s_hist, s_part);
        return;
    }
    if (count_here) {
        // cleared before any global load is in flight, so that this barrier
        // waits for nothing
        for (int e = tid; e < a.E; e += kT) s_hist[e] = 0;
        __syncthreads();
    }
    // 1. ballots of each pass's block (wavefront p % kWaves takes pass p).
    // Only the ids are loaded before them: a wavefront's memory counter
    // retires in order, so anything issued earlier would hold them up.
    int32_t ids[KMAX];
    if (wave < a.npass && b + (int64_t)wave * G < a.ngroups)
        load_token_ids(a.idx, (b + (int64_t)wave * G) * kWaves / kWave * kWave + lane, a.T, a.k,
                       ids);
    for (int p = wave; p < a.npass; p += kWaves) {
        const int64_t g = b + (int64_t)p * G;
        uint64_t mine = 0;
        if (g < a.ngroups) {
            const int64_t blk = g * kWaves / kWave;
            if (p != wave) load_token_ids(a.idx, blk * kWave + lane, a.T, a.k, ids);
            // the block's first group is taken exactly once: it also counts
            // the block's choices per expert
            const bool first = (g * kWaves) % kWave == 0;
            const uint64_t mask =
                rank_mask_of(ids, a.E, a.k, a.epr, a.st, (first && count_here) ? s_hist : nullptr);
            mine = wave_bit_transpose(mask);   // lane r < R: the ballot of rank r; others 0
            if (first && lane < R) a.wave_cnt[blk * R + lane] = (int32_t)__popcll(mine);
        }
        if (lane < R) s_ball[p][lane] = mine;
    }
    // This wavefront's row chunk of pass 0 (about 29 MB over the grid at
    // H = 7168), which stays in registers through the barrier and the table
    // read: its latency overlaps them.  Issued before the ballots it held
    // them up until it had arrived; here only the barrier's own wait for the
    // workgroup's memory operations includes it (train, median: ballots done
    // 8.2 -> 6.8 us, barrier left 13.5 -> 12.9 us after the first start).
    u32x4 v0[VPL];
    const int64_t t0 = b * kWaves + wave;   // this wavefront's token in pass 0
    if (t0 < a.T) prefetch_row_chunk<VPL>(a, t0, 0, v0);
    uint32_t gen = 0;   // the barrier's generation
    if (tid == 0) gen = grid_barrier_generation(a.bar);
    for (int p = tid; p < kPass * kMaxR; p += kT) (&s_base[0][0])[p] = 0;
    if (tid < kMaxR) s_tot[tid] = 0;
    // the streaming pack's message counters and the partial expert counts
    // (added to after the barrier) start at zero
    for (int64_t i = b * kT + tid; i < a.counters_n; i += G * kT) a.msg_arrivals[i] = 0;
    if (count_here)
        for (int64_t i = b * kT + tid; i < (int64_t)a.nparts * a.E; i += G * kT) a.exp_part[i] = 0;

    // 2. every block's counts are in the table after this
    if (!grid_barrier<false>(a.bar, (uint32_t)G, a.st, gen)) return;

    // 3. rank totals and, per pass, the rows in earlier blocks.  Thread
    // (seg, r) walks rows [lo, hi) of column r in order; pass p, whose group
    // lies in block f_p (ascending in p), takes the rows of the range below
    // f_p: the running sum when the walk reaches f_p, the whole range when
    // f_p >= hi.
    {
        const int nseg = kT / R;
        const int r = tid % R, seg = tid / R;
        const int32_t nblk = (a.T + kWave - 1) / kWave;
        const int32_t len = (nblk + nseg - 1) / nseg;
        const int32_t lo = seg * len, hi = min(lo + len, nblk);
        auto first_blk = [&](int p) {
            return (int32_t)((b + (int64_t)p * G) * kWaves / kWave);
        };
        if (seg < nseg) {
            int32_t run = 0;
            int p = 0;
            while (p < a.npass && first_blk(p) <= lo) ++p;   // nothing of this range
            constexpr int kBatch = 8;
            for (int32_t k0 = lo; k0 < hi; k0 += kBatch) {
                int32_t v[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
                    v[u] = k0 + u < hi ? a.wave_cnt[(int64_t)(k0 + u) * R + r] : 0;
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    while (p < a.npass && first_blk(p) <= k0 + u) {
                        if (run) atomicAdd(&s_base[p][r], run);
                        ++p;
                    }
                    run += v[u];
                }
            }
            for (; p < a.npass; ++p)
                if (run) atomicAdd(&s_base[p][r], run);
            atomicAdd(&s_tot[r], run);
        }
    }
    __syncthreads();
    if (wave == 0) {
        // offsets and message bases (exclusive scans across lanes, R <= 64)
        const int32_t tot = lane < R ? s_tot[lane] : 0;
        const int32_t msgs = (tot + kMsgRows - 1) / kMsgRows;
        int32_t incl = tot, mincl = msgs;
        for (int d = 1; d < kWave; d <<= 1) {
            const int32_t o = __shfl_up(incl, d);
            const int32_t mo = __shfl_up(mincl, d);
            if (lane >= d) {
                incl += o;
                mincl += mo;
            }
        }
        const int32_t off = incl - tot;
        if (lane < R) {
            rv.o[lane] = off;
            rv.cnt[lane] = tot;
            rv.mbase[lane] = mincl - msgs;
            for (int p = 0; p < a.npass; ++p) s_base[p][lane] += off;
        }
        if (b == 0) {
            if (lane < R) {
                a.cnt_rank_out[lane] = tot;
                a.rank_off_out[lane] = off;
                a.msg_base_out[lane] = mincl - msgs;
            }
            if (lane == R - 1) {
                a.rank_off_out[R] = incl;
                a.msg_base_out[R] = mincl;
            }
        }
        if (lane == R - 1) s_tot[0] = incl;   // P, read after the barrier below
    }
    __syncthreads();

    // 4. the pack
    const int64_t P = s_tot[0];
    const bool cap_ok = P <= a.cap;
    if (b == 0 && wave == 0) {
        if (!cap_ok && lane == 0) set_error(a.st, EP_ERR_CAPACITY);
        if (PUB != kPubNone) refresh_tail_cache(a);
    }
    // as in the two-kernel pack: no command goes out once an error (e.g. a
    // bad expert id found in step 1) has been reported
    const bool streaming = PUB == kPubStream && cap_ok;
    bool pub_ok = false;   // wavefront 0 only
    if (streaming && wave == 0) pub_ok = bcast(read_status(a.st), 0) == 0;
    if (pub_ok && b == 0) publish_empty_ranks(a, rv);
    // pass 0's rows come from the registers loaded before the barrier; every
    // pack workgroup has a pass 0 (b < G <= ngroups)
    int32_t s_lane = fused_rows<VPL, FMT, kWaves>(a, 0, b, G, s_ball, s_base, &v0);
    // this workgroup's expert counts, into its part (cleared before the
    // barrier), behind pass 0's row stores: nothing waits for them before
    // the group's own wait for its rows, and the table reads of step 3 did
    // not queue behind them
    if (count_here) {
        int32_t* part = a.exp_part + (b % a.nparts) * (int64_t)a.E;
        for (int e = tid; e < a.E; e += kT) {
            const int32_t h = s_hist[e];
            if (h) atomicAdd(&part[e], h);
        }
    }
    for (int p = 0;;) {
        if (streaming) {   // uniform over the workgroup
            if (lane < R) s_slot[p & 1][wave][lane] = s_lane;
            wait_vm();   // also this wavefront's expert-count atomics
            __syncthreads();
            if (wave == 0 && pub_ok) publish_group<kWaves>(a, rv, s_slot[p & 1]);
        }
        if (++p >= a.npass || b + (int64_t)p * G >= a.ngroups) break;
        s_lane = fused_rows<VPL, FMT, kWaves>(a, p, b, G, s_ball, s_base, nullptr);
    }
    // The expert counts' arrival, after the last group: wavefront 1 has no
    // rows left while wavefront 0 publishes the last group, so the arrival
    // and the last workgroup's sums run in that shadow.
    if (!count_here) return;
    if (!streaming) {   // uniform over the grid
        wait_vm();
        __syncthreads();
    }
    // its expert-count atomics are complete; s_hist is read no more
    if (wave == 1) expert_offsets_if_last(a, s_hist);
}

// ------------------------------------------------------------ per-expert mode
// Commands of the per-expert stream in closed form, by the whole last
// workgroup.  Per channel c: its ranks r = c, c + C, ... ascending, each
// rank's experts ascending, per expert the WRITEs of its <= 8-row messages
// and then its ATOMIC (value cnt_e, dst_offset 4 * local expert).  Experts
// are numbered in that order (o = position of the rank * epr + local index);
// an LDS scan of their command counts gives every command its place.
__device__ inline int ll_rank_at(int rp, int C, int q, int rem) {
    int c, i;
    if (rp < rem * (q + 1)) {
        c = rp / (q + 1);
        i = rp % (q + 1);
    } else {
        const int l2 = rp - rem * (q + 1);
        c = rem + l2 / q;
        i = l2 % q;
    }
    return c + i * C;
}

__device__ inline int ll_first_pos(int c, int q, int rem) {   // first rank position of channel c
    return c < rem ? c * (q + 1) : rem * (q + 1) + (c - rem) * q;
}

template <int WAVES>
__device__ void ll_closed_publish(const PackArgs& a, const int32_t* exp_off) {
    __shared__ int32_t s_start[kMaxE + 1];
    __shared__ int32_t s_eo[kMaxE + 1];   // expert_offset, staged once
    __shared__ int32_t s_wsum[WAVES];
    __shared__ unsigned long long s_cbase[kMaxR];
    constexpr int kT = WAVES * kWave;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int E = a.E, R = a.R, C = a.ring.channels, epr = a.epr;
    const int q = R / C, rem = R % C;
    for (int e = tid; e <= E; e += kT) s_eo[e] = exp_off[e];
    __syncthreads();
    // commands per expert, in stream order, scanned: thread tid sums a run
    const int per = (E + kT - 1) / kT;
    const int o0 = tid * per;
    int32_t sum = 0;
    for (int i = 0; i < per; ++i) {
        const int o = o0 + i;
        if (o < E) {
            const int e = ll_rank_at(o / epr, C, q, rem) * epr + o % epr;
            const int32_t cnt = s_eo[e + 1] - s_eo[e];
            s_start[o] = (cnt + kMsgRows - 1) / kMsgRows + 1;
            sum += s_start[o];
        }
    }
    int32_t incl = sum;
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
    }
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    int32_t run = incl - sum;
    for (int w = 0; w < wave; ++w) run += s_wsum[w];
    for (int i = 0; i < per; ++i) {
        const int o = o0 + i;
        if (o < E) {
            const int32_t n = s_start[o];
            s_start[o] = run;
            run += n;
        }
    }
    if (tid == kT - 1) s_start[E] = run;
    __syncthreads();
    const int32_t total = s_start[E];
    // one reservation per channel for its whole stream
    const int nch = C < R ? C : R;
    if (tid < nch) {
        const int32_t f = s_start[ll_first_pos(tid, q, rem) * epr];
        const int32_t l = tid + 1 < nch ? s_start[ll_first_pos(tid + 1, q, rem) * epr] : total;
        s_cbase[tid] = ring_reserve(a.ring, tid, (unsigned)(l - f));
    }
    __syncthreads();
    const uint64_t rb = (uint64_t)a.row_bytes;
    // the channels advance together (as in closed_publish_all): in each
    // round thread i takes channel i % nch and that channel's next command
    const int per_round = kT / nch;
    const int ch = tid % nch;
    const int32_t jt = tid / nch;
    const int32_t cfirst = s_start[ll_first_pos(ch, q, rem) * epr];
    const int32_t cnum = (ch + 1 < nch ? s_start[ll_first_pos(ch + 1, q, rem) * epr] : total) - cfirst;
    int32_t nmax = 0;
    for (int c2 = 0; c2 < nch; ++c2) {
        const int32_t f = s_start[ll_first_pos(c2, q, rem) * epr];
        const int32_t l = c2 + 1 < nch ? s_start[ll_first_pos(c2 + 1, q, rem) * epr] : total;
        nmax = l - f > nmax ? l - f : nmax;
    }
    for (int32_t j0 = 0; j0 < nmax; j0 += per_round) {
        const bool have = jt < per_round && j0 + jt < cnum;
        const int32_t g = have ? cfirst + j0 + jt : 0;
        // the expert (stream position o) that command g belongs to
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_start[mid] <= g) lo = mid;
            else hi = mid - 1;
        }
        const int o = lo;
        const int r = ll_rank_at(o / epr, C, q, rem);
        const int le = o % epr;
        const int e = r * epr + le;
        const int c = r % C;
        const int32_t eo = s_eo[e];
        const int32_t cnt = s_eo[e + 1] - eo;
        const int32_t nmsg = (cnt + kMsgRows - 1) / kMsgRows;
        const int32_t local = g - s_start[o];
        const bool write = local < nmsg;
        const int32_t rows = write ? min(kMsgRows, cnt - local * kMsgRows) : 0;
        const int32_t rbase = s_eo[r * epr];
        const unsigned long long ticket =
            have ? s_cbase[c] + (unsigned long long)(g - s_start[ll_first_pos(c, q, rem) * epr]) : 0;
        ring_publish<false>(a.ring, have, c, ticket, write ? EP_CMD_WRITE : EP_CMD_ATOMIC,
                            write ? 0 : EP_ATOMIC_ADD, (uint32_t)rows, (uint32_t)r,
                            write ? (uint32_t)(rows * rb) : (uint32_t)cnt,
                            write ? (uint64_t)(eo + local * kMsgRows) * rb : 0,
                            write ? (uint64_t)(eo - rbase + local * kMsgRows) * rb
                                  : (uint64_t)(4 * le),
                            a.st);
    }
}

// Per-expert streaming publication (large batches): as in the rank pack,
// each message -- the <= 8 consecutive rows [eo_e + 8m, ...) of expert e --
// is published by the arrival that completes it, and the expert's ATOMIC by
// the wavefront whose WRITE completes the expert's message count, with a
// ticket taken after every WRITE ticket of the expert.  Wavefront 0 of each
// workgroup stages the expert offsets and the experts' first message indices
// in LDS once per launch.
__device__ void ll_stage_experts(const PackArgs& a, int32_t* eo, int32_t* mb) {
    const int lane = lane_id(), E = a.E;
    for (int e = lane; e <= E; e += kWave) eo[e] = a.exp_off[e];
    // messages per expert, then their exclusive scan (lane l sums a run)
    const int per = (E + kWave - 1) / kWave;
    const int e0 = lane * per;
    int32_t sum = 0;
    for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        if (e < E) sum += (eo[e + 1] - eo[e] + kMsgRows - 1) / kMsgRows;
    }
    int32_t incl = sum;
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
    }
    int32_t run = incl - sum;
    for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        if (e < E) {
            mb[e] = run;
            run += (eo[e + 1] - eo[e] + kMsgRows - 1) / kMsgRows;
        }
    }
    if (lane == kWave - 1) mb[E] = incl;
}

// ATOMIC{ADD, 0} of every expert with no rows (nothing to order after), by
// wavefront 0 of one workgroup, 64 experts a round.
__device__ void ll_publish_empty(const PackArgs& a, const int32_t* eo) {
    const int lane = lane_id();
    for (int e0 = 0; e0 < a.E; e0 += kWave) {
        const int e = e0 + lane;
        int n = 0, c = 0;
        unsigned long long tk = 0;
        RingCmd cmd{};
        if (e < a.E && eo[e + 1] == eo[e]) {
            const int r = e / a.epr;
            c = r % a.ring.channels;
            tk = ring_reserve(a.ring, c, 1);
            cmd = RingCmd{EP_CMD_ATOMIC, EP_ATOMIC_ADD, 0, (uint32_t)r, 0, 0,
                          (uint64_t)(4 * (e - r * a.epr))};
            n = 1;
        }
        ring_publish_v<1>(a.ring, n ? 1u : 0u, &c, &tk, &cmd, a.st);
    }
}

// Wavefront 0, after the rows of its group are released: row[w][j] and
// ex[w][j] are the row and expert of wavefront w's choice j (-1 for none).
// The W * k pairs go in rounds of 128, two per lane; a pair adds one arrival
// (one chunk of one row) to its message.  Within a round every step is
// issued for both of a lane's pairs at once: one round trip each for the
// arrivals (with the status word and the channels' cached consumer
// positions), the WRITE tickets, the experts' message counts and the ATOMIC
// tickets.  The WRITE slots go out while the message counts are on their
// way back, so a WRITE ticket stays unwritten for one round trip only (the
// proxy pops in ticket order: an unwritten ticket holds up its channel).  A
// round's tickets are all written before the next round takes any.
template <int W>
__device__ void ll_publish_group(const PackArgs& a, const int32_t* eo, const int32_t* mb,
                                 const int32_t (*row)[kMaxK], const int32_t (*ex)[kMaxK]) {
    constexpr int P = 2;
    const int lane = lane_id();
    const int k = a.k, C = a.ring.channels;
    const int npairs = W * k;
    // an inconsistent group is reported before it counts any row or takes
    // any ticket
    bool bad = false;
    for (int f = lane; f < npairs; f += kWave) {
        const int sf = row[f / k][f % k], ef = ex[f / k][f % k];
        if (sf >= 0 && (ef < 0 || ef >= a.E || sf < eo[ef] || sf >= eo[ef + 1] ||
                        mb[ef] + (sf - eo[ef]) / kMsgRows >= a.max_msgs))
            bad = true;   // expert_slot not from this expert_offset, or the message table too small
    }
    if (__ballot(bad)) {
        if (bad) set_error(a.st, EP_ERR_INVALID_ARG);
        return;
    }
    const uint64_t rb = (uint64_t)a.row_bytes;
    for (int f0 = 0; f0 < npairs; f0 += P * kWave) {
        int32_t s[P], e[P];
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int f = f0 + lane + i * kWave;
            s[i] = f < npairs ? row[f / k][f % k] : -1;
            e[i] = f < npairs ? ex[f / k][f % k] : -1;
        }
        // arrivals, with the status word and the channels' cached positions
        const int32_t st0 = read_status(a.st);
        unsigned long long sn[P];
#pragma unroll
        for (int i = 0; i < P; ++i)
            sn[i] = s[i] >= 0 ? __hip_atomic_load(a.ring.tail_cache + (size_t)((e[i] / a.epr) % C) * kPad,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                              : 0ull;
        int32_t old[P];
#pragma unroll
        for (int i = 0; i < P; ++i)
            old[i] = s[i] >= 0
                         ? atomicAdd(&a.msg_arrivals[mb[e[i]] + (s[i] - eo[e[i]]) / kMsgRows], 1)
                         : 0;
        uint32_t done = 0;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            if (s[i] < 0) continue;
            const int32_t m = (s[i] - eo[e[i]]) / kMsgRows;
            const int32_t nrows = min(kMsgRows, eo[e[i] + 1] - eo[e[i]] - m * kMsgRows);
            if (old[i] + 1 == nrows * a.nchunks) {
                a.msg_arrivals[mb[e[i]] + m] = 0;   // every arrival is in: leave it clean
                if (st0 == 0) done |= 1u << i;
            }
        }
        if (!__ballot(done != 0)) continue;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        // WRITE tickets; once they exist the experts' message counts go out,
        // and the WRITE slots are written while the counts return.  An
        // expert's last message then takes the ATOMIC's ticket after every
        // WRITE ticket of the expert.
        int c[P];
        unsigned long long tk[P], ta[P];
        RingCmd cmd[P], cma[P];
#pragma unroll
        for (int i = 0; i < P; ++i) {
            c[i] = 0;
            tk[i] = ta[i] = 0;
            cmd[i] = cma[i] = RingCmd{};
            if (!((done >> i) & 1u)) continue;
            const int r = e[i] / a.epr;
            const int32_t eo_e = eo[e[i]];
            const int32_t m = (s[i] - eo_e) / kMsgRows;
            const int32_t nrows = min(kMsgRows, eo[e[i] + 1] - eo_e - m * kMsgRows);
            c[i] = r % C;
            tk[i] = ring_reserve(a.ring, c[i], 1);
            cmd[i] = RingCmd{EP_CMD_WRITE, 0, (uint32_t)nrows, (uint32_t)r, (uint32_t)(nrows * rb),
                             (uint64_t)(eo_e + m * kMsgRows) * rb,
                             (uint64_t)(eo_e - eo[r * a.epr] + m * kMsgRows) * rb};
        }
        int32_t dn[P];
#pragma unroll
        for (int i = 0; i < P; ++i)
            dn[i] = ((done >> i) & 1u) ? atomicAdd(&a.msgs_done[e[i]], 1 + (int32_t)(tk[i] >> 62))
                                       : 0;
        ring_publish_v<P>(a.ring, done, c, tk, cmd, a.st, sn);
        uint32_t have = 0;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            if (!((done >> i) & 1u)) continue;
            const int32_t cnt = eo[e[i] + 1] - eo[e[i]];
            if (dn[i] + 1 == (cnt + kMsgRows - 1) / kMsgRows) {
                a.msgs_done[e[i]] = 0;
                const int r = e[i] / a.epr;
                ta[i] = ring_reserve(a.ring, c[i], 1);
                cma[i] = RingCmd{EP_CMD_ATOMIC, EP_ATOMIC_ADD, 0, (uint32_t)r, (uint32_t)cnt,
                                 0, (uint64_t)(4 * (e[i] - r * a.epr))};
                have |= 1u << i;
            }
        }
        ring_publish_v<P>(a.ring, have, c, ta, cma, a.st);
    }
}

// Per-expert pack: wavefront g takes chunk g % nchunks of token g / nchunks
// and stores it to the row of every kept choice of the token (no dedup by
// rank: a token naming an expert twice sends two rows); the token's first
// chunk also writes each row's source token and gate.  With a ring, large
// batches publish as messages complete (ll_publish_group); small ones in
// closed form, by the last workgroup to finish.
template <int VPL, int FMT, int WAVES, int PUB>
__global__ __launch_bounds__(WAVES * kWave) void ll_pack_kernel(PackArgs a) {
    constexpr bool STREAM = PUB == kPubStream;
    // streaming: the group's rows and experts, per wavefront and choice, two
    // buffers by pass parity; the staged expert offsets and message bases
    __shared__ int32_t s_row[STREAM ? 2 : 1][STREAM ? WAVES : 1][kMaxK];
    __shared__ int32_t s_ex[STREAM ? 2 : 1][STREAM ? WAVES : 1][kMaxK];
    __shared__ int32_t s_eo[STREAM ? kMaxE + 1 : 1];
    __shared__ int32_t s_mb[STREAM ? kMaxE + 1 : 1];
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);
    const int64_t Q = a.exp_off[a.E];
    const bool cap_ok = Q <= a.cap;
    if (blockIdx.x == 0 && wave == 0) {
        if (!cap_ok && lane == 0) set_error(a.st, EP_ERR_CAPACITY);
        if (PUB != kPubNone) refresh_tail_cache(a);
    }
    // streaming publication runs when the ring exists and the rows fit;
    // wavefront 0 publishes only if no error was reported before the kernel
    // started (then no command goes out)
    const bool streaming = STREAM && cap_ok;
    bool pub_ok = false;   // wavefront 0 only
    if (streaming && wave == 0) {
        pub_ok = bcast(read_status(a.st), 0) == 0;
        ll_stage_experts(a, s_eo, s_mb);
        if (pub_ok && blockIdx.x == 0) ll_publish_empty(a, s_eo);
    }
    int pass = 0;
    for (int64_t grp = blockIdx.x; grp < a.ngroups; grp += gridDim.x, pass ^= 1) {
        const int64_t gw = grp * WAVES + wave;
        const int64_t t = gw / a.nchunks;
        const int chunk = (int)(gw - t * a.nchunks);
        int32_t s_lane = -1, e_lane = -1;
        if (t < a.T) {   // wavefront-uniform
            // bf16 rows: the chunk's loads go out first, so their latency
            // overlaps the two dependent rounds of routing loads below
            // (per-expert skewed step 924 -> 887 us in alternating runs).
            // fp8 rows keep the loads after them (9 us slower otherwise).
            u32x4 v[VPL];
            if (FMT == EP_FMT_BF16) prefetch_row_chunk<VPL>(a, t, chunk, v);
            float w_lane = 0.0f;
            if (lane < a.k) {
                const int e = a.idx[t * a.k + lane];
                if (e >= 0 && e < a.E) {
                    s_lane = a.expert_slot[t * a.k + lane];
                    e_lane = e;
                    w_lane = a.w[t * a.k + lane];
                    if (s_lane < a.exp_off[e] || s_lane >= a.exp_off[e + 1])
                        set_error(a.st, EP_ERR_INVALID_ARG);   // expert_slot not from this layout
                }
            }
            const uint64_t dmask = __ballot(s_lane >= 0);
            if (FMT == EP_FMT_BF16)
                store_row_chunk_v<VPL, FMT>(a, chunk, s_lane, dmask, v);
            else
                store_row_chunk<VPL, FMT>(a, t, chunk, s_lane, dmask);
            if (chunk == 0 && s_lane >= 0 && s_lane < a.cap) {
                a.slot_src[s_lane] = (int32_t)t;
                a.slot_w[s_lane] = w_lane;
            }
        }
        if (!streaming) continue;   // uniform over the workgroup
        if (lane < kMaxK) {
            s_row[pass][wave][lane] = s_lane;
            s_ex[pass][wave][lane] = e_lane;
        }
        // rows went out with system-scope stores: complete means visible
        wait_vm();
        __syncthreads();
        if (wave == 0 && pub_ok) ll_publish_group<WAVES>(a, s_eo, s_mb, s_row[pass], s_ex[pass]);
    }
    if (PUB == kPubClosed) {
        __shared__ int s_last;
        wait_vm();   // this wavefront's rows are complete (system-scope stores)
        __syncthreads();
        if (threadIdx.x == 0)
            s_last = arrive_last(a.arrive) && cap_ok && read_status(a.st) == 0;
        __syncthreads();
        if (!s_last) return;
        ll_closed_publish<WAVES>(a, a.exp_off);
    }
}

// ---------------------------------------- one-kernel per-expert small batches
// Per-expert layout, row table and pack of a batch of at most kFusedMaxT
// tokens with at most kLLFusedMaxE experts in one launch (UCCL-EP article
// s4.1: the low-latency mode serves small decode batches, where the chain of
// kernels and memory round trips is the cost).  Every workgroup derives the
// whole row table in LDS: wavefront w takes tokens 64w .. 64w + 63; for each
// round o (the o-th occurrence of an expert within a token, for repeats) its
// lanes set their bit in a per-wavefront mask per expert, a choice's place
// among the wavefront's earlier choices of its expert is the popcount of the
// mask below the lane, and the masks' popcounts are the wavefront's counts.
// The expert offsets are the scan of the totals; a wavefront's base for
// expert e is the offset plus the counts of the lower wavefronts.  No
// workgroup waits for another before copying.  Workgroup 0 writes the counts
// and offsets; the first chunk of each token writes its expert_slot row.  The
// last workgroup to finish its rows publishes in closed form.
constexpr int kLLFusedMaxE = 1024;

// KMAX: the bound on k the kernel is built for (8, or the library's bound);
// the loops over a token's choices run to it.
template <int VPL, int FMT, int KMAX>
__global__ __launch_bounds__(kPackWavesSmall* kWave) void ll_fused_small_kernel(PackArgs a) {
    constexpr int kWaves = kPackWavesSmall;
    constexpr int kT = kWaves * kWave;
    static_assert(kT == kBlock, "the expert scan takes a kBlock-thread workgroup");
    __shared__ int32_t s_cnt[kWaves][kLLFusedMaxE];              // counts, then bases
    __shared__ unsigned long long s_mask[kWaves][kLLFusedMaxE];  // one round's lanes per expert
    __shared__ int32_t s_eo[kLLFusedMaxE + 1];                   // expert offsets
    __shared__ int32_t s_tot[kLLFusedMaxE];
    __shared__ int32_t s_row[kFusedMaxT][KMAX];                 // row of choice (t, j), or -1
    __shared__ int32_t s_part[kBlock];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const bool first = blockIdx.x == 0;
    const int E = a.E, k = a.k;

    // this wavefront's chunk of its first group, loaded before the layout
    u32x4 v[VPL];
    {
        const int64_t gw = (int64_t)blockIdx.x * kWaves + wave;
        const int64_t t = gw / a.nchunks;
        if (blockIdx.x < a.ngroups && t < a.T)
            prefetch_row_chunk<VPL>(a, t, (int)(gw - t * a.nchunks), v);
    }

    // the lane's token and its choices
    const int64_t t = (int64_t)wave * kWave + lane;
    int32_t ids[KMAX];
    const int32_t* row = a.idx + t * k;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) ids[j] = (j < k && t < a.T) ? row[j] : -1;
    // s_cnt[wave] and s_mask[wave] are this wavefront's own LDS rows: it
    // clears them and runs its rounds alone, the steps ordered by
    // wavefront fences (a wavefront's LDS operations complete in order)
    for (int e = lane; e < E; e += kWave) {
        s_cnt[wave][e] = 0;
        s_mask[wave][e] = 0ull;
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
        if (ids[j] < -1 || ids[j] >= E) {
            set_error(a.st, EP_ERR_BAD_EXPERT);
            ids[j] = -1;
        }
    int32_t occ[KMAX];
    int my_rounds = 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        int o = 0;
#pragma unroll
        for (int i = 0; i < j; ++i) o += (ids[i] == ids[j]) ? 1 : 0;
        occ[j] = o;
        if (ids[j] >= 0 && o + 1 > my_rounds) my_rounds = o + 1;
    }
    int rounds = my_rounds;   // the wavefront's maximum
    for (int d = 1; d < kWave; d <<= 1) rounds = max(rounds, __shfl_xor(rounds, d));
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const unsigned long long below = (1ull << lane) - 1ull;
    int32_t pos[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) pos[j] = occ[j];
    for (int o = 0; o < rounds; ++o) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (ids[j] >= 0 && occ[j] == o) atomicOr(&s_mask[wave][ids[j]], 1ull << lane);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (ids[j] >= 0) pos[j] += __popcll(s_mask[wave][ids[j]] & below);
        for (int e = lane; e < E; e += kWave) s_cnt[wave][e] += __popcll(s_mask[wave][e]);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        for (int e = lane; e < E; e += kWave) s_mask[wave][e] = 0ull;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();   // every wavefront's counts
    // totals, per-wavefront bases, offsets
    for (int e = tid; e < E; e += kT) {
        int32_t run = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int32_t c = s_cnt[w][e];
            s_cnt[w][e] = run;
            run += c;
        }
        s_tot[e] = run;
    }
    __syncthreads();
    {
        // exclusive scan of the totals into s_eo (all kT threads)
        const int per = (E + kT - 1) / kT;
        const int b0 = tid * per;
        int32_t sum = 0;
        for (int i = 0; i < per; ++i)
            if (b0 + i < E) sum += s_tot[b0 + i];
        int32_t incl = sum;
        for (int d = 1; d < kWave; d <<= 1) {
            const int32_t o = __shfl_up(incl, d);
            if (lane >= d) incl += o;
        }
        if (lane == kWave - 1) s_part[wave] = incl;
        __syncthreads();
        int32_t run = incl - sum;
        for (int w = 0; w < wave; ++w) run += s_part[w];
        if (tid == kT - 1) s_eo[E] = run + sum;
        for (int i = 0; i < per; ++i)
            if (b0 + i < E) {
                s_eo[b0 + i] = run;
                run += s_tot[b0 + i];
            }
    }
    __syncthreads();
    if (t < a.T) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (j < k) s_row[t][j] = ids[j] >= 0 ? s_eo[ids[j]] + s_cnt[wave][ids[j]] + pos[j] : -1;
    }
    __syncthreads();

    // rows: wavefront g of the grid takes chunk g % nchunks of token g / nchunks
    const int64_t Q = s_eo[E];
    const bool cap_ok = Q <= a.cap;
    const bool refresh = first && wave == 0 && a.has_ring;   // wavefront-uniform
    unsigned long long tail_h = 0;
    if (first && wave == 0) {
        if (!cap_ok && lane == 0) set_error(a.st, EP_ERR_CAPACITY);
        if (refresh) tail_h = tail_read(a);
    }
    for (int64_t grp = blockIdx.x; grp < a.ngroups; grp += gridDim.x) {
        const int64_t gw = grp * kWaves + wave;
        const int64_t tt = gw / a.nchunks;
        const int chunk = (int)(gw - tt * a.nchunks);
        if (tt >= a.T) continue;   // wavefront-uniform
        if (grp != blockIdx.x) prefetch_row_chunk<VPL>(a, tt, chunk, v);
        const int32_t s_lane = lane < k ? s_row[tt][lane] : -1;
        const uint64_t dmask = __ballot(s_lane >= 0);
        store_row_chunk_v<VPL, FMT>(a, chunk, s_lane, dmask, v);
        if (chunk == 0 && lane < k) {
            a.send_slot_out[tt * k + lane] = s_lane;
            if (s_lane >= 0 && s_lane < a.cap) {
                a.slot_src[s_lane] = (int32_t)tt;
                a.slot_w[s_lane] = a.w[tt * k + lane];
            }
        }
    }
    if (first) {
        // counts and offsets, while the rows' stores complete
        for (int e = tid; e < E; e += kT) a.cnt_exp_out[e] = s_tot[e];
        for (int e = tid; e <= E; e += kT) a.exp_off_out[e] = s_eo[e];
    }

    // closed-form publication by the last workgroup to finish its rows
    if (!a.has_ring) return;   // grid-uniform
    if (refresh) tail_apply(a, tail_h);
    wait_vm();   // this wavefront's rows are complete
    __syncthreads();
    if (tid == 0) s_last = arrive_last(a.arrive) && cap_ok && read_status(a.st) == 0;
    __syncthreads();
    if (!s_last) return;
    ll_closed_publish<kWaves>(a, s_eo);
}

}  // namespace ep

using namespace ep;

namespace {

int64_t pack_grid_cap() {
    // per process (the library targets one GPU model); threads that race to
    // fill it compute the same value
    static std::atomic<int64_t> cached{0};
    int64_t cap = cached.load(std::memory_order_relaxed);
    if (cap == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cap = (int64_t)cus * kPackGridPerCuNum / kPackGridPerCuDen;
        if (cap < 1) cap = 1;
        cached.store(cap, std::memory_order_relaxed);
    }
    return cap;
}

// Workgroups of the rank-mode streaming pack (one-kernel or not): as many
// as leave every workgroup at least two passes, between half the CUs' worth
// and all of them.  Publication of a pass overlaps the copy of the next
// one, so a single pass would leave every descriptor to the end (train
// dispatch 116 against 99 us on all CUs); with many groups the whole chip
// copies (skewed 385 against 438 us).
int64_t stream_grid_cap(int64_t ngroups, int waves) {
    const int64_t half = pack_grid_cap() * kPackWaves / waves;
    const int64_t full = 2 * half;
    int64_t c = ceil_div(ngroups, (int64_t)2);
    if (c > full) c = full;
    if (c < half) c = half;
    return c;
}

// Rank-mode bf16 rows that one wavefront covers are split over two
// wavefronts (8 vectors a lane) when whole rows would make at least 4
// streaming passes.  Twice the passes halve each pass's burst of completed
// messages (skewed: about 370 commands a channel at a pass end, above the 256
// in flight, against about 186) with as many wavefronts in flight: its pack
// 385-393 -> 354 us.  At 2 passes the split costs more than it saves (train
// pack 99.5 -> 101-102.5 us).  The one-kernel large dispatch takes one
// wavefront per token, so split batches take the two calls.
bool rank_rows_split(const PackArgs& a, int fmt) {
    if (fmt != EP_FMT_BF16 || !a.has_ring || a.nv <= 512 || a.nv > 896) return false;
    if ((int64_t)a.T < kPackSmallWaves) return false;
    const int64_t ngroups = ceil_div((int64_t)a.T, (int64_t)kPackWaves);
    return ceil_div(ngroups, stream_grid_cap(ngroups, kPackWaves)) >= 4;
}

// SMALL: the small-batch configuration (closed-form publication; otherwise
// streaming with a ring).  LL: the per-expert pack.
template <int VPL, int FMT, int WAVES, bool SMALL, bool LL>
int launch_pack_fmt(PackArgs a, int64_t waves, hipStream_t stream) {
    const int pub = !a.has_ring ? kPubNone : SMALL ? kPubClosed : kPubStream;
    a.ngroups = ceil_div(waves, WAVES);
    // keep about the same number of wavefronts resident whatever WAVES is,
    // and give every workgroup the same number of passes (+-1 group), so no
    // few workgroups run a last pass alone.  The per-expert pack keeps half
    // the CUs' worth: more workgroups mean fewer, larger bursts of completed
    // messages for the in-flight window (train 130 -> 140 us).
    const int64_t cap = (pub == kPubStream && !LL) ? stream_grid_cap(a.ngroups, WAVES)
                                                   : pack_grid_cap() * kPackWaves / WAVES;
    const int64_t passes = ceil_div(a.ngroups, cap);
    const int64_t blocks = ceil_div(a.ngroups, passes);
    const dim3 grid((unsigned)blocks), block(WAVES * kWave);
    clear_hip_error();
    if (LL) {
        if (pub == kPubNone)
            hipLaunchKernelGGL((ll_pack_kernel<VPL, FMT, WAVES, kPubNone>), grid, block, 0, stream,
                               a);
        else if (pub == kPubClosed)
            hipLaunchKernelGGL((ll_pack_kernel<VPL, FMT, WAVES, kPubClosed>), grid, block, 0,
                               stream, a);
        else
            hipLaunchKernelGGL((ll_pack_kernel<VPL, FMT, WAVES, kPubStream>), grid, block, 0,
                               stream, a);
    } else if (pub == kPubNone)
        hipLaunchKernelGGL((pack_kernel<VPL, FMT, WAVES, kPubNone>), grid, block, 0, stream, a);
    else if (pub == kPubClosed)
        hipLaunchKernelGGL((pack_kernel<VPL, FMT, WAVES, kPubClosed>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((pack_kernel<VPL, FMT, WAVES, kPubStream>), grid, block, 0, stream, a);
    EP_HIP_CHECK(hipGetLastError());
    return EP_OK;
}

template <int VPL, int WAVES, bool SMALL, bool LL>
int launch_pack_wg(const PackArgs& a, int fmt, int64_t waves, hipStream_t stream) {
    if (fmt == EP_FMT_BF16)
        return launch_pack_fmt<VPL, EP_FMT_BF16, WAVES, SMALL, LL>(a, waves, stream);
    return launch_pack_fmt<VPL, EP_FMT_FP8_E4M3_B128, WAVES, SMALL, LL>(a, waves, stream);
}

template <int VPL, bool LL>
int launch_pack(const PackArgs& a, int fmt, int64_t waves, hipStream_t stream) {
    // fp8 holds the codes and scales too: half the wavefronts per workgroup
    // keep its registers (a 1024-thread workgroup caps a lane at 128)
    if (fmt == EP_FMT_BF16)
        return launch_pack_wg<VPL, kPackWaves, false, LL>(a, fmt, waves, stream);
    return launch_pack_wg<VPL, kPackWavesFp8, false, LL>(a, fmt, waves, stream);
}

// Small batches: short chunks and small workgroups spread the rows over the
// chip (a large workgroup of whole-row wavefronts would sit on a few CUs),
// and the descriptors go out in closed form at the end: with few rows, the
// copy is short and the publication latency is what remains.
template <int VPL, bool LL>
int launch_pack_small(const PackArgs& a, int fmt, int64_t waves, hipStream_t stream) {
    return launch_pack_wg<VPL, kPackWavesSmall, true, LL>(a, fmt, waves, stream);
}

// Vectors per lane and chunking of a pack launch (shared by both modes), then
// the launch.
template <bool LL>
int launch_pack_any(PackArgs& a, int fmt, hipStream_t stream) {
    // vectors per lane: one pass over the row when it fits (bf16: 16 per
    // lane); fp8 also holds the codes and scales, so it takes at most 8
    int vpl;
    if (a.nv <= 64) vpl = 1;
    else if (a.nv <= 128) vpl = 2;
    else if (a.nv <= 256) vpl = 4;
    else if (a.nv <= 512) vpl = 8;
    else if (fmt != EP_FMT_BF16) vpl = a.nv <= 896 ? kPackVplFp8H7168 : 8;
    // per-expert bf16 rows of up to 896 vectors take two wavefronts each: with
    // half as many tokens in flight, each pass completes half as many
    // messages at once, so the burst of publications at a pass's end fits
    // the in-flight window better (train 139 -> 131 us, skewed 618 -> 542 us)
    else if (a.nv <= 896) vpl = (LL || rank_rows_split(a, fmt)) ? 8 : kPackVplH7168;
    else vpl = 16;
    a.nchunks = (int32_t)ceil_div(a.nv, (int64_t)vpl * kWave);
    int64_t waves = (int64_t)a.T * a.nchunks;
    if (waves < kPackSmallWaves) {
        vpl = a.nv <= 64 ? 1 : 2;
        a.nchunks = (int32_t)ceil_div(a.nv, (int64_t)vpl * kWave);
        waves = (int64_t)a.T * a.nchunks;
        if (waves == 0) {
            if (!a.has_ring) return EP_OK;
            waves = 1;   // the zero-count ATOMICs still go out
        }
        return vpl == 1 ? launch_pack_small<1, LL>(a, fmt, waves, stream)
                        : launch_pack_small<2, LL>(a, fmt, waves, stream);
    }
    switch (vpl) {
        case 1: return launch_pack<1, LL>(a, fmt, waves, stream);
        case 2: return launch_pack<2, LL>(a, fmt, waves, stream);
        case 4: return launch_pack<4, LL>(a, fmt, waves, stream);
        case 8: return launch_pack<8, LL>(a, fmt, waves, stream);
        case 14: return launch_pack<14, LL>(a, fmt, waves, stream);
        default: return launch_pack<16, LL>(a, fmt, waves, stream);
    }
}

template <int VPL, int FMT>
int launch_fused_fmt(PackArgs a, int64_t waves, hipStream_t stream) {
    a.ngroups = ceil_div(waves, kPackWavesSmall);
    const int64_t cap = pack_grid_cap() * kPackWaves / kPackWavesSmall;
    const int64_t passes = ceil_div(a.ngroups, cap);
    const int64_t blocks = ceil_div(a.ngroups, passes);
    clear_hip_error();
    if (a.k <= 8)
        hipLaunchKernelGGL((fused_small_kernel<VPL, FMT, 8>), dim3((unsigned)blocks),
                           dim3(kPackWavesSmall * kWave), 0, stream, a);
    else
        hipLaunchKernelGGL((fused_small_kernel<VPL, FMT, kMaxK>), dim3((unsigned)blocks),
                           dim3(kPackWavesSmall * kWave), 0, stream, a);
    EP_HIP_CHECK(hipGetLastError());
    return EP_OK;
}

// Chunking of the one-kernel small batch: that of the small-batch pack.
int launch_fused(PackArgs& a, int fmt, hipStream_t stream) {
    const int vpl = a.nv <= 64 ? 1 : 2;
    a.nchunks = (int32_t)ceil_div(a.nv, (int64_t)vpl * kWave);
    int64_t waves = (int64_t)a.T * a.nchunks;
    if (waves == 0) waves = 1;   // the layout outputs and the zero-count ATOMICs still go out
    if (fmt == EP_FMT_BF16)
        return vpl == 1 ? launch_fused_fmt<1, EP_FMT_BF16>(a, waves, stream)
                        : launch_fused_fmt<2, EP_FMT_BF16>(a, waves, stream);
    return vpl == 1 ? launch_fused_fmt<1, EP_FMT_FP8_E4M3_B128>(a, waves, stream)
                    : launch_fused_fmt<2, EP_FMT_FP8_E4M3_B128>(a, waves, stream);
}

// One-kernel large batch: the work order of the two-kernel pack (same
// group size and grid), when it has one wavefront per token, at most
// kFusedLargeMaxPasses groups per workgroup, and room for every pack
// workgroup at once (the expert counts get a workgroup of their own when one
// more fits, else the pack workgroups take them).  kNotTaken when the batch
// does not qualify; nothing is launched then.
constexpr int kNotTaken = -1;   // no status code is negative

template <typename K>
int64_t resident_blocks(K kernel, int threads) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel),
                                                     threads, 0) != hipSuccess)
        return 0;
    return (int64_t)cus * per_cu;
}

template <int VPL, int FMT, int WAVES, int KMAX>
int launch_fused_large_fmt(PackArgs a, hipStream_t stream, bool dry) {
    a.ngroups = ceil_div(a.T, WAVES);
    const int64_t cap = a.has_ring ? stream_grid_cap(a.ngroups, WAVES)
                                   : pack_grid_cap() * kPackWaves / WAVES;
    const int64_t passes = ceil_div(a.ngroups, cap);
    const int64_t blocks = ceil_div(a.ngroups, passes);
    if (passes > kFusedLargeMaxPasses) return kNotTaken;
    // per process and ring mode (one GPU model); racing threads compute the
    // same value
    static std::atomic<int64_t> room[2] = {{-1}, {-1}};
    const int pub = a.has_ring ? kPubStream : kPubNone;
    int64_t rm = room[a.has_ring ? 1 : 0].load(std::memory_order_relaxed);
    if (rm < 0) {
        rm = a.has_ring ? resident_blocks(fused_large_kernel<VPL, FMT, WAVES, kPubStream, KMAX>,
                                          WAVES * kWave)
                        : resident_blocks(fused_large_kernel<VPL, FMT, WAVES, kPubNone, KMAX>,
                                          WAVES * kWave);
        room[a.has_ring ? 1 : 0].store(rm, std::memory_order_relaxed);
    }
    if (blocks > rm) return kNotTaken;
    if (dry) return EP_OK;
    a.npass = (int32_t)passes;
    a.nchunks = 1;
    // the expert counts' own workgroup when it fits beside the pack's
    a.expert_wg = blocks + 1 <= rm ? 1 : 0;
    const dim3 grid((unsigned)(blocks + a.expert_wg)), block(WAVES * kWave);
    clear_hip_error();
    if (pub == kPubStream)
        hipLaunchKernelGGL((fused_large_kernel<VPL, FMT, WAVES, kPubStream, KMAX>), grid, block,
                           0, stream, a);
    else
        hipLaunchKernelGGL((fused_large_kernel<VPL, FMT, WAVES, kPubNone, KMAX>), grid, block, 0,
                           stream, a);
    EP_HIP_CHECK(hipGetLastError());
    return EP_OK;
}

// The vectors per lane of the two-kernel pack for this row size, if one
// wavefront covers a row, the batch is large enough for the streaming pack
// and the two-kernel pack would not split its rows (smaller batches, smaller
// or split rows and fp8 take the two-kernel path).  dry: only whether the
// batch would take the path.
template <int VPL, int FMT, int WAVES>
int launch_fused_large_k(PackArgs& a, hipStream_t stream, bool dry) {
    return a.k <= 8 ? launch_fused_large_fmt<VPL, FMT, WAVES, 8>(a, stream, dry)
                    : launch_fused_large_fmt<VPL, FMT, WAVES, kMaxK>(a, stream, dry);
}

int launch_fused_large(PackArgs& a, int fmt, hipStream_t stream, bool dry = false) {
    if ((int64_t)a.T < kPackSmallWaves) return kNotTaken;
    const int nv = a.nv;
    if (fmt == EP_FMT_BF16) {
        if (nv <= 128) return kNotTaken;
        if (nv <= 256) return launch_fused_large_k<4, EP_FMT_BF16, kPackWaves>(a, stream, dry);
        if (nv <= 512) return launch_fused_large_k<8, EP_FMT_BF16, kPackWaves>(a, stream, dry);
        if (nv <= 896) {
            if (rank_rows_split(a, fmt)) return kNotTaken;   // two wavefronts a row
            return launch_fused_large_k<kPackVplH7168, EP_FMT_BF16, kPackWaves>(a, stream, dry);
        }
        if (nv <= 1024) return launch_fused_large_k<16, EP_FMT_BF16, kPackWaves>(a, stream, dry);
        return kNotTaken;
    }
    // fp8 rows stay with the two calls: the one-kernel version (8-wavefront
    // workgroups at 151 registers a lane, one per compute unit, expert counts
    // in the pack workgroups) made the fp8 step slower (183-184 against
    // 175.5 us)
    return kNotTaken;
}

// One-kernel per-expert small batch: the chunking of the small-batch pack.
template <int VPL, int FMT>
int launch_ll_fused_fmt(PackArgs a, int64_t waves, hipStream_t stream) {
    a.ngroups = ceil_div(waves, kPackWavesSmall);
    const int64_t cap = pack_grid_cap() * kPackWaves / kPackWavesSmall;
    const int64_t passes = ceil_div(a.ngroups, cap);
    const int64_t blocks = ceil_div(a.ngroups, passes);
    clear_hip_error();
    if (a.k <= 8)
        hipLaunchKernelGGL((ll_fused_small_kernel<VPL, FMT, 8>), dim3((unsigned)blocks),
                           dim3(kPackWavesSmall * kWave), 0, stream, a);
    else
        hipLaunchKernelGGL((ll_fused_small_kernel<VPL, FMT, kMaxK>), dim3((unsigned)blocks),
                           dim3(kPackWavesSmall * kWave), 0, stream, a);
    EP_HIP_CHECK(hipGetLastError());
    return EP_OK;
}

int launch_ll_fused(PackArgs& a, int fmt, hipStream_t stream) {
    const int vpl = a.nv <= 64 ? 1 : 2;
    a.nchunks = (int32_t)ceil_div(a.nv, (int64_t)vpl * kWave);
    int64_t waves = (int64_t)a.T * a.nchunks;
    if (waves == 0) waves = 1;   // the counts and the zero-count ATOMICs still go out
    if (fmt == EP_FMT_BF16)
        return vpl == 1 ? launch_ll_fused_fmt<1, EP_FMT_BF16>(a, waves, stream)
                        : launch_ll_fused_fmt<2, EP_FMT_BF16>(a, waves, stream);
    return vpl == 1 ? launch_ll_fused_fmt<1, EP_FMT_FP8_E4M3_B128>(a, waves, stream)
                    : launch_ll_fused_fmt<2, EP_FMT_FP8_E4M3_B128>(a, waves, stream);
}

}  // namespace

extern "C" int ep_dispatch_ll_fused(const ep_shape_t* shape, const void* x,
                                    const int32_t* topk_idx, const float* topk_w,
                                    int32_t* num_tokens_per_expert, int32_t* expert_offset,
                                    int32_t* expert_slot, void* send_buf, int64_t capacity_rows,
                                    int32_t* slot_src, float* slot_w, ep_ring_t* ring,
                                    void* workspace, size_t ws_bytes, int32_t* dev_status,
                                    hipStream_t stream) {
    int v = validate_shape(shape);
    if (v != EP_OK) return v;
    const ep_shape_t s = *shape;
    if (s.T > kFusedMaxT || s.E > kLLFusedMaxE) return EP_ERR_INVALID_ARG;
    if (!num_tokens_per_expert || !expert_offset || !dev_status || !workspace || capacity_rows < 0)
        return EP_ERR_INVALID_ARG;
    if (s.T > 0 && (!x || !topk_idx || !topk_w || !expert_slot)) return EP_ERR_INVALID_ARG;
    if (capacity_rows > 0 && (!send_buf || !slot_src || !slot_w)) return EP_ERR_INVALID_ARG;
    if (((uintptr_t)x | (uintptr_t)send_buf) & 15) return EP_ERR_INVALID_ARG;
    if (ws_bytes < workspace_bytes(s)) return EP_ERR_INVALID_ARG;
    if (ring && (uint64_t)capacity_rows * row_bytes(s.H, s.fmt) > kMaxRingOffset)
        return EP_ERR_INVALID_ARG;   // descriptor offsets are 48-bit
    Workspace w = carve_workspace(s, workspace);

    PackArgs a{};
    a.x = reinterpret_cast<const u32x4*>(x);
    a.idx = topk_idx;
    a.w = topk_w;
    a.send_buf = reinterpret_cast<uint8_t*>(send_buf);
    a.slot_src = slot_src;
    a.slot_w = slot_w;
    a.arrive = w.arrive;
    a.msg_arrivals = w.msg_arrivals;
    a.msgs_done = w.msgs_done;
    a.max_msgs = w.max_msgs;
    a.st = dev_status;
    a.ring = ring_device_view(ring);
    a.has_ring = ring != nullptr;
    a.cap = capacity_rows;
    a.row_bytes = (int64_t)row_bytes(s.H, s.fmt);
    a.T = s.T;
    a.H = s.H;
    a.E = s.E;
    a.R = s.R;
    a.k = s.k;
    a.epr = s.E / s.R;
    a.nv = s.H / 8;
    a.cnt_exp_out = num_tokens_per_expert;
    a.exp_off_out = expert_offset;
    a.send_slot_out = expert_slot;
    return launch_ll_fused(a, s.fmt, stream);
}

extern "C" int ep_dispatch_fused(const ep_shape_t* shape, const void* x, const int32_t* topk_idx,
                                 const float* topk_w, int32_t* num_tokens_per_rank,
                                 int32_t* num_tokens_per_expert, int32_t* rank_offset,
                                 int32_t* expert_offset, uint8_t* is_token_in_rank,
                                 int32_t* send_slot, void* send_buf, int64_t capacity_rows,
                                 int32_t* slot_src, int32_t* slot_local_idx, float* slot_local_w,
                                 ep_ring_t* ring, void* workspace, size_t ws_bytes,
                                 int32_t* dev_status, hipStream_t stream) {
    int v = validate_shape(shape);
    if (v != EP_OK) return v;
    const ep_shape_t s = *shape;
    if (!num_tokens_per_rank || !num_tokens_per_expert || !rank_offset || !expert_offset ||
        !dev_status || !workspace || capacity_rows < 0)
        return EP_ERR_INVALID_ARG;
    if (s.T > 0 && (!x || !topk_idx || !topk_w || !is_token_in_rank || !send_slot))
        return EP_ERR_INVALID_ARG;
    if (capacity_rows > 0 && (!send_buf || !slot_src || !slot_local_idx || !slot_local_w))
        return EP_ERR_INVALID_ARG;
    if (((uintptr_t)x | (uintptr_t)send_buf) & 15) return EP_ERR_INVALID_ARG;
    // the two-kernel fallback of large batches stores send_slot and
    // is_token_in_rank in 16- and 4-byte pieces
    if (s.T > kFusedMaxT && (((uintptr_t)send_slot & 15) || ((uintptr_t)is_token_in_rank & 3)))
        return EP_ERR_INVALID_ARG;
    if (ws_bytes < workspace_bytes(s)) return EP_ERR_INVALID_ARG;
    if (ring && (uint64_t)capacity_rows * row_bytes(s.H, s.fmt) > kMaxRingOffset)
        return EP_ERR_INVALID_ARG;   // descriptor offsets are 48-bit
    Workspace w = carve_workspace(s, workspace);

    PackArgs a{};
    a.x = reinterpret_cast<const u32x4*>(x);
    a.idx = topk_idx;
    a.w = topk_w;
    a.rank_off = rank_offset;
    a.send_slot = send_slot;
    a.send_buf = reinterpret_cast<uint8_t*>(send_buf);
    a.slot_src = slot_src;
    a.slot_local_idx = slot_local_idx;
    a.slot_local_w = slot_local_w;
    a.msg_base = w.msg_base;
    a.msg_arrivals = w.msg_arrivals;
    a.msgs_done = w.msgs_done;
    a.max_msgs = w.max_msgs;
    a.arrive = w.arrive;
    a.st = dev_status;
    a.ring = ring_device_view(ring);
    a.has_ring = ring != nullptr;
    a.cap = capacity_rows;
    a.row_bytes = (int64_t)row_bytes(s.H, s.fmt);
    a.T = s.T;
    a.H = s.H;
    a.E = s.E;
    a.R = s.R;
    a.k = s.k;
    a.epr = s.E / s.R;
    a.nv = s.H / 8;
    a.cnt_rank_out = num_tokens_per_rank;
    a.cnt_exp_out = num_tokens_per_expert;
    a.rank_off_out = rank_offset;
    a.exp_off_out = expert_offset;
    a.in_rank_out = is_token_in_rank;
    a.send_slot_out = send_slot;
    a.msg_base_out = w.msg_base;
    a.counters_n = w.counters_n;
    a.bar = w.barrier;
    a.wave_cnt = w.wave_rank_cnt;
    // the per-tile expert table of the layout kernel is free in a one-kernel
    // call (no per-expert row table reads it afterwards): at least 4 rows of
    // E here, since the one-kernel large path takes T >= 1024
    a.exp_part = w.blk_exp_cnt;
    a.nparts = w.layout_blocks < kExpParts ? w.layout_blocks : kExpParts;
    if (s.T <= kFusedMaxT) return launch_fused(a, s.fmt, stream);
    v = launch_fused_large(a, s.fmt, stream);
    if (v != kNotTaken) return v;
    // the two-kernel path: layout, then pack
    v = ep_dispatch_layout(shape, topk_idx, num_tokens_per_rank, num_tokens_per_expert,
                           rank_offset, expert_offset, is_token_in_rank, send_slot, workspace,
                           ws_bytes, dev_status, stream);
    if (v != EP_OK) return v;
    return ep_dispatch(shape, x, topk_idx, topk_w, rank_offset, send_slot, send_buf,
                       capacity_rows, slot_src, slot_local_idx, slot_local_w, ring, workspace,
                       ws_bytes, dev_status, stream);
}

extern "C" int ep_dispatch_fused_plan(const ep_shape_t* shape, int32_t with_ring) {
    int v = validate_shape(shape);
    if (v != EP_OK) return v;
    const ep_shape_t s = *shape;
    if (s.T <= kFusedMaxT) return EP_FUSED_ONE_KERNEL_SMALL;
    PackArgs a{};
    a.T = s.T;
    a.nv = s.H / 8;
    a.has_ring = with_ring != 0;
    return launch_fused_large(a, s.fmt, nullptr, true) == EP_OK ? EP_FUSED_ONE_KERNEL_LARGE
                                                                 : EP_FUSED_TWO_CALLS;
}

extern "C" int ep_dispatch(const ep_shape_t* shape, const void* x, const int32_t* topk_idx,
                           const float* topk_w, const int32_t* rank_offset,
                           const int32_t* send_slot, void* send_buf, int64_t capacity_rows,
                           int32_t* slot_src, int32_t* slot_local_idx, float* slot_local_w,
                           ep_ring_t* ring, void* workspace, size_t ws_bytes, int32_t* dev_status,
                           hipStream_t stream) {
    int v = validate_shape(shape);
    if (v != EP_OK) return v;
    const ep_shape_t s = *shape;
    if (!rank_offset || !dev_status || !workspace || capacity_rows < 0) return EP_ERR_INVALID_ARG;
    if (s.T > 0 && (!x || !topk_idx || !topk_w || !send_slot)) return EP_ERR_INVALID_ARG;
    if (capacity_rows > 0 && (!send_buf || !slot_src || !slot_local_idx || !slot_local_w))
        return EP_ERR_INVALID_ARG;
    if (((uintptr_t)x | (uintptr_t)send_buf) & 15) return EP_ERR_INVALID_ARG;
    if (ws_bytes < workspace_bytes(s)) return EP_ERR_INVALID_ARG;
    if (ring && (uint64_t)capacity_rows * row_bytes(s.H, s.fmt) > kMaxRingOffset)
        return EP_ERR_INVALID_ARG;   // descriptor offsets are 48-bit
    Workspace w = carve_workspace(s, workspace);

    PackArgs a{};
    a.x = reinterpret_cast<const u32x4*>(x);
    a.idx = topk_idx;
    a.w = topk_w;
    a.rank_off = rank_offset;
    a.send_slot = send_slot;
    a.send_buf = reinterpret_cast<uint8_t*>(send_buf);
    a.slot_src = slot_src;
    a.slot_local_idx = slot_local_idx;
    a.slot_local_w = slot_local_w;
    a.msg_base = w.msg_base;
    a.msg_arrivals = w.msg_arrivals;
    a.msgs_done = w.msgs_done;
    a.max_msgs = w.max_msgs;
    a.arrive = w.arrive;
    a.st = dev_status;
    a.ring = ring_device_view(ring);
    a.has_ring = ring != nullptr;
    a.cap = capacity_rows;
    a.row_bytes = (int64_t)row_bytes(s.H, s.fmt);
    a.T = s.T;
    a.H = s.H;
    a.E = s.E;
    a.R = s.R;
    a.k = s.k;
    a.epr = s.E / s.R;
    a.nv = s.H / 8;

    return launch_pack_any<false>(a, s.fmt, stream);
}

extern "C" int ep_dispatch_ll(const ep_shape_t* shape, const void* x, const int32_t* topk_idx,
                              const float* topk_w, const int32_t* expert_offset,
                              const int32_t* expert_slot, void* send_buf, int64_t capacity_rows,
                              int32_t* slot_src, float* slot_w, ep_ring_t* ring, void* workspace,
                              size_t ws_bytes, int32_t* dev_status, hipStream_t stream) {
    int v = validate_shape(shape);
    if (v != EP_OK) return v;
    const ep_shape_t s = *shape;
    if (!expert_offset || !dev_status || !workspace || capacity_rows < 0)
        return EP_ERR_INVALID_ARG;
    if (s.T > 0 && (!x || !topk_idx || !topk_w || !expert_slot)) return EP_ERR_INVALID_ARG;
    if (capacity_rows > 0 && (!send_buf || !slot_src || !slot_w)) return EP_ERR_INVALID_ARG;
    if (((uintptr_t)x | (uintptr_t)send_buf) & 15) return EP_ERR_INVALID_ARG;
    if (ws_bytes < workspace_bytes(s)) return EP_ERR_INVALID_ARG;
    if (ring && (uint64_t)capacity_rows * row_bytes(s.H, s.fmt) > kMaxRingOffset)
        return EP_ERR_INVALID_ARG;   // descriptor offsets are 48-bit
    Workspace w = carve_workspace(s, workspace);

    PackArgs a{};
    a.x = reinterpret_cast<const u32x4*>(x);
    a.idx = topk_idx;
    a.w = topk_w;
    a.exp_off = expert_offset;
    a.expert_slot = expert_slot;
    a.send_buf = reinterpret_cast<uint8_t*>(send_buf);
    a.slot_src = slot_src;
    a.slot_w = slot_w;
    a.arrive = w.arrive;
    a.msg_arrivals = w.msg_arrivals;
    a.msgs_done = w.msgs_done;
    a.max_msgs = w.max_msgs;
    a.st = dev_status;
    a.ring = ring_device_view(ring);
    a.has_ring = ring != nullptr;
    a.cap = capacity_rows;
    a.row_bytes = (int64_t)row_bytes(s.H, s.fmt);
    a.T = s.T;
    a.H = s.H;
    a.E = s.E;
    a.R = s.R;
    a.k = s.k;
    a.epr = s.E / s.R;
    a.nv = s.H / 8;
    return launch_pack_any<true>(a, s.fmt, stream);
}
