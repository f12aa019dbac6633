// ep_ring_proto.h -- the TransferCmd ring's slot format and its consumer side
// (UCCL-EP article s2.2: a FIFO of slots with head and tail, filled by GPU
// producers and drained in order by a CPU proxy).  Plain C++ with no HIP
// types: the GPU producer (ep_dispatch.hip) encodes slots with
// ring_slot_words, the host proxy (ep_ring.hip) pops them with ring_pop, and
// a CPU model of the protocol compiles the same code with a host compiler.
//
// One slot is four 64-bit words, each
//   bits  0..15  tag = low 16 bits of (ticket + 1)
//   bits 16..63  48 bits of the command:
//     w0: type (8) | op (8) | num_tokens (16) | 0 (16)
//     w1: dst_rank (16) | size_or_value (32)
//     w2: src_offset (48)
//     w3: dst_offset (48)
// A producer writes the four words in any order and never a separate flag.
// A consumer that finds the tag of the ticket it waits for in all four words
// (8-byte loads are single-copy atomic) has the whole command.  A stale slot
// holds the tag of ticket - depth + 1, which differs while depth < 65536.
// Producers keep a ticket t unwritten until t < consumer position +
// max_inflight (<= depth), so a slot is never overwritten before it is popped.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define EP_HOST_DEVICE __host__ __device__
#else
#define EP_HOST_DEVICE
#endif

namespace ep {

struct RingSlot {
    uint64_t w[4];
};
static_assert(sizeof(RingSlot) == 32, "ring slot is 32 bytes");
constexpr uint64_t kMaxRingOffset = (1ull << 48) - 1;
constexpr int32_t kMaxRingDepth = 65535;

// The four words of command `ticket`.
EP_HOST_DEVICE inline void ring_slot_words(unsigned long long ticket, uint32_t type, uint32_t op,
                                           uint32_t ntok, uint32_t dst_rank, uint32_t size_val,
                                           uint64_t src_off, uint64_t dst_off, uint64_t w[4]) {
    const uint64_t tag = (uint64_t)((ticket + 1) & 0xFFFFull);
    w[0] = tag | ((uint64_t)(type & 0xFF) << 16) | ((uint64_t)(op & 0xFF) << 24) |
           ((uint64_t)(ntok & 0xFFFF) << 32);
    w[1] = tag | ((uint64_t)(dst_rank & 0xFFFF) << 16) | ((uint64_t)size_val << 32);
    w[2] = tag | ((src_off & kMaxRingOffset) << 16);
    w[3] = tag | ((dst_off & kMaxRingOffset) << 16);
}

// Read one slot and decode it into *out (fields of ep_transfer_cmd_t) when
// every word carries the tag of ticket want - 1.
template <class Cmd>
inline bool ring_read_slot(const RingSlot* s, uint32_t want, Cmd* out) {
    const uint64_t tag = want & 0xFFFFu;
    uint64_t w[4];
    for (int i = 0; i < 4; ++i) {
        w[i] = __atomic_load_n(&s->w[i], __ATOMIC_ACQUIRE);
        if ((w[i] & 0xFFFFu) != tag) return false;
    }
    if (out) {
        out->seq = want;
        out->type = (uint8_t)(w[0] >> 16);
        out->op = (uint8_t)(w[0] >> 24);
        out->num_tokens = (uint16_t)(w[0] >> 32);
        out->dst_rank = (uint32_t)((w[1] >> 16) & 0xFFFFu);
        out->size_or_value = (uint32_t)(w[1] >> 32);
        out->src_offset = w[2] >> 16;
        out->dst_offset = w[3] >> 16;
    }
    return true;
}

// Pop up to `max` published commands of one channel (slots base[0..depth))
// in ticket order from consumer position *pos into out (may be NULL); when
// anything was popped, advance *pos and, if tail is not NULL, publish the new
// position there (release) so that producers may reuse the slots.  Returns
// the number popped.
template <class Cmd>
inline int64_t ring_pop(const RingSlot* base, uint32_t depth, unsigned long long* pos,
                        unsigned long long* tail, Cmd* out, int64_t max) {
    unsigned long long p = *pos;
    int64_t n = 0;
    while (n < max) {
        const RingSlot* s = base + (p % depth);
        // Slot lines written by the GPU miss in the CPU caches; touching the
        // lines a few slots ahead overlaps those misses when a backlog exists.
        if ((p & 1) == 0) {
            __builtin_prefetch(base + ((p + 8) % depth), 0, 0);
            __builtin_prefetch(base + ((p + 16) % depth), 0, 0);
        }
        if (!ring_read_slot(s, (uint32_t)(p + 1), out ? &out[n] : (Cmd*)nullptr)) break;
        ++p;
        ++n;
    }
    if (n) {
        *pos = p;
        if (tail) __atomic_store_n(tail, p, __ATOMIC_RELEASE);
    }
    return n;
}

}  // namespace ep
