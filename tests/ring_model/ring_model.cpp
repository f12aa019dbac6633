// ring_model.cpp -- a CPU model of the TransferCmd ring protocol, run against
// the library's own slot encoding and consumer (ep_ring_proto.h).
//
// Producer threads follow the producer rules the GPU kernels follow (UCCL-EP
// article s2.2: a FIFO with lock-free head and tail, batched enqueue of up to
// 8, a producer blocked while max_inflight commands are in flight):
//   - reserve 1..4 consecutive tickets with one fetch_add on head;
//   - write ticket t only once t < tail + max_inflight, refreshing the cached
//     tail from the consumer's published one when the cache says full; give
//     up with a timeout status when the wait passes the timeout;
//   - write the four tagged words of the slot, one 8-byte store each, in a
//     random order (the GPU's two 16-byte stores may land in any order).
// One consumer thread pops with ring_pop in batches of 32, as a proxy does.
//
// Checks: every ticket is popped once, in order, with the command its
// producer wrote (decoded fields equal the ones derived from the ticket); the
// number of written-but-unpopped commands, taken against the consumer's real
// position at each write, never exceeds max_inflight; with no consumer the
// producers time out instead of hanging.
//
// usage: ring_model <depth> <max_inflight> <producers> <pushes> <timeout_ms> <consume 0|1>
// Prints one JSON line; exit status 0 when every check passed.

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <thread>
#include <vector>

#include "ep_ring_proto.h"

#ifndef RING_MODEL_WINDOW_SLACK
#define RING_MODEL_WINDOW_SLACK 0   // a planted producer bug sets this to 1
#endif

namespace {

struct Cmd {
    uint32_t seq;
    uint8_t type, op;
    uint16_t num_tokens;
    uint32_t dst_rank, size_or_value;
    uint64_t src_offset, dst_offset;
};

// The command a producer writes for ticket t (distinct fields per ticket).
Cmd command_of(unsigned long long t) {
    Cmd c{};
    c.seq = (uint32_t)(t + 1);
    c.type = (uint8_t)(1 + (t & 1));
    c.op = (uint8_t)((t >> 1) & 1);
    c.num_tokens = (uint16_t)(t % 9);
    c.dst_rank = (uint32_t)(t % 64);
    c.size_or_value = (uint32_t)(t * 2654435761ull);
    c.src_offset = (t * 0x9E3779B97ull) & ep::kMaxRingOffset;
    c.dst_offset = (t ^ 0x5A5A5A5A5Aull) & ep::kMaxRingOffset;
    return c;
}

bool same(const Cmd& a, const Cmd& b) {
    return a.seq == b.seq && a.type == b.type && a.op == b.op && a.num_tokens == b.num_tokens &&
           a.dst_rank == b.dst_rank && a.size_or_value == b.size_or_value &&
           a.src_offset == b.src_offset && a.dst_offset == b.dst_offset;
}

int64_t now_ns() {
    return std::chrono::duration_cast<std::chrono::nanoseconds>(
               std::chrono::steady_clock::now().time_since_epoch())
        .count();
}

}  // namespace

int main(int argc, char** argv) {
    if (argc != 7) {
        std::fprintf(stderr, "usage: %s depth max_inflight producers pushes timeout_ms consume\n",
                     argv[0]);
        return 2;
    }
    const uint32_t depth = (uint32_t)std::atoi(argv[1]);
    const unsigned long long window = (unsigned long long)std::atoll(argv[2]);
    const int producers = std::atoi(argv[3]);
    const unsigned long long pushes = (unsigned long long)std::atoll(argv[4]);
    const int64_t timeout_ns = (int64_t)std::atoll(argv[5]) * 1000000;
    const bool consume = std::atoi(argv[6]) != 0;
    if (depth < 1 || window < 1 || window > depth || producers < 1) return 2;

    std::vector<ep::RingSlot> slots(depth);
    for (auto& s : slots)
        for (auto& w : s.w) w = 0;   // tag 0: no ticket t has tag 0 before t = 65535
    std::atomic<unsigned long long> head{0};
    unsigned long long tail = 0;                 // published by the consumer (release)
    std::atomic<unsigned long long> written{0};  // commands written by producers
    std::atomic<unsigned long long> max_inflight_seen{0};
    std::atomic<int> timeouts{0};
    std::atomic<bool> stop{false};

    auto producer = [&](int id) {
        std::mt19937_64 rng(1234 + id);
        unsigned long long cached_tail = 0;
        while (!stop.load(std::memory_order_relaxed)) {
            const unsigned n = 1 + (unsigned)(rng() % 4);
            const unsigned long long t0 = head.fetch_add(n, std::memory_order_relaxed);
            for (unsigned i = 0; i < n; ++i) {
                const unsigned long long t = t0 + i;
                if (t >= pushes) return;
                const int64_t start = now_ns();
                // wait until the ticket may be written
                while (t >= cached_tail + window + RING_MODEL_WINDOW_SLACK) {
                    cached_tail = __atomic_load_n(&tail, __ATOMIC_ACQUIRE);
                    if (t < cached_tail + window + RING_MODEL_WINDOW_SLACK) break;
                    if (now_ns() - start > timeout_ns) {
                        timeouts.fetch_add(1);
                        stop.store(true);
                        return;
                    }
                    std::this_thread::yield();
                }
                // in flight after this write, against the consumer's real position
                const unsigned long long inflight = t + 1 - __atomic_load_n(&tail, __ATOMIC_ACQUIRE);
                unsigned long long m = max_inflight_seen.load();
                while (inflight > m && !max_inflight_seen.compare_exchange_weak(m, inflight)) {
                }
                const Cmd c = command_of(t);
                uint64_t w[4];
                ep::ring_slot_words(t, c.type, c.op, c.num_tokens, c.dst_rank, c.size_or_value,
                                    c.src_offset, c.dst_offset, w);
                int order[4] = {0, 1, 2, 3};
                std::shuffle(order, order + 4, rng);
                ep::RingSlot* s = &slots[t % depth];
                for (int k = 0; k < 4; ++k) {
                    __atomic_store_n(&s->w[order[k]], w[order[k]], __ATOMIC_RELEASE);
                    if ((rng() & 63) == 0) std::this_thread::yield();   // let a reader in between
                }
                written.fetch_add(1);
            }
        }
    };

    std::vector<std::thread> th;
    for (int i = 0; i < producers; ++i) th.emplace_back(producer, i);

    unsigned long long popped = 0, pos = 0, bad = 0, first_bad = ~0ull;
    if (consume) {
        Cmd batch[32];
        int64_t idle_since = now_ns();
        while (popped < pushes) {
            const int64_t n = ep::ring_pop(slots.data(), depth, &pos, &tail, batch, 32);
            for (int64_t i = 0; i < n; ++i) {
                const unsigned long long t = popped + (unsigned long long)i;
                if (!same(batch[i], command_of(t))) {
                    ++bad;
                    if (first_bad == ~0ull) first_bad = t;
                }
            }
            popped += (unsigned long long)n;
            if (n) {
                idle_since = now_ns();
            } else {
                if (timeouts.load() || now_ns() - idle_since > 20 * timeout_ns) break;
                std::this_thread::yield();
            }
        }
    }
    // with no consumer the producers end by their own timeouts
    if (consume) stop.store(true);
    for (auto& t : th) t.join();

    const unsigned long long mx = max_inflight_seen.load();
    bool ok;
    if (consume) {
        ok = popped == pushes && bad == 0 && timeouts.load() == 0 && mx <= window && pos == pushes;
    } else {
        // nobody drains: exactly the first max_inflight commands are written,
        // then the producers give up with a timeout
        ok = timeouts.load() > 0 && written.load() == window && mx <= window;
    }
    std::printf("{\"ok\": %s, \"depth\": %u, \"max_inflight\": %llu, \"producers\": %d, "
                "\"pushes\": %llu, \"popped\": %llu, \"bad\": %llu, \"first_bad\": %lld, "
                "\"written\": %llu, \"max_inflight_seen\": %llu, \"timeouts\": %d}\n",
                ok ? "true" : "false", depth, window, producers, pushes, popped, bad,
                first_bad == ~0ull ? -1LL : (long long)first_bad, written.load(), mx,
                timeouts.load());
    return ok ? 0 : 1;
}
