// ep_ring.hip — host side of the TransferCmd FIFO (UCCL-EP article: s2.1 the
// GPU writes commands into a local FIFO, s2.2 the ring of head/tail/slots with
// an in-flight limit, s2.3 proxy threads that dequeue, execute and complete,
// s5.2 drain batch of 32).
//
// Memory placement: the consumer is a CPU thread, so the slots and the
// consumer position (tail) sit in host-pinned coherent memory, where the CPU
// polls them locally and the GPU reaches them with PCIe writes.  The producer
// ticket counter (head) and the producers' cached copy of tail sit in device
// memory, so reserving a slot is a device atomic, and the GPU reads tail over
// PCIe only when its cached copy says the channel is full.
//
// There is no network here: a proxy thread "executes" a command by logging
// it and marking it completed (advancing tail).

#include <atomic>
#include <chrono>
#include <cstring>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include "ep_common.h"

#if defined(__x86_64__)
#include <immintrin.h>
#define EP_CPU_RELAX() _mm_pause()
#else
#define EP_CPU_RELAX() ((void)0)
#endif

struct ep_ring {
    int32_t depth = 0, channels = 0, max_inflight = 0;
    int64_t timeout_ns = 0;
    int device = 0;
    ep::RingSlot* slots = nullptr;             // host-pinned
    unsigned long long* host_tail = nullptr;   // host-pinned, stride kPad
    unsigned long long* dev_state = nullptr;   // device: head, tail_cache, poll; each [C*kPad]
    unsigned long long timeout_ticks = 0;
    std::vector<unsigned long long> pos;       // consumer position per channel
    std::mutex mu;                             // serialises host-side calls
    // proxy
    std::vector<std::thread> threads;
    std::atomic<bool> stop{false};
    std::atomic<bool> running{false};
    std::atomic<int64_t> drained{0};
    std::atomic<int64_t> log_n{0};
    int64_t log_capacity = 0;
    std::vector<ep_transfer_cmd_t> log;
};

namespace ep {

RingDev ring_device_view(ep_ring_t* r) {
    RingDev d{};
    if (!r) return d;
    d.slots = r->slots;
    d.host_tail = r->host_tail;
    d.head = r->dev_state;
    d.tail_cache = r->dev_state + (size_t)r->channels * kPad;
    d.poll = r->dev_state + 2 * (size_t)r->channels * kPad;
    d.depth = r->depth;
    d.channels = r->channels;
    d.max_inflight = r->max_inflight;
    d.timeout_ticks = r->timeout_ticks;
    return d;
}

}  // namespace ep

using namespace ep;

namespace {

// Read one slot (four 8-byte loads) and decode it when every word carries
// the tag of ticket `want - 1`.
inline bool read_slot(const RingSlot* s, uint32_t want, ep_transfer_cmd_t* out) {
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

// Pop up to `max` published commands of channel c; returns the number popped.
int64_t pop_channel(ep_ring_t* r, int c, ep_transfer_cmd_t* out, int64_t max, bool publish) {
    unsigned long long p = r->pos[c];
    const RingSlot* base = r->slots + (size_t)c * r->depth;
    int64_t n = 0;
    while (n < max) {
        const RingSlot* s = base + (p % (unsigned long long)r->depth);
        // Slot lines written by the GPU miss in the CPU caches; touching the
        // lines a few slots ahead overlaps those misses when a backlog exists.
        if ((p & 1) == 0) {
            __builtin_prefetch(base + ((p + 8) % (unsigned long long)r->depth), 0, 0);
            __builtin_prefetch(base + ((p + 16) % (unsigned long long)r->depth), 0, 0);
        }
        if (!read_slot(s, (uint32_t)(p + 1), out ? &out[n] : nullptr)) break;
        ++p;
        ++n;
    }
    if (n) {
        r->pos[c] = p;
        if (publish) __atomic_store_n(&r->host_tail[(size_t)c * kPad], p, __ATOMIC_RELEASE);
    }
    return n;
}

constexpr int kDrainBatch = 32;  // UCCL-EP s5.2 DRAIN_BATCH_SIZE

void proxy_loop(ep_ring_t* r, int first, int stride) {
    ep_transfer_cmd_t batch[kDrainBatch];
    int idle = 0;
    for (;;) {
        bool stopping = r->stop.load(std::memory_order_acquire);
        int64_t got = 0;
        for (int c = first; c < r->channels; c += stride) {
            int64_t n = pop_channel(r, c, batch, kDrainBatch, true);
            if (n) {
                got += n;
                r->drained.fetch_add(n, std::memory_order_relaxed);
                int64_t at = r->log_n.fetch_add(n, std::memory_order_relaxed);
                for (int64_t i = 0; i < n && at + i < r->log_capacity; ++i) r->log[at + i] = batch[i];
            }
        }
        if (got) {
            idle = 0;
            continue;
        }
        if (stopping) break;   // nothing left after the stop request
        if (++idle < 4096) {
            EP_CPU_RELAX();
        } else {
            std::this_thread::yield();
        }
    }
}

}  // namespace

extern "C" ep_ring_t* ep_ring_create(int32_t depth, int32_t channels, int32_t max_inflight,
                                     int64_t timeout_ns) {
    if (depth < 1 || depth > kMaxRingDepth || channels < 1 || channels > kMaxR ||
        max_inflight < 1 || max_inflight > depth || timeout_ns < 1)
        return nullptr;
    ep_ring_t* r = new (std::nothrow) ep_ring_t();
    if (!r) return nullptr;
    r->depth = depth;
    r->channels = channels;
    r->max_inflight = max_inflight;
    r->timeout_ns = timeout_ns;
    r->pos.assign(channels, 0);
    bool ok = hipGetDevice(&r->device) == hipSuccess;
    int rate_khz = 0;
    ok = ok && hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, r->device) ==
                   hipSuccess;
    if (ok) {
        if (rate_khz <= 0) rate_khz = 100000;   // s_memrealtime runs at 100 MHz on CDNA
        long double ticks = (long double)timeout_ns * rate_khz / 1.0e6L;
        r->timeout_ticks = ticks < 1 ? 1ull : (unsigned long long)ticks;
    }
    const size_t slot_bytes = (size_t)channels * depth * sizeof(RingSlot);
    const size_t tail_bytes = (size_t)channels * kPad * sizeof(unsigned long long);
    ok = ok && hipHostMalloc((void**)&r->slots, slot_bytes,
                             hipHostMallocCoherent | hipHostMallocMapped) == hipSuccess;
    ok = ok && hipHostMalloc((void**)&r->host_tail, tail_bytes,
                             hipHostMallocCoherent | hipHostMallocMapped) == hipSuccess;
    ok = ok && hipMalloc((void**)&r->dev_state, 3 * tail_bytes) == hipSuccess;
    if (ok) {
        std::memset(r->slots, 0, slot_bytes);
        std::memset(r->host_tail, 0, tail_bytes);
        ok = hipMemset(r->dev_state, 0, 3 * tail_bytes) == hipSuccess &&
             hipDeviceSynchronize() == hipSuccess;
    }
    if (!ok) {
        ep_ring_destroy(r);
        return nullptr;
    }
    return r;
}

extern "C" int ep_ring_destroy(ep_ring_t* r) {
    if (!r) return EP_ERR_INVALID_ARG;
    if (r->running.load()) ep_ring_proxy_stop(r, nullptr, 0, nullptr, nullptr);
    int st = EP_OK;
    if (r->slots && hipHostFree(r->slots) != hipSuccess) st = EP_ERR_HIP;
    if (r->host_tail && hipHostFree(r->host_tail) != hipSuccess) st = EP_ERR_HIP;
    if (r->dev_state && hipFree(r->dev_state) != hipSuccess) st = EP_ERR_HIP;
    delete r;
    return st;
}

extern "C" int ep_ring_reset(ep_ring_t* r) {
    if (!r) return EP_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> g(r->mu);
    if (r->running.load()) return EP_ERR_BUSY;
    std::memset(r->slots, 0, (size_t)r->channels * r->depth * sizeof(RingSlot));
    std::memset(r->host_tail, 0, (size_t)r->channels * kPad * sizeof(unsigned long long));
    std::fill(r->pos.begin(), r->pos.end(), 0ull);
    EP_HIP_CHECK(hipMemset(r->dev_state, 0, 3 * (size_t)r->channels * kPad * sizeof(unsigned long long)));
    EP_HIP_CHECK(hipDeviceSynchronize());
    return EP_OK;
}

extern "C" int ep_ring_drain(ep_ring_t* r, int32_t channel, ep_transfer_cmd_t* out, int32_t max,
                             int32_t* n_out) {
    if (!r || channel < 0 || channel >= r->channels || max < 0 || !n_out || (max > 0 && !out))
        return EP_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> g(r->mu);
    if (r->running.load()) return EP_ERR_BUSY;
    *n_out = (int32_t)pop_channel(r, channel, out, max, true);
    return EP_OK;
}

extern "C" int ep_ring_proxy_start(ep_ring_t* r, int32_t threads, int64_t log_capacity) {
    if (!r || threads < 1 || log_capacity < 0) return EP_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> g(r->mu);
    if (r->running.load()) return EP_ERR_BUSY;
    if (threads > r->channels) threads = r->channels;
    try {
        r->log.assign((size_t)log_capacity, ep_transfer_cmd_t{});
    } catch (...) {
        return EP_ERR_INVALID_ARG;
    }
    r->log_capacity = log_capacity;
    r->log_n.store(0);
    r->drained.store(0);
    r->stop.store(false);
    r->running.store(true);
    for (int i = 0; i < threads; ++i) r->threads.emplace_back(proxy_loop, r, i, threads);
    return EP_OK;
}

extern "C" int ep_ring_proxy_stop(ep_ring_t* r, ep_transfer_cmd_t* log_out, int64_t log_max,
                                  int64_t* n_logged, int64_t* n_drained) {
    if (!r) return EP_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> g(r->mu);
    if (!r->running.load()) return EP_ERR_INVALID_ARG;
    r->stop.store(true, std::memory_order_release);
    for (auto& t : r->threads) t.join();
    r->threads.clear();
    r->running.store(false);
    int64_t logged = r->log_n.load();
    if (logged > r->log_capacity) logged = r->log_capacity;
    if (log_out && log_max > 0) {
        int64_t n = logged < log_max ? logged : log_max;
        std::memcpy(log_out, r->log.data(), (size_t)n * sizeof(ep_transfer_cmd_t));
    }
    if (n_logged) *n_logged = logged;
    if (n_drained) *n_drained = r->drained.load();
    return EP_OK;
}

extern "C" int64_t ep_ring_proxy_drained(const ep_ring_t* r) {
    return r ? r->drained.load(std::memory_order_relaxed) : -1;
}
