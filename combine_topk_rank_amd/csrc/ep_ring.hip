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
// There is no network here.  By default a proxy thread "executes" a command by
// logging it and marking it completed.  With a loopback target set, it
// executes it against local memory instead (UCCL-EP article s2.3: the proxy
// posts each WRITE and atomic; s2.2: completions are tracked per command):
// a WRITE becomes a device-to-device copy from the send buffer into the
// destination rank's receive region, an ATOMIC ADD an atomic add on the
// rank's count word, both on the proxy thread's own stream, so a channel's
// commands take effect in ticket order; a command is completed once its
// stream work has finished.  Slots are released (tail) when popped.

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstring>
#include <deque>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include <memory>

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
    unsigned long long* host_completed = nullptr;   // host-pinned, stride kPad: completed[c]
                                                    // mirrored for the GPU
    unsigned long long* dev_state = nullptr;   // device: head, tail_cache, poll; each [C*kPad]
    unsigned long long timeout_ticks = 0;
    // per channel, each on its own 64-byte line: proxy threads that serve
    // different channels never write the same line
    struct alignas(64) ChannelState {
        unsigned long long pos = 0;              // consumer position
        std::atomic<int64_t> completed{0};       // commands completed
    };
    std::unique_ptr<ChannelState[]> ch;
    std::mutex mu;                             // serialises host-side calls
    // proxy
    std::vector<std::thread> threads;
    std::atomic<bool> stop{false};
    std::atomic<bool> running{false};
    std::atomic<int64_t> drained{0};
    std::atomic<int64_t> log_n{0};
    int64_t log_capacity = 0;
    std::vector<ep_transfer_cmd_t> log;
    // loopback execution
    bool loopback = false;
    const uint8_t* lb_src = nullptr;
    uint64_t lb_src_bytes = 0;
    std::vector<uint8_t*> lb_dst;
    std::vector<uint64_t> lb_dst_bytes;
    std::vector<uint8_t*> lb_cnt;
    std::vector<uint64_t> lb_cnt_bytes;
    std::atomic<int64_t> lb_errors{0};
    std::atomic<int64_t> lb_done{0};
    std::atomic<int64_t> lb_lat_sum_ns{0};
    std::atomic<int64_t> lb_lat_max_ns{0};
    std::atomic<int64_t> lb_copies{0};
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
    d.completed = r->host_completed;
    d.depth = r->depth;
    d.channels = r->channels;
    d.max_inflight = r->max_inflight;
    d.timeout_ticks = r->timeout_ticks;
    return d;
}

}  // namespace ep

using namespace ep;

namespace {

// Pop up to `max` published commands of channel c (the slot format and the
// pop itself: ep_ring_proto.h); returns the number popped.
int64_t pop_channel(ep_ring_t* r, int c, ep_transfer_cmd_t* out, int64_t max, bool publish) {
    return ring_pop(r->slots + (size_t)c * r->depth, (uint32_t)r->depth, &r->ch[c].pos,
                    publish ? &r->host_tail[(size_t)c * kPad] : nullptr, out, max);
}

constexpr int kDrainBatch = 32;  // UCCL-EP s5.2 DRAIN_BATCH_SIZE

// One popped batch's copies and adds, passed by value in the kernel
// arguments (no staging memory).  Rows are 16-byte multiples at 16-byte
// offsets, so the copies move 16-byte vectors.
struct CopyList {
    const uint4* src[kDrainBatch];
    uint4* dst[kDrainBatch];
    uint64_t vecs[kDrainBatch];
    int32_t n;
};
struct AddList {
    int32_t* p[kDrainBatch];
    int32_t v[kDrainBatch];
    int32_t n;
};
constexpr int kCopyBlocksPerEntry = 16;

__global__ __launch_bounds__(256) void loopback_copy(CopyList l) {
    const int e = blockIdx.x / kCopyBlocksPerEntry;
    const int part = blockIdx.x % kCopyBlocksPerEntry;
    if (e >= l.n) return;
    const uint4* src = l.src[e];
    uint4* dst = l.dst[e];
    const uint64_t n = l.vecs[e];
    for (uint64_t i = (uint64_t)part * 256 + threadIdx.x; i < n; i += kCopyBlocksPerEntry * 256)
        dst[i] = src[i];
}

__global__ void loopback_add(AddList l) {
    if ((int)threadIdx.x < l.n) atomicAdd(l.p[threadIdx.x], l.v[threadIdx.x]);
}

// Count n more commands of channel c as completed, and publish the new
// count where the GPU can read it (one writer per channel at a time: the
// proxy thread serving it, or ep_ring_drain while no proxy runs).
void add_completed(ep_ring_t* r, int c, int64_t n) {
    const int64_t v = r->ch[c].completed.fetch_add(n, std::memory_order_release) + n;
    __atomic_store_n(&r->host_completed[(size_t)c * kPad], (unsigned long long)v, __ATOMIC_RELEASE);
}

// One thread per queried command: 1 if complete, 0 if not, 2 for a channel
// outside the ring.
__global__ void check_completion_kernel(RingDev g, const int32_t* channels,
                                        const uint64_t* tickets, int32_t n, uint8_t* done) {
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i >= n) return;
    const int c = channels[i];
    done[i] = (c < 0 || c >= g.channels) ? 2 : (ring_check_completion(g, c, tickets[i]) ? 1 : 0);
}

int64_t now_ns() {
    return std::chrono::duration_cast<std::chrono::nanoseconds>(
               std::chrono::steady_clock::now().time_since_epoch())
        .count();
}

// Work of one popped batch in flight on a proxy thread's stream.
struct Pending {
    hipEvent_t ev;
    int c;
    int64_t n;
    int64_t t_pop;
};

// Execute a popped batch against the loopback target on `stream`: one copy
// kernel for its WRITEs (a WRITE that continues the previous one of the same
// rank joins its entry), then one add kernel for its ATOMICs, so every count
// lands after the rows popped with or before it.  Commands outside the
// registered regions are skipped and counted as errors (still completed).
void execute_batch(ep_ring_t* r, const ep_transfer_cmd_t* b, int64_t n, hipStream_t stream) {
    CopyList cl{};
    AddList al{};
    uint64_t last_src = 0, last_dst = 0, last_end = ~0ull;
    uint32_t last_rank = ~0u;
    for (int64_t i = 0; i < n; ++i) {
        const ep_transfer_cmd_t& d = b[i];
        const uint32_t rank = d.dst_rank;
        if (rank >= r->lb_dst.size()) {
            r->lb_errors.fetch_add(1);
            continue;
        }
        if (d.type == EP_CMD_WRITE) {
            const uint64_t src = d.src_offset, dst = d.dst_offset, size = d.size_or_value;
            if (src + size > r->lb_src_bytes || dst + size > r->lb_dst_bytes[rank] ||
                !r->lb_dst[rank] || (src | dst | size) % 16 != 0) {
                r->lb_errors.fetch_add(1);
                last_rank = ~0u;
                continue;
            }
            if (cl.n > 0 && rank == last_rank && src == last_src + (last_end - last_dst) &&
                dst == last_end) {
                cl.vecs[cl.n - 1] += size / 16;   // continues the previous entry
                last_end += size;
                continue;
            }
            cl.src[cl.n] = reinterpret_cast<const uint4*>(r->lb_src + src);
            cl.dst[cl.n] = reinterpret_cast<uint4*>(r->lb_dst[rank] + dst);
            cl.vecs[cl.n] = size / 16;
            ++cl.n;
            last_rank = rank;
            last_src = src;
            last_dst = dst;
            last_end = dst + size;
        } else if (d.type == EP_CMD_ATOMIC && d.op == EP_ATOMIC_ADD) {
            if (d.dst_offset % 4 != 0 || d.dst_offset + 4 > r->lb_cnt_bytes[rank] ||
                !r->lb_cnt[rank]) {
                r->lb_errors.fetch_add(1);
                continue;
            }
            al.p[al.n] = reinterpret_cast<int32_t*>(r->lb_cnt[rank] + d.dst_offset);
            al.v[al.n] = (int32_t)d.size_or_value;
            ++al.n;
        } else {
            r->lb_errors.fetch_add(1);
        }
    }
    if (cl.n) {
        hipLaunchKernelGGL(loopback_copy, dim3(cl.n * kCopyBlocksPerEntry), dim3(256), 0, stream,
                           cl);
        if (hipGetLastError() != hipSuccess) r->lb_errors.fetch_add(cl.n);
        else r->lb_copies.fetch_add(cl.n);
    }
    if (al.n) {
        hipLaunchKernelGGL(loopback_add, dim3(1), dim3(kDrainBatch), 0, stream, al);
        if (hipGetLastError() != hipSuccess) r->lb_errors.fetch_add(al.n);
    }
}

void finish(ep_ring_t* r, const Pending& p) {
    add_completed(r, p.c, p.n);
    r->lb_done.fetch_add(p.n);
    const int64_t lat = now_ns() - p.t_pop;
    r->lb_lat_sum_ns.fetch_add(lat * p.n);
    int64_t m = r->lb_lat_max_ns.load();
    while (lat > m && !r->lb_lat_max_ns.compare_exchange_weak(m, lat)) {
    }
}

void proxy_loop(ep_ring_t* r, int first, int stride) {
    ep_transfer_cmd_t batch[kDrainBatch];
    hipStream_t stream = nullptr;
    std::vector<hipEvent_t> free_ev;
    std::deque<Pending> pending;
    if (r->loopback) {
        (void)hipSetDevice(r->device);
        if (hipStreamCreateWithFlags(&stream, hipStreamNonBlocking) != hipSuccess) stream = nullptr;
    }
    int idle = 0;
    for (;;) {
        bool stopping = r->stop.load(std::memory_order_acquire);
        int64_t got = 0;
        for (int c = first; c < r->channels; c += stride) {
            int64_t n = pop_channel(r, c, batch, kDrainBatch, true);
            if (n) {
                const int64_t t_pop = now_ns();
                got += n;
                r->drained.fetch_add(n, std::memory_order_relaxed);
                if (r->log_capacity > 0) {
                    const int64_t at = r->log_n.fetch_add(n, std::memory_order_relaxed);
                    for (int64_t i = 0; i < n && at + i < r->log_capacity; ++i)
                        r->log[at + i] = batch[i];
                }
                if (stream) {
                    execute_batch(r, batch, n, stream);
                    hipEvent_t ev = nullptr;
                    if (!free_ev.empty()) {
                        ev = free_ev.back();
                        free_ev.pop_back();
                    } else if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
                        ev = nullptr;
                    }
                    if (ev && hipEventRecord(ev, stream) == hipSuccess) {
                        pending.push_back({ev, c, n, t_pop});
                    } else {
                        (void)hipStreamSynchronize(stream);
                        finish(r, Pending{nullptr, c, n, t_pop});
                        if (ev) free_ev.push_back(ev);
                    }
                } else {
                    add_completed(r, c, n);
                }
            }
        }
        // completions, in order
        while (!pending.empty() && hipEventQuery(pending.front().ev) == hipSuccess) {
            finish(r, pending.front());
            free_ev.push_back(pending.front().ev);
            pending.pop_front();
        }
        if (got) {
            idle = 0;
            continue;
        }
        if (stopping && pending.empty()) break;   // nothing left after the stop request
        if (++idle < 4096) {
            EP_CPU_RELAX();
        } else {
            std::this_thread::yield();
        }
    }
    for (hipEvent_t ev : free_ev) (void)hipEventDestroy(ev);
    if (stream) (void)hipStreamDestroy(stream);
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
    r->ch.reset(new (std::nothrow) ep_ring::ChannelState[channels]);
    if (!r->ch) {
        delete r;
        return nullptr;
    }
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
    ok = ok && hipHostMalloc((void**)&r->host_completed, tail_bytes,
                             hipHostMallocCoherent | hipHostMallocMapped) == hipSuccess;
    ok = ok && hipMalloc((void**)&r->dev_state, 3 * tail_bytes) == hipSuccess;
    if (ok) {
        std::memset(r->slots, 0, slot_bytes);
        std::memset(r->host_tail, 0, tail_bytes);
        std::memset(r->host_completed, 0, tail_bytes);
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
    if (r->host_completed && hipHostFree(r->host_completed) != hipSuccess) st = EP_ERR_HIP;
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
    std::memset(r->host_completed, 0, (size_t)r->channels * kPad * sizeof(unsigned long long));
    for (int c = 0; c < r->channels; ++c) {
        r->ch[c].pos = 0;
        r->ch[c].completed.store(0);
    }
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
    add_completed(r, channel, *n_out);
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

extern "C" int ep_ring_set_loopback(ep_ring_t* r, const void* src, uint64_t src_bytes, int32_t R,
                                    void* const* dst, const uint64_t* dst_bytes,
                                    void* const* counts, const uint64_t* count_bytes) {
    if (!r || R < 0 || R > kMaxR) return EP_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> g(r->mu);
    if (r->running.load()) return EP_ERR_BUSY;
    if (!src) {   // back to log-only draining
        r->loopback = false;
        r->lb_src = nullptr;
        r->lb_dst.clear();
        r->lb_dst_bytes.clear();
        r->lb_cnt.clear();
        r->lb_cnt_bytes.clear();
        return EP_OK;
    }
    if (R < 1 || !dst || !dst_bytes || !counts || !count_bytes) return EP_ERR_INVALID_ARG;
    r->lb_src = reinterpret_cast<const uint8_t*>(src);
    r->lb_src_bytes = src_bytes;
    r->lb_dst.assign(R, nullptr);
    r->lb_dst_bytes.assign(R, 0);
    r->lb_cnt.assign(R, nullptr);
    r->lb_cnt_bytes.assign(R, 0);
    for (int i = 0; i < R; ++i) {
        r->lb_dst[i] = reinterpret_cast<uint8_t*>(dst[i]);
        r->lb_dst_bytes[i] = dst[i] ? dst_bytes[i] : 0;
        r->lb_cnt[i] = reinterpret_cast<uint8_t*>(counts[i]);
        r->lb_cnt_bytes[i] = counts[i] ? count_bytes[i] : 0;
    }
    r->lb_errors.store(0);
    r->lb_done.store(0);
    r->lb_lat_sum_ns.store(0);
    r->lb_lat_max_ns.store(0);
    r->lb_copies.store(0);
    r->loopback = true;
    return EP_OK;
}

extern "C" int64_t ep_ring_completed(const ep_ring_t* r, int32_t channel) {
    if (!r || channel < 0 || channel >= r->channels) return -1;
    return r->ch[channel].completed.load(std::memory_order_acquire);
}

extern "C" int ep_ring_check_completion(const ep_ring_t* r, const int32_t* channels,
                                        const uint64_t* tickets, int32_t n, uint8_t* done,
                                        hipStream_t stream) {
    if (!r || n < 0 || (n > 0 && (!channels || !tickets || !done))) return EP_ERR_INVALID_ARG;
    if (n == 0) return EP_OK;
    clear_hip_error();
    hipLaunchKernelGGL(check_completion_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0,
                       stream, ring_device_view(const_cast<ep_ring_t*>(r)), channels, tickets, n,
                       done);
    EP_HIP_CHECK(hipGetLastError());
    return EP_OK;
}

extern "C" int ep_ring_wait_complete(ep_ring_t* r, int64_t timeout_ns) {
    if (!r || timeout_ns < 0) return EP_ERR_INVALID_ARG;
    // every command published so far: the producers' ticket counters
    std::vector<unsigned long long> head((size_t)r->channels * kPad);
    EP_HIP_CHECK(hipMemcpy(head.data(), r->dev_state, head.size() * sizeof(unsigned long long),
                           hipMemcpyDeviceToHost));
    const int64_t t0 = now_ns();
    for (;;) {
        bool done = true;
        for (int c = 0; c < r->channels && done; ++c)
            done = r->ch[c].completed.load(std::memory_order_acquire) >=
                   (int64_t)head[(size_t)c * kPad];
        if (done) break;
        if (now_ns() - t0 > timeout_ns) return EP_ERR_RING_TIMEOUT;
        std::this_thread::yield();
    }
    return r->lb_errors.load() ? EP_ERR_INVALID_ARG : EP_OK;
}

extern "C" int ep_ring_loopback_stats(const ep_ring_t* r, int64_t* n_done, int64_t* n_errors,
                                      int64_t* n_copies, double* mean_latency_us,
                                      double* max_latency_us) {
    if (!r) return EP_ERR_INVALID_ARG;
    const int64_t n = r->lb_done.load();
    if (n_done) *n_done = n;
    if (n_errors) *n_errors = r->lb_errors.load();
    if (n_copies) *n_copies = r->lb_copies.load();
    if (mean_latency_us) *mean_latency_us = n ? r->lb_lat_sum_ns.load() / 1e3 / n : 0.0;
    if (max_latency_us) *max_latency_us = r->lb_lat_max_ns.load() / 1e3;
    return EP_OK;
}
