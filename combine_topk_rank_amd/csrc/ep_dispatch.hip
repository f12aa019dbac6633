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
// token g / nchunks.  It reads its chunk of x once (16-byte loads), and stores
// it to every destination slot of the token (16-byte stores; 8-byte stores of
// codes for fp8), so x is read once and the packed rows written once.  A
// message is the <= 8 consecutive rows [o_r + 8m, ...) of rank r; those rows
// come from different tokens, hence different wavefronts.  Each wavefront
// makes its stores visible system-wide (release fence) and then counts itself
// into the message's arrival counter; the last arrival publishes the WRITE.
// The last WRITE of a rank is followed by that rank's ATOMIC (its row count),
// reserved after every WRITE ticket of the rank, so the proxy, which pops in
// ticket order, sees the count after the rows.

#include "ep_common.h"

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
    int32_t* rank_msgs_done;      // [R]
    int32_t* st;
    RingDev ring;
    int64_t max_msgs;             // entries of msg_arrivals
    int64_t cap;
    int64_t row_bytes;
    int32_t T, H, E, R, k, epr;
    int32_t nv;                   // 16-byte vectors per x row (H/8)
    int32_t nchunks;              // wavefronts per token
    int32_t has_ring;
    int64_t ngroups;              // groups of kPackWaves wavefronts
};

// ------------------------------------------------------------------ ring

// Write one command into its slot: four tagged 8-byte words in two plain
// 16-byte stores.  The caller makes them visible to the CPU with one
// system-scope release per round of writes (see ring_publish); the tags make
// the order in which the words land irrelevant.  The rows the command points
// to were released at system scope before the command's ticket was taken.
__device__ inline void ring_write(const RingDev& g, int c, unsigned long long ticket, uint32_t type,
                                  uint32_t op, uint32_t ntok, uint32_t dst_rank, uint32_t size_val,
                                  uint64_t src_off, uint64_t dst_off) {
    RingSlot* slot = g.slots + (size_t)c * g.depth + (size_t)(ticket % (unsigned long long)g.depth);
    const uint64_t tag = (uint64_t)((ticket + 1) & 0xFFFFull);
    const uint64_t w0 = tag | ((uint64_t)(type & 0xFF) << 16) | ((uint64_t)(op & 0xFF) << 24) |
                        ((uint64_t)(ntok & 0xFFFF) << 32);
    const uint64_t w1 = tag | ((uint64_t)(dst_rank & 0xFFFF) << 16) | ((uint64_t)size_val << 32);
    const uint64_t w2 = tag | ((src_off & kMaxRingOffset) << 16);
    const uint64_t w3 = tag | ((dst_off & kMaxRingOffset) << 16);
    u64x2* p = reinterpret_cast<u64x2*>(slot);
    p[0] = u64x2{w0, w1};
    p[1] = u64x2{w2, w3};
}

// Reserve n consecutive tickets on channel c (one atomic per reservation).
__device__ inline unsigned long long ring_reserve(const RingDev& g, int c, unsigned n) {
    return atomicAdd(g.head + (size_t)c * kPad, (unsigned long long)n);
}

// One command per lane (lanes with `have`): wait until the lane's ticket may
// be written -- fewer than max_inflight commands of its channel published but
// not yet drained -- write it, and release it at system scope.  The wait and the write share one
// wave-uniform loop, so a lane whose ticket is ready writes at once even while
// other lanes of the wavefront still wait (their tickets may wait on it).
// A lane gives up when the ring's timeout passes (status set) or when another
// producer has already failed.
__device__ void ring_publish(const RingDev& g, bool have, int c, unsigned long long ticket,
                             uint32_t type, uint32_t op, uint32_t ntok, uint32_t dst_rank,
                             uint32_t size_val, uint64_t src_off, uint64_t dst_off, int32_t* st) {
    if (!__ballot(have)) return;
    const unsigned long long lim = (unsigned long long)g.max_inflight;
    unsigned long long* cache = g.tail_cache + (size_t)c * kPad;
    unsigned long long* poll = g.poll + (size_t)c * kPad;
    const unsigned long long* htail = g.host_tail + (size_t)c * kPad;
    unsigned long long seen = 0, t0 = 0;
    bool pending = have;
    bool polled = false;
    if (pending) seen = __hip_atomic_load(cache, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (__ballot(pending)) {
        bool progress = false;
        if (pending) {
            if (ticket >= seen + lim) {
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
            if (ticket < seen + lim) {
                ring_write(g, c, ticket, type, op, ntok, dst_rank, size_val, src_off, dst_off);
                pending = false;
                progress = true;
            } else if (read_status(st) != 0) {
                pending = false;
            } else {
                const unsigned long long now = __builtin_amdgcn_s_memrealtime();
                if (!polled) {
                    polled = true;
                    t0 = now;
                } else if (now - t0 > g.timeout_ticks) {
                    set_error(st, EP_ERR_RING_TIMEOUT);
                    pending = false;
                }
            }
        }
        if (__ballot(progress)) {
            // one system-scope release pushes this round's slots out of the
            // L2 to host memory, where the proxy polls them
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
        } else if (__ballot(pending)) {
            __builtin_amdgcn_s_sleep(16);
        }
    }
}

// ATOMIC{ADD, cnt} for ranks that receive no rows (nothing to order after).
__device__ void publish_empty_ranks(const PackArgs& a) {
    const int lane = lane_id();
    bool have = false;
    int c = 0;
    unsigned long long tk = 0;
    if (lane < a.R && a.rank_off[lane + 1] == a.rank_off[lane]) {
        have = true;
        c = lane % a.ring.channels;
        tk = ring_reserve(a.ring, c, 1);
    }
    ring_publish(a.ring, have, c, tk, EP_CMD_ATOMIC, EP_ATOMIC_ADD, 0, (uint32_t)lane, 0, 0, 0,
                 a.st);
}

// Lane r of a wavefront that wrote (one chunk of) the row in slot s of rank r
// (`mine`), after the wavefront's release fence: count the row into its
// message; the last arrival of a message publishes the WRITE, and the last
// WRITE of a rank is followed by the rank's ATOMIC.  All lanes of the
// wavefront call this together.
__device__ void arrive_and_publish(const PackArgs& a, bool mine, int r, int32_t s) {
    bool pub = false;
    int32_t o = 0, cnt = 0, m = 0, nrows = 0;
    if (mine) {
        o = a.rank_off[r];
        cnt = a.rank_off[r + 1] - o;
        m = (s - o) / kMsgRows;
        nrows = min(kMsgRows, cnt - m * kMsgRows);
        const int32_t gm = a.msg_base[r] + m;
        if (s < o || s >= o + cnt || gm < 0 || gm >= a.max_msgs) {
            // send_slot does not belong to rank_offset: not from the same layout
            set_error(a.st, EP_ERR_INVALID_ARG);
        } else {
            const int32_t old = atomicAdd(&a.msg_arrivals[gm], 1);
            if (old == nrows * a.nchunks - 1) {
                pub = true;
                a.msg_arrivals[gm] = 0;   // every arrival is in: leave the counter clean
            }
        }
    }
    if (!__ballot(pub)) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const int c = r % a.ring.channels;
    unsigned long long tk = 0;
    bool ok = false;
    if (pub) {
        ok = read_status(a.st) == 0;
        tk = ring_reserve(a.ring, c, 1);
    }
    const uint64_t rb = (uint64_t)a.row_bytes;
    ring_publish(a.ring, pub && ok, c, tk, EP_CMD_WRITE, 0, (uint32_t)nrows, (uint32_t)r,
                 (uint32_t)(nrows * rb), (uint64_t)(o + m * kMsgRows) * rb,
                 (uint64_t)(m * kMsgRows) * rb, a.st);
    // count the message into its rank only after its WRITE ticket exists: the
    // added value depends on the ticket, so the two atomics cannot reorder
    bool pub_a = false;
    if (pub) {
        const int32_t nmsgs = (cnt + kMsgRows - 1) / kMsgRows;
        const int32_t one = 1 + (int32_t)(tk >> 62);
        const int32_t done = atomicAdd(&a.rank_msgs_done[r], one);
        if (done == nmsgs - 1) {
            pub_a = true;
            a.rank_msgs_done[r] = 0;
        }
    }
    unsigned long long tka = 0;
    bool ok_a = false;
    if (pub_a) {
        ok_a = read_status(a.st) == 0;
        tka = ring_reserve(a.ring, c, 1);
    }
    ring_publish(a.ring, pub_a && ok_a, c, tka, EP_CMD_ATOMIC, EP_ATOMIC_ADD, 0, (uint32_t)r,
                 (uint32_t)cnt, 0, 0, a.st);
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
// bit pattern (finite values).
__device__ inline uint32_t max_bf16_mag(uint32_t a, uint32_t b) {
    const uint32_t a0 = a & 0x7FFFu, a1 = (a >> 16) & 0x7FFFu;
    const uint32_t b0 = b & 0x7FFFu, b1 = (b >> 16) & 0x7FFFu;
    const uint32_t x = a0 > a1 ? a0 : a1;
    const uint32_t y = b0 > b1 ? b0 : b1;
    return x > y ? x : y;
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
// Vectors per lane for rows of up to 896 vectors (H = 7168): 14 = one
// wavefront per row, 7 = two.
constexpr int kPackVplH7168 = 14;
constexpr int kPackVplFp8H7168 = 14;
// Pack workgroups per compute unit, at most: with fewer workgroups than
// groups, each workgroup loops, so rows complete (and descriptors are
// published) in several generations instead of all at the end of the kernel.
// Half the compute units already saturate HBM with 16 wavefronts each.
constexpr int kPackGridPerCuNum = 1, kPackGridPerCuDen = 2;

template <int VPL, int FMT, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void pack_kernel(PackArgs a) {
    constexpr int kWaves = WAVES;
    __shared__ int32_t s_pair_slot[kWaves][kMaxR];
    __shared__ int32_t s_pair_rank[kWaves][kMaxR];
    __shared__ int32_t s_npairs[kWaves];
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);
    const int64_t P = a.rank_off[a.R];
    const bool cap_ok = P <= a.cap;
    if (blockIdx.x == 0 && wave == 0) {
        if (!cap_ok && lane == 0) set_error(a.st, EP_ERR_CAPACITY);
        if (a.has_ring && cap_ok) publish_empty_ranks(a);
    }
    // groups of kWaves wavefronts, taken in launch order; a workgroup that
    // finishes a group (rows, then descriptors) moves on to the next one
    for (int64_t grp = blockIdx.x; grp < a.ngroups; grp += gridDim.x) {
    const int64_t gw = grp * kWaves + wave;
    const int64_t t = gw / a.nchunks;
    const int chunk = (int)(gw - t * a.nchunks);
    const bool active = t < a.T;   // wavefront-uniform

    int32_t s_lane = -1;
    uint64_t dmask = 0;
    if (active) {
        if (lane < a.R) s_lane = a.send_slot[t * a.R + lane];
        dmask = __ballot(s_lane >= 0);

        // load this wavefront's chunk of the row: vectors v0 + lane + 64 i
        const int v0 = chunk * VPL * kWave;
        const u32x4* xr = a.x + t * a.nv;
        u32x4 v[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            int vi = v0 + lane + i * kWave;
            if (vi < a.nv) v[i] = xr[vi];
            else v[i] = u32x4{0, 0, 0, 0};
        }

        if (FMT == EP_FMT_BF16) {
            for (uint64_t m = dmask; m; m &= m - 1) {
                const int r = __builtin_ctzll(m);
                const int32_t s = bcast(s_lane, r);
                if (s >= a.cap) continue;
                u32x4* dst = reinterpret_cast<u32x4*>(a.send_buf + (int64_t)s * a.row_bytes);
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    int vi = v0 + lane + i * kWave;
                    if (vi < a.nv) __builtin_nontemporal_store(v[i], dst + vi);
                }
            }
        } else {
            // quantise once: per 128-element block, a = max(amax, 1e-4),
            // codes = e4m3(x * (448 / a)), scale = a / 448.  The block max is
            // taken on the bf16 bits: magnitudes of finite values order like
            // unsigned integers, so no float copy of the row stays live.
            u32x2 q[VPL];
            float scale[VPL];
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const u32x4 u = v[i];
                const uint32_t m01 = max_bf16_mag(u.x, u.y);
                const uint32_t m23 = max_bf16_mag(u.z, u.w);
                const uint32_t mw = m01 > m23 ? m01 : m23;
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
            }
            for (uint64_t m = dmask; m; m &= m - 1) {
                const int r = __builtin_ctzll(m);
                const int32_t s = bcast(s_lane, r);
                if (s >= a.cap) continue;
                uint8_t* row = a.send_buf + (int64_t)s * a.row_bytes;
                u32x2* codes = reinterpret_cast<u32x2*>(row);
                float* scales = reinterpret_cast<float*>(row + a.H);
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    int vi = v0 + lane + i * kWave;
                    if (vi < a.nv) {
                        __builtin_nontemporal_store(q[i], codes + vi);
                        if ((lane & 15) == 0) __builtin_nontemporal_store(scale[i], scales + vi / 16);
                    }
                }
            }
        }

        // per-slot metadata, written by the token's first chunk
        if (chunk == 0) {
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
                    const bool local = e >= 0 && e < a.E && e / a.epr == r;
                    a.slot_local_idx[(int64_t)s * a.k + lane] = local ? e - r * a.epr : -1;
                    a.slot_local_w[(int64_t)s * a.k + lane] = local ? wt : 0.0f;
                }
                if (lane == 0) a.slot_src[s] = (int32_t)t;
            }
        }
    }

    if (!(a.has_ring && cap_ok)) continue;   // uniform over the workgroup
    // hand this wavefront's (slot, rank) pairs to wavefront 0
    if ((dmask >> lane) & 1ull) {
        const int j = lane_prefix(dmask);
        s_pair_slot[wave][j] = s_lane;
        s_pair_rank[wave][j] = lane;
    }
    if (lane == 0) s_npairs[wave] = (int32_t)__popcll(dmask);
    __syncthreads();
    if (wave == 0) {
        // One system-scope release for the rows and metadata of the whole
        // group (ordered after the other wavefronts' stores by the barrier),
        // then the arrivals and the descriptors.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
        int total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) total += s_npairs[w];
        for (int base = 0; base < total; base += kWave) {
            int p = base + lane;
            const bool mine = p < total;
            int r = 0;
            int32_t s = 0;
            if (mine) {
                int w = 0;
                while (p >= s_npairs[w]) {
                    p -= s_npairs[w];
                    ++w;
                }
                s = s_pair_slot[w][p];
                r = s_pair_rank[w][p];
            }
            arrive_and_publish(a, mine, r, s);
        }
    }
    __syncthreads();   // the pair lists are reused by the next group
    }
}

}  // namespace ep

using namespace ep;

namespace {

int64_t pack_grid_cap() {
    static int64_t cap = 0;   // per process; the library targets one GPU model
    if (cap == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cap = (int64_t)cus * kPackGridPerCuNum / kPackGridPerCuDen;
        if (cap < 1) cap = 1;
    }
    return cap;
}

template <int VPL>
int launch_pack(PackArgs a, int fmt, int64_t waves, hipStream_t stream) {
    // fp8 holds the codes and scales too: half the wavefronts per workgroup
    // keep its registers (a 1024-thread workgroup caps a lane at 128)
    const int wg_waves = fmt == EP_FMT_BF16 ? kPackWaves : kPackWavesFp8;
    a.ngroups = ceil_div(waves, wg_waves);
    const int64_t cap = pack_grid_cap() * (kPackWaves / wg_waves);
    const int64_t blocks = a.ngroups < cap ? a.ngroups : cap;
    clear_hip_error();
    if (fmt == EP_FMT_BF16)
        hipLaunchKernelGGL((pack_kernel<VPL, EP_FMT_BF16, kPackWaves>), dim3((unsigned)blocks),
                           dim3(kPackWaves * kWave), 0, stream, a);
    else
        hipLaunchKernelGGL((pack_kernel<VPL, EP_FMT_FP8_E4M3_B128, kPackWavesFp8>),
                           dim3((unsigned)blocks), dim3(kPackWavesFp8 * kWave), 0, stream, a);
    EP_HIP_CHECK(hipGetLastError());
    return EP_OK;
}

}  // namespace

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
    a.rank_msgs_done = w.rank_msgs_done;
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

    // vectors per lane: one pass over the row when it fits (bf16: 16 per
    // lane); fp8 also holds the codes and scales, so it takes at most 8
    int vpl;
    if (a.nv <= 64) vpl = 1;
    else if (a.nv <= 128) vpl = 2;
    else if (a.nv <= 256) vpl = 4;
    else if (a.nv <= 512) vpl = 8;
    else if (s.fmt != EP_FMT_BF16) vpl = a.nv <= 896 ? kPackVplFp8H7168 : 8;
    else if (a.nv <= 896) vpl = kPackVplH7168;
    else vpl = 16;
    a.nchunks = (int32_t)ceil_div(a.nv, (int64_t)vpl * kWave);
    int64_t waves = (int64_t)s.T * a.nchunks;
    if (waves == 0) {
        if (!a.has_ring) return EP_OK;
        waves = 1;   // the zero-count ATOMICs still go out
    }
    switch (vpl) {
        case 1: return launch_pack<1>(a, s.fmt, waves, stream);
        case 2: return launch_pack<2>(a, s.fmt, waves, stream);
        case 4: return launch_pack<4>(a, s.fmt, waves, stream);
        case 8: return launch_pack<8>(a, s.fmt, waves, stream);
        case 7: return launch_pack<7>(a, s.fmt, waves, stream);
        case 14: return launch_pack<14>(a, s.fmt, waves, stream);
        default: return launch_pack<16>(a, s.fmt, waves, stream);
    }
}
