// ep_combine.hip — combine: gather the expert outputs returned to this GPU and
// take the gate-weighted sum per token (UCCL-EP article s6, EP combine; GPU
// communication notes s5, DeepEP combine).
//
// The returned rows y sit in the dispatch layout: y[send_slot[t,r]] is what
// rank r sends back for token t, already summed over r's experts of t.  Its
// weight is W[t,r], the sum of t's gate weights on r:
//   out[t,:] = bf16_rne( sum_{r ascending, send_slot[t,r] >= 0}
//                          W[t,r] * y[send_slot[t,r], :] )
// accumulated in float registers with fma; W adds in ascending j.
//
// Work decomposition: wavefront g handles chunk g % nchunks of token
// g / nchunks (16-byte loads of 8 bf16 per lane per vector); each returned row
// is read once and each output row written once.

#include "ep_common.h"

namespace ep {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Below this many wavefronts in the default layout, combine switches to
// short chunks with eight rows in flight per wavefront.
constexpr int64_t kCombineSmallWaves = 2048;

struct CombineArgs {
    const u32x4* y;            // [P, H/8] (per-expert mode: [Q, H/8])
    const int32_t* idx;        // [T, k]
    const float* w;            // [T, k]
    const int32_t* send_slot;  // [T, R] (per-expert mode: expert_slot [T, k])
    u32x4* out;                // [T, H/8]
    int32_t* st;
    int64_t y_rows;
    int32_t T, E, R, k, epr;
    int32_t nv;
    int32_t nchunks;
};

__device__ inline uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;  // NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ inline uint32_t pack2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// B destination rows are loaded before any of them is accumulated (memory
// parallelism within a wavefront); accumulation stays in ascending rank order
// (per-expert mode, LL: ascending choice order).
//
// Per-expert mode (UCCL-EP article s4.1, low-latency mode): the rows sit in
// the per-expert layout, row expert_slot[t,j] holding expert e_j's output for
// token t, and
//   out[t,:] = bf16_rne( sum_{j ascending, e_j kept} w[t,j] * y[expert_slot[t,j], :] ).
template <int VPL, int B, bool LL>
__global__ __launch_bounds__(kBlock) void combine_kernel(CombineArgs a) {
    const int lane = lane_id();
    const int64_t gw = (int64_t)blockIdx.x * (kBlock / kWave) + (threadIdx.x / kWave);
    const int64_t t = gw / a.nchunks;
    const int chunk = (int)(gw - t * a.nchunks);
    if (t >= a.T) return;

    int32_t s_lane = -1;
    float W = 0.0f;
    if (LL) {
        // lane j: choice j's row and gate
        if (lane < a.k) {
            const int e = a.idx[t * a.k + lane];
            if (e >= 0 && e < a.E) {
                s_lane = a.send_slot[t * a.k + lane];
                W = a.w[t * a.k + lane];
            }
        }
    } else {
        if (lane < a.R) s_lane = a.send_slot[t * a.R + lane];
        // W for lane r: gate weights of t's experts on rank r, ascending j
        int e_l = -1;
        float w_l = 0.0f;
        if (lane < a.k) {
            e_l = a.idx[t * a.k + lane];
            w_l = a.w[t * a.k + lane];
        }
        // e / epr == lane, for e in [0, E), without a division
        const int first_e = lane * a.epr;
        for (int j = 0; j < a.k; ++j) {
            const int e = bcast(e_l, j);
            const float wj = bcastf(w_l, j);
            if (e >= 0 && e < a.E && (unsigned)(e - first_e) < (unsigned)a.epr) W += wj;
        }
    }
    if (s_lane >= a.y_rows) {
        set_error(a.st, EP_ERR_CAPACITY);   // a slot beyond the rows of y: skipped
        s_lane = -1;
    }
    const uint64_t dmask = __ballot(s_lane >= 0);

    const int v0 = chunk * VPL * kWave;
    float acc[VPL][8];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[i][q] = 0.0f;

    for (uint64_t m = dmask; m;) {
        int32_t ss[B];
        float ww[B];
        int nb = 0;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            ss[b] = 0;
            ww[b] = 0.0f;
            if (m) {
                const int r = __builtin_ctzll(m);
                m &= m - 1;
                ss[b] = bcast(s_lane, r);
                ww[b] = bcastf(W, r);
                nb = b + 1;
            }
        }
        u32x4 v[B][VPL];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const u32x4* yr = a.y + (int64_t)ss[b] * a.nv;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int vi = v0 + lane + i * kWave;
                v[b][i] = (b < nb && vi < a.nv) ? __builtin_nontemporal_load(yr + vi)
                                                : u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (b >= nb) break;
            const float Wr = ww[b];
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const u32x4 u = v[b][i];
                acc[i][0] = fmaf(Wr, __uint_as_float(u.x << 16), acc[i][0]);
                acc[i][1] = fmaf(Wr, __uint_as_float(u.x & 0xFFFF0000u), acc[i][1]);
                acc[i][2] = fmaf(Wr, __uint_as_float(u.y << 16), acc[i][2]);
                acc[i][3] = fmaf(Wr, __uint_as_float(u.y & 0xFFFF0000u), acc[i][3]);
                acc[i][4] = fmaf(Wr, __uint_as_float(u.z << 16), acc[i][4]);
                acc[i][5] = fmaf(Wr, __uint_as_float(u.z & 0xFFFF0000u), acc[i][5]);
                acc[i][6] = fmaf(Wr, __uint_as_float(u.w << 16), acc[i][6]);
                acc[i][7] = fmaf(Wr, __uint_as_float(u.w & 0xFFFF0000u), acc[i][7]);
            }
        }
    }

    u32x4* orow = a.out + t * a.nv;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        int vi = v0 + lane + i * kWave;
        if (vi < a.nv) {
            u32x4 o;
            o.x = pack2(acc[i][0], acc[i][1]);
            o.y = pack2(acc[i][2], acc[i][3]);
            o.z = pack2(acc[i][4], acc[i][5]);
            o.w = pack2(acc[i][6], acc[i][7]);
            __builtin_nontemporal_store(o, orow + vi);
        }
    }
}

}  // namespace ep

using namespace ep;

namespace {
template <int VPL, int B, bool LL>
int launch_combine(const CombineArgs& a, int64_t waves, hipStream_t stream) {
    const int64_t blocks = ceil_div(waves, kBlock / kWave);
    clear_hip_error();
    hipLaunchKernelGGL((combine_kernel<VPL, B, LL>), dim3((unsigned)blocks), dim3(kBlock), 0,
                       stream, a);
    EP_HIP_CHECK(hipGetLastError());
    return EP_OK;
}

// Large batches: rows wider than 512 vectors take 4 vectors per lane (four
// wavefronts per 7168-wide row) with four rows in flight per wavefront; 7
// vectors and one row in flight, 7 and two, 8 and one, 2 and four all
// measured the same or slower (train 86-88 us, skewed 275 against 280-286 us).
// Small batches (few wavefronts): 1-2 vectors per lane and eight rows in
// flight, so each wavefront does not wait on its token's rows one after
// another.
template <bool LL>
int launch_combine_any(CombineArgs& a, hipStream_t stream) {
    const int vpl_big = a.nv <= 64 ? 1 : a.nv <= 128 ? 2 : a.nv <= 256 ? 4 : a.nv <= 512 ? 8 : 4;
    const int64_t waves_big = (int64_t)a.T * ceil_div(a.nv, (int64_t)vpl_big * kWave);
    if (waves_big < kCombineSmallWaves) {
        const int vpl = a.nv <= 64 ? 1 : 2;
        a.nchunks = (int32_t)ceil_div(a.nv, (int64_t)vpl * kWave);
        const int64_t waves = (int64_t)a.T * a.nchunks;
        return vpl == 1 ? launch_combine<1, 8, LL>(a, waves, stream)
                        : launch_combine<2, 8, LL>(a, waves, stream);
    }
    a.nchunks = (int32_t)ceil_div(a.nv, (int64_t)vpl_big * kWave);
    const int64_t waves = (int64_t)a.T * a.nchunks;
    switch (vpl_big) {
        case 1: return launch_combine<1, 4, LL>(a, waves, stream);
        case 2: return launch_combine<2, 4, LL>(a, waves, stream);
        case 4: return launch_combine<4, 4, LL>(a, waves, stream);
        default: return launch_combine<8, 1, LL>(a, waves, stream);
    }
}
}  // namespace

extern "C" int ep_combine(const ep_shape_t* shape, const void* y, int64_t y_rows,
                          const int32_t* topk_idx, const float* topk_w, const int32_t* send_slot,
                          void* out, int32_t* dev_status, hipStream_t stream) {
    int v = validate_shape(shape);
    if (v != EP_OK) return v;
    const ep_shape_t s = *shape;
    if (!dev_status) return EP_ERR_INVALID_ARG;
    if (s.T == 0) return EP_OK;
    if (y_rows < 0 || (y_rows > 0 && !y) || !topk_idx || !topk_w || !send_slot || !out)
        return EP_ERR_INVALID_ARG;
    if (((uintptr_t)y | (uintptr_t)out) & 15) return EP_ERR_INVALID_ARG;
    CombineArgs a{};
    a.y = reinterpret_cast<const u32x4*>(y);
    a.idx = topk_idx;
    a.w = topk_w;
    a.send_slot = send_slot;
    a.out = reinterpret_cast<u32x4*>(out);
    a.st = dev_status;
    a.y_rows = y_rows;
    a.T = s.T;
    a.E = s.E;
    a.R = s.R;
    a.k = s.k;
    a.epr = s.E / s.R;
    a.nv = s.H / 8;
    return launch_combine_any<false>(a, stream);
}

extern "C" int ep_combine_ll(const ep_shape_t* shape, const void* y, int64_t y_rows,
                             const int32_t* topk_idx, const float* topk_w,
                             const int32_t* expert_slot, void* out, int32_t* dev_status,
                             hipStream_t stream) {
    int v = validate_shape(shape);
    if (v != EP_OK) return v;
    const ep_shape_t s = *shape;
    if (!dev_status) return EP_ERR_INVALID_ARG;
    if (s.T == 0) return EP_OK;
    if (y_rows < 0 || (y_rows > 0 && !y) || !topk_idx || !topk_w || !expert_slot || !out)
        return EP_ERR_INVALID_ARG;
    if (((uintptr_t)y | (uintptr_t)out) & 15) return EP_ERR_INVALID_ARG;
    CombineArgs a{};
    a.y = reinterpret_cast<const u32x4*>(y);
    a.idx = topk_idx;
    a.w = topk_w;
    a.send_slot = expert_slot;
    a.out = reinterpret_cast<u32x4*>(out);
    a.st = dev_status;
    a.y_rows = y_rows;
    a.T = s.T;
    a.E = s.E;
    a.R = s.R;
    a.k = s.k;
    a.epr = s.E / s.R;
    a.nv = s.H / 8;
    return launch_combine_any<true>(a, stream);
}
