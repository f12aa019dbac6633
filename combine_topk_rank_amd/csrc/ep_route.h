// ep_route.h — device functions of the routing layout shared by the layout
// kernels and the one-kernel small-batch dispatch: a token's rank mask, the
// per-rank ballots of a wavefront's tokens, and a workgroup's exclusive scan.
#pragma once

#include "ep_common.h"

namespace ep {

// The k expert ids of token t (-1 past k, and for t >= T), all loads
// issued before any is used (one memory latency, not k).
__device__ inline void load_token_ids(const int32_t* __restrict__ idx, int64_t t, int T, int k,
                                      int32_t (&ids)[kMaxK]) {
    const int32_t* row = idx + t * k;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) ids[j] = (t < T && j < k) ? row[j] : -1;
}

// Rank mask of a token from its ids; bad ids are reported and skipped.  When
// `hist` is given, the token's valid experts are counted in it (LDS).
__device__ inline uint64_t rank_mask_of(const int32_t (&ids)[kMaxK], int E, int k, int epr,
                                        int32_t* st, int32_t* hist) {
    uint64_t m = 0;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        const int e = ids[j];
        if (j >= k || e == -1) continue;
        if (e < -1 || e >= E) {
            set_error(st, EP_ERR_BAD_EXPERT);
            continue;
        }
        m |= 1ull << (e / epr);
        if (hist) atomicAdd(&hist[e], 1);
    }
    return m;
}

// Rank mask of token t (0 for t >= T), as above.
__device__ inline uint64_t token_rank_mask(const int32_t* __restrict__ idx, int64_t t, int T,
                                           int E, int k, int epr, int32_t* st, int32_t* hist) {
    int32_t ids[kMaxK];
    load_token_ids(idx, t, T, k, ids);
    return rank_mask_of(ids, E, k, epr, st, hist);
}

// Per-wave rank ballots: bit i of ball_r = the wave's token i goes to rank r.
// Lane l ends up holding ball_{l mod R} (all lanes, so that every group of R
// lanes has the full set); lanes < R write their count to wcnt[r] and, when
// given, the ballot to ball[r].
__device__ inline uint64_t wave_rank_counts(uint64_t mask, int R, int32_t* wcnt,
                                            uint64_t* ball = nullptr) {
    const int lane = lane_id();
    const int my_r = lane % R;
    uint64_t mine = 0;
    for (int r = 0; r < R; ++r) {
        const uint64_t b = __ballot((mask >> r) & 1ull);
        if (my_r == r) mine = b;
    }
    if (lane < R) {
        wcnt[lane] = (int32_t)__popcll(mine);
        if (ball) ball[lane] = mine;
    }
    return mine;
}

// Exclusive scan of n (<= kMaxE) ints held in LDS `v`, written to `out`
// (n+1 entries, out[n] = total).  All kBlock threads take part: each thread
// sums a contiguous run of `per` values, the 256 run sums are scanned with
// wavefront shuffles and a 4-entry scan of the wavefront totals.
__device__ inline void block_exclusive_scan_store(const int32_t* v, int n, int32_t* out,
                                                  int32_t* s_wtot) {
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int per = (n + kBlock - 1) / kBlock;
    const int b0 = tid * per;
    int32_t sum = 0;
    for (int i = 0; i < per; ++i)
        if (b0 + i < n) sum += v[b0 + i];
    int32_t incl = sum;
    for (int d = 1; d < kWave; d <<= 1) {
        int32_t o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    if (lane == kWave - 1) s_wtot[wave] = incl;
    __syncthreads();
    int32_t run = incl - sum;
    for (int w = 0; w < wave; ++w) run += s_wtot[w];
    if (tid == kBlock - 1) out[n] = run + sum;
    for (int i = 0; i < per; ++i) {
        if (b0 + i < n) {
            out[b0 + i] = run;
            run += v[b0 + i];
        }
    }
}

}  // namespace ep
