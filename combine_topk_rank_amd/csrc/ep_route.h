// ep_route.h — device functions of the routing layout shared by the layout
// kernels and the one-kernel small-batch dispatch: a token's rank mask, the
// per-rank ballots of a wavefront's tokens, and a workgroup's exclusive scan.
#pragma once

#include "ep_common.h"

namespace ep {

// The k expert ids of token t (-1 past k, and for t >= T), all loads
// issued before any is used (one memory latency, not k).  KMAX >= k bounds
// the unrolled code: kernels built for k <= 8 carry a quarter of it.
template <int KMAX>
__device__ inline void load_token_ids(const int32_t* __restrict__ idx, int64_t t, int T, int k,
                                      int32_t (&ids)[KMAX]) {
    const int32_t* row = idx + t * k;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) ids[j] = (t < T && j < k) ? row[j] : -1;
}

// Owner rank e / epr of expert e in [0, E), by one float multiply instead of
// an integer division (a long dependent sequence of quarter-rate multiplies).
// Exact: E <= 4096 and R = E / epr <= 64, so the quotient (e + 1/2) / epr is
// at most 64 and lies at least 1/(2 epr) >= 2^-13 from every integer, while
// the float product, with inv_epr = 1/epr correctly rounded, is within
// 64 * 2^-23 = 2^-17 of it; truncation therefore gives floor(e / epr).
__device__ inline float inv_experts_per_rank(int epr) { return 1.0f / (float)epr; }
__device__ inline int rank_of_expert(int e, float inv_epr) {
    return (int)(((float)e + 0.5f) * inv_epr);
}

// Rank mask of a token from its ids; bad ids are reported (once per token)
// and skipped.  When `hist` is given, the token's valid experts are counted
// in it (LDS).
template <int KMAX>
__device__ inline uint64_t rank_mask_of(const int32_t (&ids)[KMAX], int E, int k, int epr,
                                        int32_t* st, int32_t* hist) {
    const float inv_epr = inv_experts_per_rank(epr);
    uint64_t m = 0;
    bool bad = false;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const int e = ids[j];
        if (j >= k || e == -1) continue;
        if ((unsigned)e >= (unsigned)E) {   // below -1, or E and above
            bad = true;
            continue;
        }
        m |= 1ull << rank_of_expert(e, inv_epr);
        if (hist) atomicAdd(&hist[e], 1);
    }
    if (bad) set_error(st, EP_ERR_BAD_EXPERT);
    return m;
}

// Rank mask of token t (0 for t >= T), as above, for k <= KMAX.
template <int KMAX>
__device__ inline uint64_t token_rank_mask(const int32_t* __restrict__ idx, int64_t t, int T,
                                           int E, int k, int epr, int32_t* st, int32_t* hist) {
    int32_t ids[KMAX];
    load_token_ids(idx, t, T, k, ids);
    return rank_mask_of(ids, E, k, epr, st, hist);
}

// Transpose of the wave's 64 x 64 bit matrix whose row l is lane l's
// `mask`: lane j receives the word whose bit i is bit j of lane i's mask
// (with lane = token and bit = rank, lane r gets the ballot of rank r; lanes
// past the highest rank get zero).  Six butterfly steps instead of one ballot
// per rank: at step s, lanes i and i ^ s (i without bit s) swap the
// off-diagonal blocks, i's bits at positions with bit s set against its
// partner's bits at positions with bit s clear.  One 32-bit shuffle per step:
// for s = 32 a lane sends the word its partner takes; below that, the 16 bits
// wanted of each half are packed into one word.  All lanes must be active.
__device__ inline uint64_t wave_bit_transpose(uint64_t mask) {
    const int lane = lane_id();
    uint32_t lo = (uint32_t)mask, hi = (uint32_t)(mask >> 32);
    {
        const bool up = (lane & 32) != 0;
        const uint32_t got = (uint32_t)__shfl_xor((int)(up ? lo : hi), 32);
        if (up)
            lo = got;
        else
            hi = got;
    }
#pragma unroll
    for (int step = 0; step < 5; ++step) {
        const int s = 16 >> step;
        // the positions with bit s clear
        const uint32_t m = step == 0 ? 0x0000FFFFu
                         : step == 1 ? 0x00FF00FFu
                         : step == 2 ? 0x0F0F0F0Fu
                         : step == 3 ? 0x33333333u
                                     : 0x55555555u;
        const bool up = (lane & s) != 0;
        const uint32_t send_lo = up ? (lo & m) : ((lo >> s) & m);
        const uint32_t send_hi = up ? (hi & m) : ((hi >> s) & m);
        const uint32_t got = (uint32_t)__shfl_xor((int)(send_lo | (send_hi << s)), s);
        const uint32_t glo = got & m, ghi = (got >> s) & m;
        if (up) {
            lo = glo | (lo & ~m);
            hi = ghi | (hi & ~m);
        } else {
            lo = (lo & m) | (glo << s);
            hi = (hi & m) | (ghi << s);
        }
    }
    return ((uint64_t)hi << 32) | lo;
}

// Per-wave rank ballots: bit i of ball_r = the wave's token i goes to rank r.
// Lane l ends up holding ball_{l mod R} (all lanes, so that every group of R
// lanes has the full set); lanes < R write their count to wcnt[r] and, when
// given, the ballot to ball[r].  The ballots are the transpose of the
// tokens' rank masks; one more shuffle gives lanes >= R the ballot of lane
// mod R.
__device__ inline uint64_t wave_rank_counts(uint64_t mask, int R, int32_t* wcnt,
                                            uint64_t* ball = nullptr) {
    const int lane = lane_id();
    uint64_t mine = wave_bit_transpose(mask);
    if (R < kWave) {
        const int src = lane % R;
        const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)mine, src);
        const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(mine >> 32), src);
        mine = ((uint64_t)hi << 32) | lo;
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
