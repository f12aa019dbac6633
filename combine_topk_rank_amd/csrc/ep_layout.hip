// ep_layout.hip — routing layout (per-rank and per-expert histograms, offsets,
// stable send slots) for one GPU's share of an EP group.
//
// A token is sent once to every rank that owns one of its top-k experts
// (NCCL GIN article, s3.1.1 device-side token routing; UCCL-EP article, s1
// token-level exchange); expert e lives on rank e / (E/R).  Rank r's rows are
// [o_r, o_{r+1}) in ascending token order, so the slot of (t, r) is
// o_r + #{t' < t routed to r}: a stable compaction over T x R bits.  It is
// computed with wavefront ballots (64-lane, UCCL-EP s5.1) and integer prefix
// sums only, so the result never depends on scheduling order.
//
// Two passes when T spans several 256-token tiles:
//   layout_count_kernel : per tile, rank counts (ballot + popcount per rank)
//                         and an LDS expert histogram -> workspace;
//   layout_main_kernel  : per tile, prefix over the earlier tiles' counts,
//                         then the slots of its tokens.  Tile 0 also writes
//                         the counts, offsets and message bases.
// When every tile can be resident at once, both passes run in one kernel
// (layout_main_kernel<2>) whose tiles meet at a grid barrier instead of a
// kernel boundary; one workgroup does everything when T fits one tile.
// With several tiles, the second pass has one workgroup more than there are
// tiles: it sums the tiles' expert histograms and scans them, in parallel
// with the tiles' slot stores, so no tile carries the expert work.

#include <atomic>

#include "ep_common.h"
#include "ep_route.h"

namespace ep {

// Column totals of the [nrows, R] int32 matrix m (the tiles' rank counts,
// nrows >= 1) and its sums over rows < split, for lanes < R of wavefront 0
// (*tot, *pre; other threads get zeros).  Lane c < R of wavefront w adds
// column c over rows w, w + 4, ..., kColBatch loads in flight at a time (one
// memory latency for up to 4 * kColBatch rows); wavefront 0 then adds the
// four partials from LDS (part_tot, part_pre: kBlock entries each).  Loads
// past the last row re-read it and count nothing, so no load is predicated;
// every load is coalesced and no LDS atomic is involved.  Contains a
// workgroup barrier.
constexpr int kColBatch = 8;
__device__ inline void rank_column_sums(const int32_t* __restrict__ m, int nrows, int R, int split,
                                        int32_t* part_tot, int32_t* part_pre, int32_t* tot,
                                        int32_t* pre) {
    constexpr int NW = kBlock / kWave;
    const int lane = lane_id(), w = threadIdx.x / kWave;
    if (lane < R) {
        int32_t st = 0, sp = 0;
        for (int r0 = w; r0 < nrows; r0 += kColBatch * NW) {
            int32_t q[kColBatch];
#pragma unroll
            for (int u = 0; u < kColBatch; ++u)
                q[u] = m[(int64_t)min(r0 + u * NW, nrows - 1) * R + lane];
#pragma unroll
            for (int u = 0; u < kColBatch; ++u) {
                const int r = r0 + u * NW;
                st += r < nrows ? q[u] : 0;
                sp += r < split ? q[u] : 0;
            }
        }
        part_tot[w * kWave + lane] = st;
        part_pre[w * kWave + lane] = sp;
    }
    __syncthreads();
    int32_t a = 0, p = 0;
    if (w == 0 && lane < R) {
#pragma unroll
        for (int h = 0; h < NW; ++h) {
            a += part_tot[h * kWave + lane];
            p += part_pre[h * kWave + lane];
        }
    }
    *tot = a;
    *pre = p;
}

// Totals of the [nrows, ncols] int32 matrix m over its rows, one column per
// thread (consecutive threads read consecutive columns, so every load is
// coalesced), 16 rows in flight per thread; into LDS acc[ncols].
// Each column of m is replaced by its exclusive prefix over the rows (row i:
// the sum of rows < i), which the per-expert row table reads.
__device__ inline void column_totals(int32_t* __restrict__ m, int nrows, int ncols,
                                     int32_t* acc) {
    constexpr int kRows = 16;
    for (int c = threadIdx.x; c < ncols; c += kBlock) {
        int32_t sum = 0;
        for (int r0 = 0; r0 < nrows; r0 += kRows) {
            int32_t q[kRows];
#pragma unroll
            for (int u = 0; u < kRows; ++u)
                q[u] = r0 + u < nrows ? m[(int64_t)(r0 + u) * ncols + c] : 0;
#pragma unroll
            for (int u = 0; u < kRows; ++u) {
                if (r0 + u < nrows) m[(int64_t)(r0 + u) * ncols + c] = sum;
                sum += q[u];
            }
        }
        acc[c] = sum;
    }
}

__device__ inline void zero_counters(int32_t* p, int64_t n, int64_t first, int64_t stride) {
    for (int64_t i = first; i < n; i += stride) p[i] = 0;
}

template <int KMAX>
__global__ __launch_bounds__(kBlock) void layout_count_kernel(
    const int32_t* __restrict__ idx, int T, int E, int R, int k, int epr,
    int32_t* __restrict__ blk_rank_cnt, int32_t* __restrict__ blk_exp_cnt,
    int32_t* __restrict__ counters, int64_t counters_n, int32_t* st) {
    __shared__ int32_t s_hist[kMaxE];
    __shared__ int32_t s_wcnt[kBlock / kWave][kMaxR];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int64_t t = (int64_t)blockIdx.x * kLayoutTile + tid;
    int32_t ids[KMAX];
    load_token_ids(idx, t, T, k, ids);   // in flight while the histogram clears
    for (int e = tid; e < E; e += kBlock) s_hist[e] = 0;
    __syncthreads();
    uint64_t mask = rank_mask_of(ids, E, k, epr, st, s_hist);
    wave_rank_counts(mask, R, s_wcnt[wave]);
    __syncthreads();
    if (tid < R) {
        int32_t c = 0;
        for (int w = 0; w < kBlock / kWave; ++w) c += s_wcnt[w][tid];
        blk_rank_cnt[(int64_t)blockIdx.x * R + tid] = c;
    }
    for (int e = tid; e < E; e += kBlock) blk_exp_cnt[(int64_t)blockIdx.x * E + e] = s_hist[e];
    zero_counters(counters, counters_n, (int64_t)blockIdx.x * kBlock + tid,
                  (int64_t)gridDim.x * kBlock);
}

// MODE 0: one tile (the whole layout in one workgroup).
// MODE 1: second pass after layout_count_kernel.
// MODE 2: both passes in one kernel, the tiles meeting at a grid barrier
//         (used only when every tile can be resident at once).
// In modes 1 and 2 the grid has nblocks + 1 workgroups: workgroup nblocks
// owns no tokens and computes the expert totals and offsets.
template <int MODE, int KMAX>
__global__ __launch_bounds__(kBlock) void layout_main_kernel(
    const int32_t* __restrict__ idx, int T, int E, int R, int k, int epr, int nblocks,
    int32_t* __restrict__ blk_rank_cnt, int32_t* __restrict__ blk_exp_cnt,
    int32_t* __restrict__ cnt_rank, int32_t* __restrict__ cnt_exp,
    int32_t* __restrict__ rank_off, int32_t* __restrict__ exp_off, int32_t* __restrict__ msg_base,
    uint8_t* __restrict__ in_rank, int32_t* __restrict__ send_slot,
    int32_t* __restrict__ counters, int64_t counters_n, uint32_t* __restrict__ bar,
    int32_t* st) {
    constexpr bool SINGLE = MODE == 0;
    constexpr bool FUSED = MODE == 2;
    __shared__ int32_t s_hist[(SINGLE || FUSED) ? kMaxE : 1];
    __shared__ int32_t s_exp[kMaxE];
    __shared__ int32_t s_wcnt[kBlock / kWave][kMaxR];
    __shared__ int32_t s_base[kMaxR];    // first slot of rank r in this tile
    __shared__ int32_t s_part[kBlock];
    __shared__ int32_t s_part2[kBlock];
    __shared__ uint64_t s_ball[kBlock / kWave][kMaxR];   // per-wave rank ballots
    __shared__ int32_t s_wbase[kBlock / kWave][kMaxR];   // first slot of rank r in the wave
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int b = blockIdx.x;
    // the extra workgroup of modes 1 and 2: expert totals and offsets only
    const bool expert_wg = !SINGLE && b == nblocks;
    // the barrier's generation, loaded now so that its latency overlaps the
    // counting (thread 0 only)
    uint32_t gen = 0;
    if (FUSED && tid == 0) gen = grid_barrier_generation(bar);

    const int64_t t_first = (int64_t)b * kLayoutTile;
    const int64_t t = t_first + tid;
    // the token's expert ids are requested first, so that their latency
    // overlaps the clearing of the histogram (the expert workgroup's tokens
    // are all past T: nothing is loaded there)
    int32_t ids[KMAX];
    load_token_ids(idx, t, T, k, ids);
    if (SINGLE || FUSED) {
        for (int e = tid; e < E; e += kBlock) s_hist[e] = 0;
        __syncthreads();
    }
    uint64_t mask = 0, my_ball = 0;
    if (!expert_wg) {
        mask = rank_mask_of(ids, E, k, epr, st, (SINGLE || FUSED) ? s_hist : nullptr);
        my_ball = wave_rank_counts(mask, R, s_wcnt[wave], s_ball[wave]);
    }
    __syncthreads();

    if (FUSED) {
        // first pass: this tile's counts for the others, then meet them
        if (!expert_wg) {
            if (tid < R) {
                int32_t c = 0;
                for (int w = 0; w < kBlock / kWave; ++w) c += s_wcnt[w][tid];
                blk_rank_cnt[(int64_t)b * R + tid] = c;
            }
            for (int e = tid; e < E; e += kBlock)
                blk_exp_cnt[(int64_t)b * E + e] = s_hist[e];
        }
        if (!grid_barrier<false>(bar, (uint32_t)gridDim.x, st, gen)) return;
        // the dispatch's message counters start at zero; cleared after the
        // barrier so that its wait for this workgroup's stores does not
        // include them (the kernel's end completes them)
        zero_counters(counters, counters_n, (int64_t)b * kBlock + tid, (int64_t)gridDim.x * kBlock);
    }

    if (expert_wg) {
        // per-expert totals of all tiles and their exclusive scan
        column_totals(blk_exp_cnt, nblocks, E, s_exp);
        __syncthreads();
        for (int e = tid; e < E; e += kBlock) cnt_exp[e] = s_exp[e];
        block_exclusive_scan_store(s_exp, E, exp_off, s_part);
        return;
    }

    // rank totals and the prefix over earlier tiles, in lanes < R of wave 0
    int32_t my_tot = 0, my_pre = 0;
    if (SINGLE) {
        if (tid < R)
            for (int w = 0; w < kBlock / kWave; ++w) my_tot += s_wcnt[w][tid];
    } else {
        rank_column_sums(blk_rank_cnt, nblocks, R, b, s_part, s_part2, &my_tot, &my_pre);
    }
    if (wave == 0) {
        // exclusive scan of the rank totals across lanes (R <= 64)
        int32_t tot = lane < R ? my_tot : 0;
        int32_t msgs = (tot + kMsgRows - 1) / kMsgRows;
        int32_t incl = tot, mincl = msgs;
        for (int d = 1; d < kWave; d <<= 1) {
            int32_t o = __shfl_up(incl, d);
            int32_t mo = __shfl_up(mincl, d);
            if (lane >= d) {
                incl += o;
                mincl += mo;
            }
        }
        int32_t off = incl - tot;
        if (lane < R) s_base[lane] = off + my_pre;
        if (b == 0) {
            if (lane < R) {
                cnt_rank[lane] = tot;
                rank_off[lane] = off;
                msg_base[lane] = mincl - msgs;
            }
            if (lane == R - 1) {
                rank_off[R] = incl;
                msg_base[R] = mincl;
            }
        }
    }
    __syncthreads();

    // slots in closed form: for the wave's token i and rank r,
    //   slot = (first slot of r in this wave) + popcount(ball[r] below bit i)
    // The wave's rows of send_slot / is_token_in_rank are one contiguous
    // block of n*R entries, written with 16-byte stores by all lanes.
    if (lane < R) {
        int32_t run = s_base[lane];
        for (int w = 0; w < wave; ++w) run += s_wcnt[w][lane];
        s_wbase[wave][lane] = run;
    }
    __syncthreads();
    const int64_t t_wave = t_first + (int64_t)wave * kWave;
    const int n = (int)max((int64_t)0, min((int64_t)kWave, (int64_t)T - t_wave));   // tokens in this wave
    const int64_t nel = (int64_t)n * R;
    const uint64_t* ball = s_ball[wave];
    const int32_t* wbase = s_wbase[wave];
    int32_t* slot_out = send_slot + t_wave * R;
    uint8_t* in_out = in_rank + t_wave * R;
    if ((R & 3) == 0 && (kWave % R) == 0) {
        // R in {4, 8, 16, 32, 64}: lane l serves ranks r0 .. r0+3, r0 =
        // 4 (l mod R/4), of tokens l / (R/4), l / (R/4) + 256 / R, ...: per
        // token one 16-byte slot store and one 4-byte flag store, the wave's
        // lanes covering 64 * 16 consecutive bytes of send_slot per store.
        // The lane's four ballots and bases stay in registers throughout.
        const int q = R >> 2;          // lanes per token
        const int step = kWave / q;    // tokens per pass of the wave
        const int r0 = (lane % q) * 4;
        uint64_t bl[4];
        int32_t wb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            bl[u] = ball[r0 + u];
            wb[u] = wbase[r0 + u];
        }
        for (int i = lane / q; i < n; i += step) {
            const uint64_t below = (1ull << i) - 1ull;   // i < 64
            int32_t v[4];
            uint32_t bytes = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t bit = (uint32_t)(bl[u] >> i) & 1u;
                v[u] = bit ? wb[u] + (int32_t)__popcll(bl[u] & below) : -1;
                bytes |= bit << (8 * u);
            }
            *reinterpret_cast<int4*>(slot_out + (int64_t)i * R + r0) = int4{v[0], v[1], v[2], v[3]};
            *reinterpret_cast<uint32_t*>(in_out + (int64_t)i * R + r0) = bytes;
        }
    } else if ((kWave % R) == 0) {
        // R = 1 or 2: lane l serves rank l % R of token (j * 64 + l) / R,
        // so each store covers 64 consecutive entries; the ballot and base
        // are already in the lane's registers.
        const int G = kWave / R;
        const int my_r = lane % R;
        const int my_g = lane / R;
        const int32_t my_base = s_wbase[wave][my_r];
        for (int j = 0; j * G < n; ++j) {
            const int i = j * G + my_g;
            if (i < n) {
                const int bit = (int)((my_ball >> i) & 1ull);
                const int32_t sl =
                    bit ? my_base + (int32_t)__popcll(my_ball & ((1ull << i) - 1ull)) : -1;
                slot_out[j * kWave + lane] = sl;
                in_out[j * kWave + lane] = (uint8_t)bit;
            }
        }
    } else {
    // (t_wave * R) % 4 == 0 because kWave * R is a multiple of 4: 4-entry groups
    for (int g = lane; g * 4 < (int)nel; g += kWave) {
        int32_t v[4];
        uint32_t bytes = 0;
        int i = (g * 4) / R;            // token of the group's first entry
        int r = g * 4 - i * R;          // its rank
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            int32_t sl = -1;
            if (g * 4 + q < (int)nel) {
                const uint64_t br = ball[r];
                if ((br >> i) & 1ull) {
                    sl = wbase[r] + (int32_t)__popcll(br & ((1ull << i) - 1ull));
                    bytes |= 1u << (8 * q);
                }
            }
            v[q] = sl;
            if (++r == R) {
                r = 0;
                ++i;
            }
        }
        if (g * 4 + 4 <= nel) {
            *reinterpret_cast<int4*>(slot_out + g * 4) = int4{v[0], v[1], v[2], v[3]};
            *reinterpret_cast<uint32_t*>(in_out + g * 4) = bytes;
        } else {
            for (int q = 0; q < 4 && g * 4 + q < nel; ++q) {
                slot_out[g * 4 + q] = v[q];
                in_out[g * 4 + q] = (uint8_t)((bytes >> (8 * q)) & 1u);
            }
        }
    }
    }
    if (SINGLE) {
        // per-expert totals and their exclusive scan, while the slot stores
        // complete
        for (int e = tid; e < E; e += kBlock) {
            s_exp[e] = s_hist[e];
            cnt_exp[e] = s_hist[e];
        }
        __syncthreads();
        block_exclusive_scan_store(s_exp, E, exp_off, s_part);
        zero_counters(counters, counters_n, tid, kBlock);
    }
}

// ------------------------------------------------------------ per-expert mode
// Row of every kept choice in the per-expert layout (UCCL-EP article s4.1,
// low-latency mode: tokens go per expert; NCCL GIN article s3.1.1: each to
// its expert's owner):
//   expert_slot[t,j] = expert_offset[e] + #{kept (t',j') < (t,j) with e' = e}
// in (t, j) order, e = topk_idx[t,j], or -1 for a dropped (or bad) choice.
//
// One wavefront per 64 tokens.  Its base per expert is expert_offset, plus
// the counts of the earlier 256-token tiles (the layout leaves their
// per-tile prefix in the workspace: one row to read), plus the choices of the
// earlier 64-token groups of its own tile (counted from topk_idx).  Inside the wavefront, every lane sets its
// bit in an LDS mask per expert it names (64-bit atomic OR); a choice's place
// among the same expert's choices of lower lanes is the popcount of that mask
// below the lane.  A token naming an expert o+1 times takes part in o+1
// rounds (round o: the masks of lanes with more than o such choices), so
// repeats count once per choice.  No atomic decides an order: deterministic.
__global__ __launch_bounds__(kWave) void ll_slot_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k,
    const int32_t* __restrict__ blk_exp_pre, const int32_t* __restrict__ exp_off,
    int32_t* __restrict__ expert_slot, int32_t* st) {
    __shared__ int32_t s_base[kMaxE];
    __shared__ unsigned long long s_mask[kMaxE];
    const int lane = threadIdx.x;
    const int64_t q = blockIdx.x;                       // 64-token group
    const int64_t tile = q / (kLayoutTile / kWave);      // its 256-token tile
    const int64_t t_tile = tile * kLayoutTile;
    const int64_t t = q * kWave + lane;
    // this lane's choices: all loads issued before any is used
    int32_t ids[kMaxK];
    const int32_t* row = idx + t * k;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) ids[j] = (j < k && t < T) ? row[j] : -1;
    for (int e = lane; e < E; e += kWave) {
        s_base[e] = 0;
        s_mask[e] = 0ull;
    }
    __syncthreads();
    // earlier tiles: the layout left, per tile, the exclusive prefix of the
    // tiles' expert counts
    if (tile > 0)
        for (int e = lane; e < E; e += kWave) s_base[e] = blk_exp_pre[tile * (int64_t)E + e];
    __syncthreads();
    // earlier 64-token groups of this tile, from topk_idx
    {
        const int64_t n = (q * kWave - t_tile) * k;   // choices before this group in the tile
        const int32_t* base = idx + t_tile * k;
        constexpr int kBatch = 8;
        for (int64_t i0 = lane; i0 < n; i0 += (int64_t)kWave * kBatch) {
            int32_t v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int64_t i = i0 + (int64_t)u * kWave;
                v[u] = i < n ? base[i] : -1;
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                if (v[u] >= 0 && v[u] < E) atomicAdd(&s_base[v[u]], 1);
        }
    }
    __syncthreads();
    for (int e = lane; e < E; e += kWave) s_base[e] += exp_off[e];
    // validate; occurrence of each choice among the lane's earlier choices
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        if (ids[j] < -1 || ids[j] >= E) {
            set_error(st, EP_ERR_BAD_EXPERT);
            ids[j] = -1;
        }
    }
    int32_t occ[kMaxK];
    int my_rounds = 0;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        int o = 0;
        if (j < k) {
#pragma unroll
            for (int i = 0; i < j; ++i) o += (ids[i] == ids[j]) ? 1 : 0;
        }
        occ[j] = o;
        if (ids[j] >= 0 && o + 1 > my_rounds) my_rounds = o + 1;
    }
    int rounds = my_rounds;
    for (int d = 1; d < kWave; d <<= 1) rounds = max(rounds, __shfl_xor(rounds, d));
    const unsigned long long below = (1ull << lane) - 1ull;
    int32_t pos[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) pos[j] = occ[j];
    __syncthreads();
    for (int o = 0; o < rounds; ++o) {
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (ids[j] >= 0 && occ[j] == o) atomicOr(&s_mask[ids[j]], 1ull << lane);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (ids[j] >= 0) pos[j] += __popcll(s_mask[ids[j]] & below);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (ids[j] >= 0) s_mask[ids[j]] = 0ull;
        __syncthreads();
    }
    if (t < T) {
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j >= k) break;
            expert_slot[t * k + j] = ids[j] >= 0 ? s_base[ids[j]] + pos[j] : -1;
        }
    }
}

// ------------------------------------------------ per-expert layout, one kernel
// Counts, offsets and the row table of the per-expert mode in one launch
// (the rank layout is not needed there).  Tiles of 256 tokens, one wavefront
// per 64 tokens, E <= kLLLayoutMaxE:
//   1. each wavefront counts its choices per expert in LDS; the tile stores
//      its histogram to a [NB, E] table;
//   2. grid barrier (every tile resident);
//   3. every tile sums the table's columns: the expert totals (their
//      exclusive scan is expert_offset) and the rows of each expert in the
//      earlier tiles;
//   4. a choice's row is expert_offset[e] + (earlier tiles) + (earlier
//      wavefronts of the tile) + (earlier choices of e in its wavefront, in
//      (t, j) order), the last from per-wavefront LDS masks as in
//      ll_slot_kernel.
// Integer counts only: the rows do not depend on scheduling order.
constexpr int kLLLayoutMaxE = 1024;

template <int KMAX>
__global__ __launch_bounds__(kBlock) void ll_layout_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k, int nblocks,
    int32_t* __restrict__ blk_exp_cnt, int32_t* __restrict__ cnt_exp,
    int32_t* __restrict__ exp_off, int32_t* __restrict__ expert_slot,
    int32_t* __restrict__ counters, int64_t counters_n, uint32_t* __restrict__ bar,
    int32_t* st) {
    constexpr int kW = kBlock / kWave;
    __shared__ int32_t s_whist[kW][kLLLayoutMaxE];             // choices per expert, per wavefront
    __shared__ unsigned long long s_mask[kW][kLLLayoutMaxE];   // one round's lanes per expert
    __shared__ int32_t s_base[kLLLayoutMaxE];                  // offset + earlier tiles
    __shared__ int32_t s_tot[kLLLayoutMaxE];
    __shared__ int32_t s_wsum[kW];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int b = blockIdx.x;
    uint32_t gen = 0;
    if (tid == 0) gen = grid_barrier_generation(bar);
    // this lane's token: its choices, all loads issued first
    const int64_t t = (int64_t)b * kLayoutTile + tid;
    int32_t ids[KMAX];
    {
        const int32_t* row = idx + t * k;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) ids[j] = (j < k && t < T) ? row[j] : -1;
    }
    for (int e = lane; e < E; e += kWave) {
        s_whist[wave][e] = 0;
        s_mask[wave][e] = 0ull;
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
        if (ids[j] < -1 || ids[j] >= E) {
            set_error(st, EP_ERR_BAD_EXPERT);
            ids[j] = -1;
        }
    // occurrence of each choice among the token's earlier choices
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
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
        if (ids[j] >= 0) atomicAdd(&s_whist[wave][ids[j]], 1);
    __syncthreads();
    // 1. the tile's histogram for the others (the per-wavefront counts become
    // their exclusive prefix over the wavefronts, which step 4 reads); the
    // dispatch's counters start at zero
    for (int e = tid; e < E; e += kBlock) {
        int32_t c = 0;
#pragma unroll
        for (int w = 0; w < kW; ++w) {
            const int32_t h = s_whist[w][e];
            s_whist[w][e] = c;
            c += h;
        }
        blk_exp_cnt[(int64_t)b * E + e] = c;
    }
    zero_counters(counters, counters_n, (int64_t)b * kBlock + tid, (int64_t)gridDim.x * kBlock);
    // 2. every tile's histogram is in the table after this
    if (!grid_barrier<false>(bar, (uint32_t)gridDim.x, st, gen)) return;
    // 3. column sums: totals, and the rows in earlier tiles (32 rows in
    // flight per thread; loads past the last row re-read it and count
    // nothing, so none is predicated)
    constexpr int kRows = 32;
    for (int e = tid; e < E; e += kBlock) {
        int32_t tot = 0, pre = 0;
        for (int r0 = 0; r0 < nblocks; r0 += kRows) {
            int32_t q[kRows];
#pragma unroll
            for (int u = 0; u < kRows; ++u)
                q[u] = blk_exp_cnt[(int64_t)min(r0 + u, nblocks - 1) * E + e];
#pragma unroll
            for (int u = 0; u < kRows; ++u) {
                tot += r0 + u < nblocks ? q[u] : 0;
                pre += r0 + u < b ? q[u] : 0;
            }
        }
        s_tot[e] = tot;
        s_base[e] = pre;
    }
    __syncthreads();
    // exclusive scan of the totals: thread tid takes a run of `per` experts
    {
        const int per = (E + kBlock - 1) / kBlock;
        const int e0 = tid * per;
        int32_t sum = 0;
        for (int i = 0; i < per; ++i)
            if (e0 + i < E) sum += s_tot[e0 + i];
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
            const int e = e0 + i;
            if (e < E) {
                if (b == 0) {
                    cnt_exp[e] = s_tot[e];
                    exp_off[e] = run;
                }
                s_base[e] += run;
                run += s_tot[e];
            }
        }
        if (b == 0 && tid == kBlock - 1) exp_off[E] = run;
    }
    __syncthreads();
    // 4. rows: base + earlier wavefronts of the tile + earlier lanes (rounds
    // by occurrence, as in ll_slot_kernel) + earlier choices of the token
    int32_t pos[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        pos[j] = occ[j];
        if (ids[j] >= 0) pos[j] += s_base[ids[j]] + s_whist[wave][ids[j]];
    }
    // The rounds are the wavefront's own (its masks are its own LDS rows):
    // their count is the wavefront's maximum, and a wavefront-scope fence
    // between the steps orders them (a wavefront's LDS operations complete
    // in order), so no workgroup barrier is needed.
    const unsigned long long below = (1ull << lane) - 1ull;
    int rounds = my_rounds;
    for (int d = 1; d < kWave; d <<= 1) rounds = max(rounds, __shfl_xor(rounds, d));
    for (int o = 0; o < rounds; ++o) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (ids[j] >= 0 && occ[j] == o) atomicOr(&s_mask[wave][ids[j]], 1ull << lane);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (ids[j] >= 0) pos[j] += __popcll(s_mask[wave][ids[j]] & below);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (ids[j] >= 0) s_mask[wave][ids[j]] = 0ull;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
    if (t < T) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j >= k) break;
            expert_slot[t * k + j] = ids[j] >= 0 ? pos[j] : -1;
        }
    }
}

// Tiles of the one-kernel per-expert layout that can be resident at once (per
// process; threads that race to fill it compute the same value), or 0.
template <int KMAX>
int64_t max_resident_ll_tiles() {
    static std::atomic<int64_t> cached{-1};
    int64_t v = cached.load(std::memory_order_relaxed);
    if (v < 0) {
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void*>(ll_layout_kernel<KMAX>), kBlock, 0) ==
                hipSuccess)
            v = (int64_t)cus * per_cu;
        else
            v = 0;
        cached.store(v, std::memory_order_relaxed);
    }
    return v;
}

// Tiles of the one-kernel layout that can be resident at once on the current
// device (workgroups per CU from the occupancy calculator x CUs), or 0.
template <int KMAX>
int64_t max_resident_layout_tiles() {
    // per process (the library targets one GPU model); threads that race to
    // fill it compute the same value
    static std::atomic<int64_t> cached{-1};
    int64_t v = cached.load(std::memory_order_relaxed);
    if (v < 0) {
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void*>(layout_main_kernel<2, KMAX>), kBlock, 0) ==
                hipSuccess)
            v = (int64_t)cus * per_cu;
        else
            v = 0;
        cached.store(v, std::memory_order_relaxed);
    }
    return v;
}

// The layout's kernels for k <= KMAX: one workgroup when T fits one tile,
// else the one-kernel form when every tile (and the expert workgroup) can be
// resident at once, else the counting pass and the second pass.
template <int KMAX>
void launch_layout(const ep_shape_t& s, const Workspace& w, const int32_t* topk_idx,
                   int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                   int32_t* rank_offset, int32_t* expert_offset, uint8_t* is_token_in_rank,
                   int32_t* send_slot, int32_t* dev_status, hipStream_t stream) {
    const int epr = s.E / s.R;
    const int nb = w.layout_blocks;
    int32_t* counters = w.msg_arrivals;
    if (nb == 1) {
        hipLaunchKernelGGL((layout_main_kernel<0, KMAX>), dim3(1), dim3(kBlock), 0, stream,
                           topk_idx, s.T, s.E, s.R, s.k, epr, 1, (int32_t*)nullptr,
                           (int32_t*)nullptr, num_tokens_per_rank, num_tokens_per_expert,
                           rank_offset, expert_offset, w.msg_base, is_token_in_rank, send_slot,
                           counters, w.counters_n, w.barrier, dev_status);
    } else if (nb + 1 <= max_resident_layout_tiles<KMAX>()) {
        hipLaunchKernelGGL((layout_main_kernel<2, KMAX>), dim3(nb + 1), dim3(kBlock), 0, stream,
                           topk_idx, s.T, s.E, s.R, s.k, epr, nb, w.blk_rank_cnt, w.blk_exp_cnt,
                           num_tokens_per_rank, num_tokens_per_expert, rank_offset, expert_offset,
                           w.msg_base, is_token_in_rank, send_slot, counters, w.counters_n,
                           w.barrier, dev_status);
    } else {
        hipLaunchKernelGGL((layout_count_kernel<KMAX>), dim3(nb), dim3(kBlock), 0, stream,
                           topk_idx, s.T, s.E, s.R, s.k, epr, w.blk_rank_cnt, w.blk_exp_cnt,
                           counters, w.counters_n, dev_status);
        hipLaunchKernelGGL((layout_main_kernel<1, KMAX>), dim3(nb + 1), dim3(kBlock), 0, stream,
                           topk_idx, s.T, s.E, s.R, s.k, epr, nb, w.blk_rank_cnt, w.blk_exp_cnt,
                           num_tokens_per_rank, num_tokens_per_expert, rank_offset, expert_offset,
                           w.msg_base, is_token_in_rank, send_slot, counters, w.counters_n,
                           w.barrier, dev_status);
    }
}

}  // namespace ep

using namespace ep;

extern "C" int ep_dispatch_layout(const ep_shape_t* shape, const int32_t* topk_idx,
                                  int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                                  int32_t* rank_offset, int32_t* expert_offset,
                                  uint8_t* is_token_in_rank, int32_t* send_slot, void* workspace,
                                  size_t ws_bytes, int32_t* dev_status, hipStream_t stream) {
    int v = validate_shape(shape);
    if (v != EP_OK) return v;
    const ep_shape_t s = *shape;
    if (!num_tokens_per_rank || !num_tokens_per_expert || !rank_offset || !expert_offset ||
        !dev_status || !workspace)
        return EP_ERR_INVALID_ARG;
    if (s.T > 0 && (!topk_idx || !is_token_in_rank || !send_slot)) return EP_ERR_INVALID_ARG;
    if (((uintptr_t)send_slot & 15) || ((uintptr_t)is_token_in_rank & 3)) return EP_ERR_INVALID_ARG;
    if (ws_bytes < workspace_bytes(s)) return EP_ERR_INVALID_ARG;
    Workspace w = carve_workspace(s, workspace);
    clear_hip_error();
    if (s.k <= 8)
        launch_layout<8>(s, w, topk_idx, num_tokens_per_rank, num_tokens_per_expert, rank_offset,
                         expert_offset, is_token_in_rank, send_slot, dev_status, stream);
    else
        launch_layout<kMaxK>(s, w, topk_idx, num_tokens_per_rank, num_tokens_per_expert,
                             rank_offset, expert_offset, is_token_in_rank, send_slot, dev_status,
                             stream);
    EP_HIP_CHECK(hipGetLastError());
    return EP_OK;
}

extern "C" int ep_dispatch_layout_ll(const ep_shape_t* shape, const int32_t* topk_idx,
                                     const int32_t* expert_offset, int32_t* expert_slot,
                                     void* workspace, size_t ws_bytes, int32_t* dev_status,
                                     hipStream_t stream) {
    int v = validate_shape(shape);
    if (v != EP_OK) return v;
    const ep_shape_t s = *shape;
    if (!expert_offset || !dev_status || !workspace) return EP_ERR_INVALID_ARG;
    if (s.T == 0) return EP_OK;
    if (!topk_idx || !expert_slot) return EP_ERR_INVALID_ARG;
    if (ws_bytes < workspace_bytes(s)) return EP_ERR_INVALID_ARG;
    Workspace w = carve_workspace(s, workspace);
    clear_hip_error();
    hipLaunchKernelGGL(ll_slot_kernel, dim3((unsigned)ceil_div(s.T, kWave)), dim3(kWave), 0, stream,
                       topk_idx, s.T, s.E, s.k, w.blk_exp_cnt, expert_offset, expert_slot,
                       dev_status);
    EP_HIP_CHECK(hipGetLastError());
    return EP_OK;
}

extern "C" int ep_dispatch_ll_layout(const ep_shape_t* shape, const int32_t* topk_idx,
                                     int32_t* num_tokens_per_expert, int32_t* expert_offset,
                                     int32_t* expert_slot, void* workspace, size_t ws_bytes,
                                     int32_t* dev_status, hipStream_t stream) {
    int v = validate_shape(shape);
    if (v != EP_OK) return v;
    const ep_shape_t s = *shape;
    if (!num_tokens_per_expert || !expert_offset || !dev_status || !workspace)
        return EP_ERR_INVALID_ARG;
    if (s.T > 0 && (!topk_idx || !expert_slot)) return EP_ERR_INVALID_ARG;
    if (ws_bytes < workspace_bytes(s)) return EP_ERR_INVALID_ARG;
    if (s.E > kLLLayoutMaxE) {
        record_error("ep_dispatch_ll_layout: E > 1024 (use ep_dispatch_layout + ep_dispatch_layout_ll)");
        return EP_ERR_INVALID_ARG;
    }
    Workspace w = carve_workspace(s, workspace);
    const int nb = w.layout_blocks;
    const bool small_k = s.k <= 8;
    const int64_t room = small_k ? max_resident_ll_tiles<8>() : max_resident_ll_tiles<kMaxK>();
    if (nb > room) {
        record_error("ep_dispatch_ll_layout: more tiles than the device holds at once (use "
                     "ep_dispatch_layout + ep_dispatch_layout_ll)");
        return EP_ERR_INVALID_ARG;
    }
    clear_hip_error();
    if (small_k)
        hipLaunchKernelGGL(ll_layout_kernel<8>, dim3(nb), dim3(kBlock), 0, stream, topk_idx, s.T,
                           s.E, s.k, nb, w.blk_exp_cnt, num_tokens_per_expert, expert_offset,
                           expert_slot, w.msg_arrivals, w.counters_n, w.barrier, dev_status);
    else
        hipLaunchKernelGGL(ll_layout_kernel<kMaxK>, dim3(nb), dim3(kBlock), 0, stream, topk_idx,
                           s.T, s.E, s.k, nb, w.blk_exp_cnt, num_tokens_per_expert, expert_offset,
                           expert_slot, w.msg_arrivals, w.counters_n, w.barrier, dev_status);
    EP_HIP_CHECK(hipGetLastError());
    return EP_OK;
}
